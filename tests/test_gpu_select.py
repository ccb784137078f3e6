"""GPU parity of ts_partial_kv_select against the float64 oracle.

Scores: |s_gpu - s_ref| <= 1e-5 * max|s_ref| (fp32 accumulation of bf16
products). Selected index set: bit-exact outside the cut band
|sigma_j - sigma_cut| <= 1e-4 * max(|sigma_cut|, 1); same size, ascending,
-1 padded. Partial cache: sink U selected U recent rows copied bit-exactly.
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import bf16_to_f64, draft_attention, partial_kv_select, verify_attention
from synth import CONFIGS, attention_inputs, bf16_round, tree_parent
from tests.gpu_util import banner, dev_bf16, rel_max_err

pytestmark = pytest.mark.gpu


def _check(x, n_ctx, Hq, Hkv, n_sink, budget, n_recent, heads=None, strict=False, ws=None):
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    sel, kp, vp, n_part, sc = ts.partial_kv_select(q, k, v, n_ctx, n_sink, budget, n_recent, want_scores=True, ws=ws)
    torch.cuda.synchronize()
    sel, sc = sel.cpu().numpy(), sc.cpu().numpy()[:, :n_ctx]
    kp = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    vp = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    G = Hq // Hkv
    heads = range(Hkv) if heads is None else heads
    for g in heads:
        ref = partial_kv_select(bf16_to_f64(x["q"][g * G:(g + 1) * G]), bf16_to_f64(x["k"][g:g + 1, :n_ctx]),
                                n_ctx, 1, n_sink, budget, n_recent)
        assert n_part == ref.n_part
        s_ref = ref.scores[0]
        if n_ctx:
            assert np.max(np.abs(sc[g] - s_ref)) <= 1e-5 * max(np.max(np.abs(s_ref)), 1e-30)
        got = sel[g]
        b_eff = int((ref.sel_idx[0] >= 0).sum())
        assert np.all(got[b_eff:] == -1)
        gs = got[:b_eff]
        assert np.all(np.diff(gs) > 0)
        rs = ref.sel_idx[0][:b_eff]
        diff = np.setxor1d(gs, rs)
        if strict:   # exactly equal scores: the row order decides, with no rounding band
            assert len(diff) == 0, (g, diff[:10])
        if len(diff):
            cut = ref.cutoff[0]
            band = 1e-4 * max(abs(cut), 1.0)
            assert np.all(np.abs(s_ref[diff] - cut) <= band), (g, diff, s_ref[diff], cut)
        # partial cache rows: sink, the GPU's own selection, recent
        rows = np.concatenate([np.arange(min(n_sink, n_ctx)), gs, np.arange(max(n_sink, n_ctx - n_recent), n_ctx)])
        assert len(rows) == n_part
        np.testing.assert_array_equal(kp[g, :n_part], x["k"][g, rows])
        np.testing.assert_array_equal(vp[g, :n_part], x["v"][g, rows])
    return sel, n_part


def test_tiny_workload():
    c = CONFIGS["tiny"]
    banner("select tiny")
    x = attention_inputs(c["seed"], c["Hq"], c["Hkv"], c["d"], c["n_ctx"], c["T"])
    _check(x, c["n_ctx"], c["Hq"], c["Hkv"], c["n_sink"], c["budget"], c["n_recent"])
    _check(x, c["n_ctx"], c["Hq"], c["Hkv"], 0, c["budget"], 0)


@pytest.mark.parametrize("n_ctx,n_sink,budget,n_recent", [
    (1000, 4, 100, 8), (1000, 0, 1000, 0), (1000, 4, 988, 8), (1000, 4, 5000, 8), (1000, 4, 0, 8), (70, 4, 16, 64),
    (68, 4, 16, 64), (3, 4, 16, 8), (0, 4, 16, 8), (5000, 4, 1, 64), (33_333, 4, 4096, 64),
])
def test_edge_cases(n_ctx, n_sink, budget, n_recent):
    banner(f"select n_ctx={n_ctx} sink={n_sink} B={budget} recent={n_recent}")
    x = attention_inputs(n_ctx + 3, 8, 2, 128, max(n_ctx, 1), 4)
    _check(x, n_ctx, 8, 2, n_sink, budget, n_recent)


def test_exact_ties_go_to_earlier_rows():
    n_ctx = 3000
    x = attention_inputs(12, 8, 2, 128, n_ctx, 4)
    x["k"][:, 1500:1600] = x["k"][:, 100:200]    # 100 exact score ties per head
    _check(x, n_ctx, 8, 2, 4, 150, 64)


@pytest.mark.parametrize("kind", ["top", "zero"])
def test_massive_ties_span_blocks(kind):
    """Tens of thousands of exactly equal scores at the cut: more cut-bin keys
    than the in-LDS refinement holds, ties spread over many blocks, and the
    earliest tied rows must be the ones taken."""
    n_ctx, Hq, Hkv = 60_000, 8, 2
    banner(f"select massive ties {kind}")
    x = attention_inputs(21, Hq, Hkv, 128, n_ctx, 4)
    G = Hq // Hkv
    if kind == "top":
        # rows 1000..44999 share one key whose score tops every random row
        for g in range(Hkv):
            qbar = bf16_to_f64(x["q"][g * G:(g + 1) * G]).sum(axis=(0, 1))
            u = np.where(qbar >= 0, 3.0, -3.0).astype(np.float32)
            x["k"][g, 1000:45000] = bf16_round(u)[None, :]
        _check(x, n_ctx, Hq, Hkv, 4, 30_000, 64, strict=True)
    else:
        x["k"][:] = 0   # every score is exactly 0
        _check(x, n_ctx, Hq, Hkv, 4, 5_000, 64, strict=True)


def test_crowded_cut_bin_with_long_lists():
    """About 5900 keys in the cut's first-digit bin (under the 8192 refined in
    LDS) spread over all 30 blocks of a head: every block's list of cut-bin
    keys runs past 64 entries (47 to 205), and the keys take only ~16 distinct
    values, so the row order decides exactly."""
    n_ctx, Hq, Hkv = 30_000, 8, 2
    banner("select crowded cut bin")
    x = attention_inputs(22, Hq, Hkv, 128, n_ctx, 4)
    G = Hq // Hkv
    rng = np.random.default_rng(22)
    for g in range(Hkv):
        qbar = bf16_to_f64(x["q"][g * G:(g + 1) * G]).sum(axis=(0, 1))
        u = np.where(qbar >= 0, 3.0, -3.0)
        rows = np.arange(7, n_ctx, 5)    # every fifth row: 6000 rows over all blocks
        k = u[None, :] * (1.0 + 0.01 * rng.standard_normal((rows.size, 1)))
        x["k"][g, rows] = bf16_round(k.astype(np.float32))
    _check(x, n_ctx, Hq, Hkv, 4, 3000, 64, strict=True)


def test_long_chunks_span_several_sub_chunks():
    """600K rows over 8 KV heads (64 blocks per head): each block's chunk
    (about 9400 rows) spans three 4096-row sub-chunks in the cut-bin and emit
    passes (later keys reloaded, output runs carried across sub-chunks);
    sampled heads."""
    n_ctx, Hq, Hkv = 600_000, 32, 8
    banner("select 600K rows")
    x = attention_inputs(31, Hq, Hkv, 128, n_ctx, 24)
    _check(x, n_ctx, Hq, Hkv, 4, 4096, 64, heads=[0, 7])


@pytest.mark.parametrize("T,Hq,Hkv", [(128, 8, 2), (100, 40, 8)])
def test_many_query_rows_per_head(T, Hq, Hkv):
    """More than 256 query rows per KV head (512 and 500): the score pass sums
    the group's queries in two rounds of 256 rows."""
    n_ctx = 5000
    banner(f"select T={T} Hq={Hq} Hkv={Hkv}")
    x = attention_inputs(40 + T, Hq, Hkv, 128, n_ctx, T)
    _check(x, n_ctx, Hq, Hkv, 4, 700, 64)


@pytest.mark.parametrize("fill", [0xFF, 0x01])
def test_workspace_not_at_zero(fill):
    """The calls leave the first-digit histogram at zero for the next call;
    a workspace that does not hold a zero histogram (first use, or filled
    with other data) is recounted from the scores: exact either way, on two
    calls in a row (the second with a smaller budget) and through the
    scored entry point."""
    n_ctx, Hq, Hkv = 20_000, 32, 8
    banner(f"select on a workspace filled with {fill:#x}")
    x = attention_inputs(81, Hq, Hkv, 128, n_ctx, 24)
    need = ts.lib().ts_partial_kv_select_workspace_size(n_ctx, 24, Hq, Hkv, 128, 2000)
    ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda:0")
    _check(x, n_ctx, Hq, Hkv, 4, 2000, 64, ws=ws)
    _check(x, n_ctx, Hq, Hkv, 4, 700, 64, ws=ws)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    _, _, _, _, sc = ts.partial_kv_select(q, k, v, n_ctx, 4, 2000, 64, want_scores=True)
    wss = torch.full((ts.lib().ts_partial_kv_select_scored_workspace_size(n_ctx, Hkv, 128, 2000),), fill,
                     dtype=torch.uint8, device="cuda:0")
    sel1 = ts.partial_kv_select_scored(sc, k, v, n_ctx, 4, 2000, 64, ws=wss)[0]
    sel2 = ts.partial_kv_select_scored(sc, k, v, n_ctx, 4, 2000, 64, ws=wss)[0]
    ref = ts.partial_kv_select(q, k, v, n_ctx, 4, 2000, 64)[0]
    torch.cuda.synchronize()
    assert torch.equal(sel1, ref) and torch.equal(sel2, ref)


def test_full_budget_draft_equals_verification():
    Hq, Hkv, d, n_ctx, Tq = 8, 2, 128, 1234, 4
    x = attention_inputs(13, Hq, Hkv, d, n_ctx, Tq)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    sel, kp, vp, n_part, _ = ts.partial_kv_select(q, k, v, n_ctx, 4, 100_000, 64, extra_rows=Tq)
    assert n_part == n_ctx
    kp[:, n_part:n_part + Tq] = k[:, n_ctx:n_ctx + Tq]
    vp[:, n_part:n_part + Tq] = v[:, n_ctx:n_ctx + Tq]
    draft = ts.draft_attn(q, kp, vp, n_part)
    full = ts.verify_attn(q, k, v, n_ctx, tree_parent("chain", Tq))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(draft.cpu().numpy(), full.cpu().numpy())
    ref = verify_attention(bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"]), n_ctx, tree_parent("chain", Tq))
    assert rel_max_err(draft.cpu().numpy(), ref) <= 2e-3


@pytest.mark.parametrize("Hq,Hkv,n_ctx,budget,T", [
    (32, 32, 66_666, 4096, 24),   # the 7B layout: 16 blocks per head, chunks of two sub-chunks
    (4, 4, 5000, 700, 24),
    (4, 4, 1000, 100, 1),
    (3, 3, 300, 500, 4),          # budget past the candidates
])
def test_one_query_head_per_kv_head(Hq, Hkv, n_ctx, budget, T):
    """MHA (TokenSwift summary §4.2 measures MHA and GQA models): each KV
    head's group is a single query head, so the grouped score of §3.3 is that
    head's own products summed over the tree nodes."""
    banner(f"select MHA Hq=Hkv={Hkv} n_ctx={n_ctx} B={budget} T={T}")
    x = attention_inputs(50 + Hkv + T, Hq, Hkv, 128, n_ctx, T)
    _check(x, n_ctx, Hq, Hkv, 4, budget, 64)


@pytest.mark.parametrize("name,heads", [("8b", [0, 6]), ("14b", [4]), ("1.5b", [1]), ("7b", [0, 31])])
def test_full_size_sampled_heads(name, heads):
    c = CONFIGS[name]
    banner(f"select full {name}")
    x = attention_inputs(c["seed"], c["Hq"], c["Hkv"], c["d"], c["n_ctx"], c["T"], k_scale=c.get("k_scale"))
    _check(x, c["n_ctx"], c["Hq"], c["Hkv"], c["n_sink"], c["budget"], c["n_recent"], heads=heads)
