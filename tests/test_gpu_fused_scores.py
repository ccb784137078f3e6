"""GPU parity of the fused score path: ts_verify_attn_scored and
ts_partial_kv_select_scored against the float64 oracle.

Attention output: bitwise equal to ts_verify_attn on the same call (the score
sums only read the S tiles). Scores: |s_gpu - s_ref| <= 1e-5 * max|s_ref|
(bf16 products, float32 sums). Selection from those scores: bit-exact outside
the cut band |sigma_j - sigma_cut| <= 1e-4 * max(|sigma_cut|, 1), as for
ts_partial_kv_select; partial cache rows copied bit-exactly. With the scores
of ts_partial_kv_select given, the scored selection equals it bitwise.
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from long_kv_attention_amd.binding import TSError
from oracle import bf16_to_f64, partial_kv_select, verify_attention
from synth import CONFIGS, attention_inputs, tree_parent
from tests.gpu_util import banner, dev_bf16, rel_max_err

pytestmark = pytest.mark.gpu


def _oracle_scores(x, n_ctx, Hq, Hkv, g, n_sink=0, budget=0, n_recent=0):
    G = Hq // Hkv
    return partial_kv_select(bf16_to_f64(x["q"][g * G:(g + 1) * G]), bf16_to_f64(x["k"][g:g + 1, :n_ctx]), n_ctx, 1,
                             n_sink, budget, n_recent)


def _check_scores(sc, ref_scores):
    if ref_scores.size:
        err = np.max(np.abs(sc.astype(np.float64) - ref_scores))
        assert err <= 1e-5 * max(np.max(np.abs(ref_scores)), 1e-30), err


def _check_selection(x, g, sel, kp, vp, n_part, ref, n_ctx, n_sink, n_recent):
    assert n_part == ref.n_part
    b_eff = int((ref.sel_idx[0] >= 0).sum())
    got = sel[g]
    assert np.all(got[b_eff:] == -1)
    gs = got[:b_eff]
    assert np.all(np.diff(gs) > 0)
    diff = np.setxor1d(gs, ref.sel_idx[0][:b_eff])
    if len(diff):
        cut = ref.cutoff[0]
        assert np.all(np.abs(ref.scores[0][diff] - cut) <= 1e-4 * max(abs(cut), 1.0)), (g, diff, cut)
    rows = np.concatenate([np.arange(min(n_sink, n_ctx)), gs, np.arange(max(n_sink, n_ctx - n_recent), n_ctx)])
    assert len(rows) == n_part
    np.testing.assert_array_equal(kp[g, :n_part], x["k"][g, rows])
    np.testing.assert_array_equal(vp[g, :n_part], x["v"][g, rows])


def _host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# T values reach every workgroup shape the kernel picks for 4 query heads per
# KV head (1 to 16 row tiles); n_ctx leaves a ragged last tile.
@pytest.mark.parametrize("T", [1, 4, 8, 12, 16, 24, 32, 36, 48, 64])
@pytest.mark.parametrize("n_split", [0, 1])
def test_scores_and_unchanged_output(T, n_split):
    Hq, Hkv, d, n_ctx = 8, 2, 128, 3001
    banner(f"fused scores T={T} n_split={n_split}")
    x = attention_inputs(40 + T, Hq, Hkv, d, n_ctx, T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    parent = tree_parent("chain", T) if T < 10 else tree_parent("tokenswift", T)
    out, sc = ts.verify_attn_scored(q, k, v, n_ctx, parent, n_split=n_split)
    plain = ts.verify_attn(q, k, v, n_ctx, parent, n_split=n_split)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), plain.cpu().numpy())
    sc = sc.cpu().numpy()
    for g in range(Hkv):
        _check_scores(sc[g, :n_ctx], _oracle_scores(x, n_ctx, Hq, Hkv, g).scores[0])


@pytest.mark.parametrize("d,n_ctx,T", [(64, 2048, 8), (64, 129, 3), (128, 1, 1), (128, 127, 24), (128, 128, 24),
                                       (128, 0, 4)])
def test_small_and_empty_contexts(d, n_ctx, T):
    Hq, Hkv = 8, 2
    banner(f"fused scores d={d} n_ctx={n_ctx} T={T}")
    x = attention_inputs(7 + n_ctx, Hq, Hkv, d, max(n_ctx, 1), T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    parent = tree_parent("chain", T)
    out, sc = ts.verify_attn_scored(q, k, v, n_ctx, parent)
    plain = ts.verify_attn(q, k, v, n_ctx, parent)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), plain.cpu().numpy())
    sc = sc.cpu().numpy()
    for g in range(Hkv):
        _check_scores(sc[g, :n_ctx], _oracle_scores(x, n_ctx, Hq, Hkv, g).scores[0])


@pytest.mark.parametrize("n_ctx,n_sink,budget,n_recent", [
    (3000, 4, 300, 64), (3000, 0, 3000, 0), (3000, 4, 0, 8), (70, 4, 16, 64), (3, 4, 16, 8), (0, 4, 16, 8),
    (20_000, 4, 4096, 64),
])
def test_selection_from_fused_scores(n_ctx, n_sink, budget, n_recent):
    Hq, Hkv, d, T = 8, 2, 128, 24
    banner(f"scored select n_ctx={n_ctx} sink={n_sink} B={budget} recent={n_recent}")
    x = attention_inputs(n_ctx + 11, Hq, Hkv, d, max(n_ctx, 1), T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    _, sc = ts.verify_attn_scored(q, k, v, n_ctx, tree_parent("tokenswift", T))
    sel, kp, vp, n_part = ts.partial_kv_select_scored(sc, k, v, n_ctx, n_sink, budget, n_recent)
    torch.cuda.synchronize()
    sel, kp, vp = sel.cpu().numpy(), _host_u16(kp), _host_u16(vp)
    for g in range(Hkv):
        ref = _oracle_scores(x, n_ctx, Hq, Hkv, g, n_sink, budget, n_recent)
        _check_selection(x, g, sel, kp, vp, n_part, ref, n_ctx, n_sink, n_recent)


@pytest.mark.parametrize("zero_keys", [False, True])
def test_given_scores_select_like_the_query_pass(zero_keys):
    """The same scores give the same selection bitwise, whichever pass made
    them (with all-zero keys every score ties and row order decides)."""
    Hq, Hkv, d, T, n_ctx = 8, 2, 128, 4, 60_000
    banner(f"scored select equals query pass zero_keys={zero_keys}")
    x = attention_inputs(5, Hq, Hkv, d, n_ctx, T)
    if zero_keys:
        x["k"][:] = 0
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    sel, kp, vp, n_part, sc = ts.partial_kv_select(q, k, v, n_ctx, 4, 5000, 64, want_scores=True)
    sel2, kp2, vp2, n_part2 = ts.partial_kv_select_scored(sc, k, v, n_ctx, 4, 5000, 64)
    torch.cuda.synchronize()
    assert n_part == n_part2
    np.testing.assert_array_equal(sel.cpu().numpy(), sel2.cpu().numpy())
    np.testing.assert_array_equal(_host_u16(kp)[:, :n_part], _host_u16(kp2)[:, :n_part])
    np.testing.assert_array_equal(_host_u16(vp)[:, :n_part], _host_u16(vp2)[:, :n_part])


@pytest.mark.parametrize("name,heads", [("8b", [0, 5]), ("1.5b", [1])])
def test_full_size_sampled_heads(name, heads):
    c = CONFIGS[name]
    banner(f"fused scores full {name}")
    x = attention_inputs(c["seed"], c["Hq"], c["Hkv"], c["d"], c["n_ctx"], c["T"], k_scale=c.get("k_scale"))
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    n_ctx = c["n_ctx"]
    parent = tree_parent(c["tree"], c["T"])
    # automatic and forced split counts: the output is bitwise the plain call's;
    # scores, selection and output against the oracle
    out, sc = ts.verify_attn_scored(q, k, v, n_ctx, parent)
    plain = ts.verify_attn(q, k, v, n_ctx, parent)
    sel, kp, vp, n_part = ts.partial_kv_select_scored(sc, k, v, n_ctx, c["n_sink"], c["budget"], c["n_recent"])
    out_f, sc_f = ts.verify_attn_scored(q, k, v, n_ctx, parent, n_split=7)
    plain_f = ts.verify_attn(q, k, v, n_ctx, parent, n_split=7)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    assert torch.equal(out_f, plain_f)
    assert torch.equal(sc, sc_f)   # each score is one workgroup's sum, whatever the split count
    sc, sel, kp, vp = sc.cpu().numpy(), sel.cpu().numpy(), _host_u16(kp), _host_u16(vp)
    G = c["Hq"] // c["Hkv"]
    out = out.cpu().numpy()
    for g in heads:
        ref = _oracle_scores(x, n_ctx, c["Hq"], c["Hkv"], g, c["n_sink"], c["budget"], c["n_recent"])
        _check_scores(sc[g], ref.scores[0])
        _check_selection(x, g, sel, kp, vp, n_part, ref, n_ctx, c["n_sink"], c["n_recent"])
        oref = verify_attention(bf16_to_f64(x["q"][g * G:(g + 1) * G]), bf16_to_f64(x["k"][g:g + 1]),
                                bf16_to_f64(x["v"][g:g + 1]), n_ctx, parent)
        assert rel_max_err(out[g * G:(g + 1) * G], oref) <= 2e-3


@pytest.mark.parametrize("Hkv,T,n_ctx", [(4, 1, 3001), (4, 24, 3001), (4, 64, 3001), (4, 128, 3001),
                                         (32, 24, 20_000)])
def test_one_query_head_per_kv_head(Hkv, T, n_ctx):
    """MHA (TokenSwift summary §4.2): one query head per KV head, so every
    workgroup's rows are the T tree nodes of one head; the scores and the
    selection from them against the oracle, the output against the plain call."""
    Hq, d, budget = Hkv, 128, min(4096, n_ctx // 2)
    banner(f"fused scores MHA Hkv={Hkv} T={T} n_ctx={n_ctx}")
    x = attention_inputs(60 + T + Hkv, Hq, Hkv, d, n_ctx, T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    parent = tree_parent("chain", T) if T < 10 else tree_parent("tokenswift", T)
    out, sc = ts.verify_attn_scored(q, k, v, n_ctx, parent)
    plain = ts.verify_attn(q, k, v, n_ctx, parent)
    out_f, _ = ts.verify_attn_scored(q, k, v, n_ctx, parent, n_split=3)
    plain_f = ts.verify_attn(q, k, v, n_ctx, parent, n_split=3)
    sel, kp, vp, n_part = ts.partial_kv_select_scored(sc, k, v, n_ctx, 4, budget, 64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), plain.cpu().numpy())
    np.testing.assert_array_equal(out_f.cpu().numpy(), plain_f.cpu().numpy())
    out = out.cpu().numpy()
    sc, sel, kp, vp = sc.cpu().numpy(), sel.cpu().numpy(), _host_u16(kp), _host_u16(vp)
    for g in sorted({0, Hkv // 2, Hkv - 1}):
        ref = _oracle_scores(x, n_ctx, Hq, Hkv, g, 4, budget, 64)
        _check_scores(sc[g, :n_ctx], ref.scores[0])
        _check_selection(x, g, sel, kp, vp, n_part, ref, n_ctx, 4, 64)
        oref = verify_attention(bf16_to_f64(x["q"][g:g + 1]), bf16_to_f64(x["k"][g:g + 1]), bf16_to_f64(x["v"][g:g + 1]),
                                n_ctx, parent)
        assert rel_max_err(out[g:g + 1], oref) <= 2e-3


def test_too_many_rows_per_head_is_refused():
    # 5 query heads per KV head x 64 nodes = 320 rows: more than one workgroup sums
    Hq, Hkv, d, T, n_ctx = 10, 2, 128, 64, 500
    x = attention_inputs(3, Hq, Hkv, d, n_ctx, T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    with pytest.raises(TSError, match="TS_ENOTSUP"):
        ts.verify_attn_scored(q, k, v, n_ctx, tree_parent("chain", T))
