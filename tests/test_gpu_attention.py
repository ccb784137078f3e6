"""GPU parity of ts_verify_attn / ts_draft_attn against the float64 oracle.

Bar: max|O_gpu - O_ref| / max|O_ref| <= 2e-3 per call (bf16 inputs, fp32
accumulation). Covers the small workload in full, ragged context lengths
around the 64-row tiles, empty context, random and wide trees of up to 128
nodes (two ancestor words past 64), MHA/GQA groupings, both head sizes,
forced split counts, NaN-poisoned rows past the tree, and sampled KV heads of
the full-size workloads (up to the 128-node tree at 100K rows).
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import bf16_to_f64, draft_attention, verify_attention
from synth import CONFIGS, attention_inputs, tree_parent
from tests.gpu_util import banner, dev_bf16, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run_verify(x, n_ctx, parent, n_split=0, scale=0.0):
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out = ts.verify_attn(q, k, v, n_ctx, parent, scale=scale, n_split=n_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(x, n_ctx, parent, heads=None, scale=None):
    if heads is None:
        q, k, v = bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"])
        return verify_attention(q, k, v, n_ctx, parent, scale)
    Hq, Hkv = x["q"].shape[0], x["k"].shape[0]
    G = Hq // Hkv
    rows = n_ctx + len(parent)
    outs = {}
    for g in heads:  # one KV head's group at a time
        outs[g] = verify_attention(bf16_to_f64(x["q"][g * G:(g + 1) * G]), bf16_to_f64(x["k"][g:g + 1, :rows]),
                                   bf16_to_f64(x["v"][g:g + 1, :rows]), n_ctx, parent, scale)
    return outs


@pytest.mark.parametrize("n_split", [0, 1, 7, 10_000])
def test_tiny_workload(n_split):
    c = CONFIGS["tiny"]
    banner(f"tiny verify n_split={n_split}")
    x = attention_inputs(c["seed"], c["Hq"], c["Hkv"], c["d"], c["n_ctx"], c["T"], cap=c["n_ctx"] + 100, poison_tail=True)
    parent = tree_parent("tiny8")
    got = _run_verify(x, c["n_ctx"], parent, n_split)
    ref = _oracle(x, c["n_ctx"], parent)
    assert rel_max_err(got, ref) <= TOL


SHAPES = [
    # Hq, Hkv, d, n_ctx, tree
    (4, 1, 128, 0, "chain4"), (4, 1, 64, 1, "tiny8"), (8, 2, 128, 63, "tiny8"), (8, 2, 128, 64, "tiny8"),
    (8, 2, 128, 65, "ts24"), (32, 8, 128, 1000, "chain4"), (12, 2, 128, 777, "ts24"), (32, 32, 128, 300, "ts24"),
    (40, 8, 128, 1500, "ts64"), (32, 8, 128, 2049, "ts64"), (8, 8, 64, 129, "rand17"), (6, 2, 64, 5000, "rand64"),
    (64, 2, 128, 333, "rand40"), (16, 1, 128, 96, "rand9"), (24, 4, 64, 4097, "ts24"),
    # the headline grouping with several tiles per split and a ragged last tile
    (32, 8, 128, 700, "ts24"),
    # trees past 64 nodes (two ancestor words per node)
    (8, 2, 128, 1000, "wide88"), (32, 8, 128, 3001, "wide88"), (8, 2, 64, 77, "rand128"), (4, 1, 128, 200, "chain128"),
    (40, 8, 128, 500, "rand100"), (8, 2, 128, 64, "rand65"),
    # row blocks of unequal live row tiles: 25 tiles as 13 + 12, 17 as 9 + 8
    (8, 2, 128, 777, "rand100"), (8, 2, 64, 1234, "rand68"),
]


def _tree(name, seed):
    if name == "chain4":
        return tree_parent("chain", 4)
    if name.startswith("chain"):
        return tree_parent("chain", int(name[5:]))
    if name.startswith("wide"):
        return tree_parent("wide", int(name[4:]))
    if name == "tiny8":
        return tree_parent("tiny8")
    if name.startswith("ts"):
        return tree_parent("tokenswift", int(name[2:]))
    rng = np.random.default_rng(seed)
    T = int(name[4:])
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}q{s[1]}kv_d{s[2]}_L{s[3]}_{s[4]}" for s in SHAPES])
def test_shapes_and_trees(shape):
    Hq, Hkv, d, n_ctx, tname = shape
    parent = _tree(tname, n_ctx)
    T = len(parent)
    banner(f"verify Hq={Hq} Hkv={Hkv} d={d} n_ctx={n_ctx} T={T}")
    x = attention_inputs(1000 + n_ctx, Hq, Hkv, d, n_ctx, T, cap=n_ctx + T + 64, poison_tail=True)
    for n_split in (0, 1, 3):   # automatic, one split (every tile in one workgroup), three
        got = _run_verify(x, n_ctx, parent, n_split)
        ref = _oracle(x, n_ctx, parent)
        assert np.isfinite(got).all()
        assert rel_max_err(got, ref) <= TOL, (n_split, rel_max_err(got, ref))


def test_explicit_scale():
    x = attention_inputs(5, 8, 2, 128, 500, 8)
    parent = tree_parent("tiny8")
    got = _run_verify(x, 500, parent, scale=0.05)
    assert rel_max_err(got, _oracle(x, 500, parent, scale=0.05)) <= TOL


def test_repeatable_bitwise():
    x = attention_inputs(6, 32, 8, 128, 20_000, 24)
    parent = tree_parent("tokenswift", 24)
    a = _run_verify(x, 20_000, parent)
    b = _run_verify(x, 20_000, parent)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Tq,n_part,Hq,Hkv", [(1, 4164, 32, 8), (4, 4164, 32, 8), (4, 8260, 40, 8), (4, 4164, 12, 2),
                                              (3, 10, 8, 2), (5, 0, 8, 8), (64, 8260, 40, 8), (128, 4164, 32, 8)])
def test_draft_attention(Tq, n_part, Hq, Hkv):
    banner(f"draft Tq={Tq} n_part={n_part} Hq={Hq} Hkv={Hkv}")
    x = attention_inputs(77 + n_part, Hq, Hkv, 128, n_part, Tq, cap=n_part + Tq + 32, poison_tail=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    got = ts.draft_attn(q, k, v, n_part)
    torch.cuda.synchronize()
    ref = draft_attention(bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"]), n_part)
    assert rel_max_err(got.cpu().numpy(), ref) <= TOL


def test_verify_rejects_bad_tree_on_device_path():
    x = attention_inputs(8, 8, 2, 128, 100, 3)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    with pytest.raises(ts.TSError) as e:
        ts.verify_attn(q, k, v, 100, [-1, 2, 0])
    assert e.value.code == -1


def _bf16_bits(value):
    """bfloat16 bit pattern of a value that bfloat16 holds exactly."""
    b = np.array([value], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, value
    return np.uint16(b >> 16)


@pytest.mark.parametrize("n_split", [1, 0, 7])
def test_v_at_the_float16_limit(n_split):
    """V entries of +-65280, the largest bfloat16 magnitude inside the float16
    range, go through the float16 P.V product unclamped (verification and
    draft entry points)."""
    banner(f"verify/draft V = +-65280 n_split={n_split}")
    Hq, Hkv, d, n_ctx = 8, 2, 128, 3000
    parent = tree_parent("tokenswift", 24)
    x = attention_inputs(41, Hq, Hkv, d, n_ctx, len(parent))
    rng = np.random.default_rng(41)
    for _ in range(64):   # committed and tree rows, both signs
        g, j, c = int(rng.integers(0, Hkv)), int(rng.integers(0, n_ctx + len(parent))), int(rng.integers(0, d))
        x["v"][g, j, c] = _bf16_bits(65280.0 if rng.integers(0, 2) else -65280.0)
    got = _run_verify(x, n_ctx, parent, n_split)
    assert np.isfinite(got).all()
    assert rel_max_err(got, _oracle(x, n_ctx, parent)) <= TOL
    q, k, v = dev_bf16(x["q"][:, :4]), dev_bf16(x["k"]), dev_bf16(x["v"])
    gd = ts.draft_attn(q, k, v, n_ctx, n_split=n_split)
    torch.cuda.synchronize()
    refd = draft_attention(bf16_to_f64(x["q"][:, :4]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"]), n_ctx)
    assert rel_max_err(gd.cpu().numpy(), refd) <= TOL


@pytest.mark.parametrize("n_split", [1, 0, 7])
def test_v_beyond_float16_range_is_not_clamped(n_split):
    """A V entry past the float16 range (2^20 in a committed row: every query
    sees it) makes that channel of every output row of its KV head's group
    non-finite instead of a silently clamped value; every other channel and
    group still matches the oracle."""
    banner(f"verify V = 2^20 n_split={n_split}")
    Hq, Hkv, d, n_ctx = 8, 2, 128, 3000
    G = Hq // Hkv
    parent = tree_parent("tokenswift", 24)
    x = attention_inputs(43, Hq, Hkv, d, n_ctx, len(parent))
    g, j, c = 1, 1234, 5
    x["v"][g, j, c] = _bf16_bits(2.0 ** 20)
    got = _run_verify(x, n_ctx, parent, n_split)
    assert not np.isfinite(got[g * G:(g + 1) * G, :, c]).any()
    ok = np.ones(got.shape, dtype=bool)
    ok[g * G:(g + 1) * G, :, c] = False
    assert np.isfinite(got[ok]).all()
    ref = _oracle(x, n_ctx, parent)
    assert rel_max_err(got[ok], ref[ok]) <= TOL


FULL = [("8b", 24, "tokenswift", [0, 5]), ("8b", 64, "tokenswift", [3]), ("8b", 4, "chain", [7]),
        ("1.5b", 24, "tokenswift", [1]), ("7b", 24, "tokenswift", [0, 31]), ("14b", 64, "tokenswift", [2]),
        ("8b", 88, "wide", [6]), ("8b", 128, "wide", [1])]


@pytest.mark.parametrize("name,T,tree,heads", FULL, ids=[f"{f[0]}_T{f[1]}" for f in FULL])
def test_full_size_sampled_heads(name, T, tree, heads):
    """Full 100K-context workloads in the benchmark's launch configuration; the
    oracle checks sampled KV heads (each head's group is independent)."""
    c = CONFIGS[name]
    banner(f"full {name} T={T} heads={heads}")
    parent = tree_parent(tree, T)
    x = attention_inputs(c["seed"], c["Hq"], c["Hkv"], c["d"], c["n_ctx"], T, k_scale=c.get("k_scale"))
    got = _run_verify(x, c["n_ctx"], parent)
    G = c["Hq"] // c["Hkv"]
    refs = _oracle(x, c["n_ctx"], parent, heads=heads)
    for g, ref in refs.items():
        err = rel_max_err(got[g * G:(g + 1) * G], ref)
        assert err <= TOL, (g, err)
