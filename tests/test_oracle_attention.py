"""Pins for the verification / draft attention oracle.

Each test checks the oracle against something other than itself: torch's
scaled_dot_product_attention in float64 (a library special case), closed
forms, and invariants that a wrong mask direction, head mapping, scale or
softmax axis would break.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ancestor_sets, bf16_to_f64, draft_attention, verify_attention
from synth import attention_inputs, bf16_round, tree_parent


def _random_parent(rng, T):
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


def _reach_mask(parent, n_ctx):
    """Visibility by transitive closure of the child->parent adjacency.

    Independent of the oracle's parent walk: boolean matrix powers of the
    adjacency (plus identity) until it stops growing.
    """
    T = len(parent)
    A = torch.zeros(T, T, dtype=torch.bool)
    for i in range(1, T):
        A[i, parent[i]] = True
    R = A | torch.eye(T, dtype=torch.bool)
    while True:
        R2 = R | ((R.to(torch.int64) @ R.to(torch.int64)) > 0)
        if torch.equal(R2, R):
            break
        R = R2
    mask = torch.ones(T, n_ctx + T, dtype=torch.bool)
    mask[:, n_ctx:] = R  # row i: which tree rows node i may see
    return mask


def _sdpa(q, k, v, n_ctx, mask, scale=None, gqa=True):
    qt = torch.from_numpy(q)[None]                  # [1][Hq][T][d]
    kt = torch.from_numpy(np.ascontiguousarray(k[:, : n_ctx + q.shape[1]]))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v[:, : n_ctx + q.shape[1]]))[None]
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=gqa)
    return out[0].numpy()


@pytest.mark.parametrize("seed", range(6))
def test_random_tree_matches_torch_sdpa_fp64(seed):
    rng = np.random.default_rng(100 + seed)
    Hkv = int(rng.integers(1, 4))
    G = int(rng.integers(1, 5))
    Hq, d = Hkv * G, int(rng.choice([8, 16, 64]))
    n_ctx, T = int(rng.integers(0, 70)), int(rng.integers(1, 12))
    parent = _random_parent(rng, T)
    x = attention_inputs(seed, Hq, Hkv, d, n_ctx, T)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    got = verify_attention(q, k, v, n_ctx, parent)
    ref = _sdpa(q, k, v, n_ctx, _reach_mask(parent, n_ctx))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_explicit_scale_matches_sdpa():
    x = attention_inputs(7, 4, 2, 32, 40, 5)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    parent = [-1, 0, 0, 1, 3]
    got = verify_attention(q, k, v, 40, parent, scale=0.37)
    ref = _sdpa(q, k, v, 40, _reach_mask(parent, 40), scale=0.37)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_chain_tree_is_causal_decode():
    # A chain is ordinary decoding: token i sees rows [0, n_ctx + i].
    n_ctx, T = 57, 6
    x = attention_inputs(3, 6, 2, 16, n_ctx, T)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    got = verify_attention(q, k, v, n_ctx, tree_parent("chain", T))
    causal = torch.ones(T, n_ctx + T, dtype=torch.bool).tril(diagonal=n_ctx)
    ref = _sdpa(q, k, v, n_ctx, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # token by token: one query at a time over the first n_ctx + i + 1 rows
    for i in range(T):
        one = verify_attention(q[:, i:i + 1], k[:, : n_ctx + i + 1], v[:, : n_ctx + i + 1], n_ctx + i, [-1])
        np.testing.assert_allclose(got[:, i:i + 1], one, rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    x = attention_inputs(4, 8, 2, 16, 30, 8)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    parent = tree_parent("tiny8")
    gqa = verify_attention(q, k, v, 30, parent)
    mha = verify_attention(q, np.repeat(k, 4, axis=0), np.repeat(v, 4, axis=0), 30, parent)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-14)


def test_uniform_keys_give_mean_of_visible_values():
    n_ctx, T, d = 20, 8, 8
    x = attention_inputs(5, 2, 1, d, n_ctx, T)
    q, v = bf16_to_f64(x["q"]), bf16_to_f64(x["v"])
    k = np.ones((1, n_ctx + T, d))
    parent = tree_parent("tiny8")
    got = verify_attention(q, k, v, n_ctx, parent)
    # node 3's ancestors are 0,1,2,3; node 5's are 0 and 5
    for i, anc in ((0, [0]), (3, [0, 1, 2, 3]), (5, [0, 5])):
        rows = list(range(n_ctx)) + [n_ctx + a for a in anc]
        np.testing.assert_allclose(got[:, i], np.broadcast_to(v[0, rows].mean(axis=0), (2, d)), rtol=1e-13, atol=1e-14)


def test_empty_context_single_node_returns_its_value():
    x = attention_inputs(6, 3, 1, 16, 0, 1)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    got = verify_attention(q, k, v, 0, [-1])
    np.testing.assert_array_equal(got, np.broadcast_to(v[0, 0], (3, 1, 16)))


def test_dominant_key_selects_its_value():
    n_ctx, T, d = 50, 3, 16
    x = attention_inputs(8, 1, 1, d, n_ctx, T)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    k[0, 17] = 40.0 * q[0, 0]  # huge score for node 0 at row 17
    got = verify_attention(q, k, v, n_ctx, [-1, 0, 1])
    np.testing.assert_allclose(got[0, 0], v[0, 17], atol=1e-9)


def test_mask_direction_only_ancestors_matter():
    n_ctx, T, d = 12, 8, 8
    x = attention_inputs(9, 2, 1, d, n_ctx, T)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    parent = tree_parent("tiny8")  # node 2's ancestors: 0, 1, 2
    base = verify_attention(q, k, v, n_ctx, parent)
    for other in (3, 4, 7):        # a descendant and two non-ancestors of node 2
        k2, v2 = k.copy(), v.copy()
        k2[0, n_ctx + other] += 5.0
        v2[0, n_ctx + other] -= 3.0
        out = verify_attention(q, k2, v2, n_ctx, parent)
        np.testing.assert_array_equal(out[:, 2], base[:, 2])
    v3 = v.copy()
    v3[0, n_ctx + 1] += 1.0        # an ancestor of node 2
    assert not np.allclose(verify_attention(q, k, v3, n_ctx, parent)[:, 2], base[:, 2])


def test_permuting_committed_rows_is_invariant():
    n_ctx, T = 33, 4
    x = attention_inputs(10, 4, 2, 16, n_ctx, T)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    perm = np.concatenate([np.random.default_rng(1).permutation(n_ctx), np.arange(n_ctx, n_ctx + T)])
    parent = [-1, 0, 1, 0]
    a = verify_attention(q, k, v, n_ctx, parent)
    b = verify_attention(q, k[:, perm], v[:, perm], n_ctx, parent)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_draft_attention_is_chain_verification():
    x = attention_inputs(11, 4, 1, 16, 25, 4)
    q, k, v = (bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    np.testing.assert_array_equal(draft_attention(q, k, v, 25), verify_attention(q, k, v, 25, [-1, 0, 1, 2]))


def test_ancestor_sets_and_validation():
    assert ancestor_sets(tree_parent("tiny8")) == [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3], [0, 4], [0, 5], [0, 6], [0, 7]]
    for bad in ([0], [-1, 1], [-1, 0, 3], [-1, -1]):
        with pytest.raises(ValueError):
            ancestor_sets(bad)


def test_tree_generator_shapes():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tree_shapes.json")))
    for T in (10, 24, 64):
        par = tree_parent("tokenswift", T)
        assert len(par) == T and par[0] == -1 and all(0 <= par[i] < i for i in range(1, T))
        depth = [0] * T
        for i in range(1, T):
            depth[i] = depth[par[i]] + 1
        # root + one level per extra head; a reused 4-gram adds its 3 continuation tokens
        assert max(depth) == g["extra_heads"] == g["ngram_len"] - 1 == len(g["tree_levels"]) - 1
        # the head part: 3 candidates per level along the top-1 path
        kids = lambda n: [i for i in range(T) if par[i] == n]
        assert kids(1)[:3] == [4, 5, 6] and kids(4) == [7, 8, 9]
    assert tree_parent("chain", 4) == [-1, 0, 1, 2]


def test_bf16_round_trip_is_exact_and_nearest_even():
    x = np.array([1.0, -2.5, 3.140625, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0], dtype=np.float32)
    back = bf16_to_f64(bf16_round(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    np.testing.assert_array_equal(back, [1.0, -2.5, 3.140625, 1.0, 1.0 + 2.0 ** -6, 65536.0])
