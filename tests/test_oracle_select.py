"""Pins for the partial-KV selection oracle.

The selection is checked against a rank characterisation written
independently of the oracle's sort, the linear rewrite of the grouped score,
planted keys, the full-budget property (drafting over the partial cache then
equals verification over the full cache), and the degenerate cases.
"""

import numpy as np
import pytest

from oracle import bf16_to_f64, draft_attention, partial_kv_select, verify_attention
from oracle.select import gather_partial
from synth import attention_inputs, tree_parent


def _inputs(seed, Hq, Hkv, d, n_ctx, T):
    x = attention_inputs(seed, Hq, Hkv, d, n_ctx, T)
    return (bf16_to_f64(x[n]) for n in ("q", "k", "v"))


@pytest.mark.parametrize("seed", range(5))
def test_selection_matches_rank_characterisation_with_ties(seed):
    rng = np.random.default_rng(seed)
    Hkv, G, d, n_ctx, T = 2, 3, 8, 60, 4
    q, k, v = _inputs(seed, Hkv * G, Hkv, d, n_ctx, T)
    # exact ties: duplicate key rows give bit-identical scores
    for g in range(Hkv):
        src = rng.choice(np.arange(4, 50), size=6, replace=False)
        k[g, src[3:]] = k[g, src[:3]]
    n_sink, n_recent, budget = 3, 5, int(rng.integers(1, 40))
    r = partial_kv_select(q, k, n_ctx, Hkv, n_sink, budget, n_recent)
    cand = list(range(n_sink, n_ctx - n_recent))
    b_eff = min(budget, len(cand))
    for g in range(Hkv):
        sig = np.einsum("htc,jc->j", q[g * G:(g + 1) * G], k[g, :n_ctx])
        # j is chosen iff fewer than b_eff candidates beat it (higher score, or equal and earlier)
        want = [j for j in cand
                if sum(1 for i in cand if sig[i] > sig[j] or (sig[i] == sig[j] and i < j)) < b_eff]
        got = [int(j) for j in r.sel_idx[g] if j >= 0]
        assert got == want
        assert list(r.sel_idx[g][b_eff:]) == [-1] * (budget - b_eff)


def test_grouped_score_equals_aggregated_query():
    q, k, _ = _inputs(21, 12, 2, 32, 200, 24)
    r = partial_kv_select(q, k, 200, 2, 4, 16, 8)
    for g in range(2):
        qbar = q[g * 6:(g + 1) * 6].sum(axis=(0, 1))
        np.testing.assert_allclose(r.scores[g], k[g, :200] @ qbar, rtol=1e-9, atol=1e-9)


def test_planted_keys():
    q, k, _ = _inputs(22, 4, 1, 16, 120, 3)
    qbar = q.sum(axis=(0, 1))
    k[0, 40] = 3.0 * qbar / np.linalg.norm(qbar)   # strongly aligned: must be selected
    k[0, 41] = -30.0 * qbar / np.linalg.norm(qbar)  # strongly anti-aligned: must not
    r = partial_kv_select(q, k, 120, 1, 4, 10, 8)
    assert 40 in r.sel_idx[0] and 41 not in r.sel_idx[0]


def test_full_budget_partial_draft_equals_full_verification():
    # With the budget covering every candidate, the partial cache is the whole
    # committed cache and drafting over it equals chain verification.
    Hq, Hkv, d, n_ctx, Tq = 8, 2, 16, 90, 4
    q, k, v = _inputs(23, Hq, Hkv, d, n_ctx, Tq)
    r = partial_kv_select(q, k, n_ctx, Hkv, 4, 10_000, 8)
    assert r.n_part == n_ctx
    for g in range(Hkv):
        np.testing.assert_array_equal(r.rows[g], np.arange(n_ctx))
    kp, vp = gather_partial(k[:, :n_ctx], v[:, :n_ctx], r.rows)
    kp = np.concatenate([kp, k[:, n_ctx:n_ctx + Tq]], axis=1)
    vp = np.concatenate([vp, v[:, n_ctx:n_ctx + Tq]], axis=1)
    np.testing.assert_array_equal(draft_attention(q, kp, vp, r.n_part),
                                  verify_attention(q, k, v, n_ctx, tree_parent("chain", Tq)))


@pytest.mark.parametrize("n_ctx,n_sink,budget,n_recent", [
    (100, 4, 16, 8), (100, 0, 16, 0), (100, 4, 0, 8), (10, 4, 16, 8), (12, 4, 16, 8),
    (3, 4, 16, 8), (0, 4, 16, 8), (100, 4, 88, 8), (100, 4, 89, 8),
])
def test_kept_rows_structure(n_ctx, n_sink, budget, n_recent):
    q, k, _ = _inputs(24, 4, 2, 8, max(n_ctx, 1), 2)
    r = partial_kv_select(q, k, n_ctx, 2, n_sink, budget, n_recent)
    n_cand = max(0, n_ctx - n_recent - n_sink)
    expect_n = min(n_sink, n_ctx) + min(budget, n_cand) + (n_ctx - max(n_sink, n_ctx - n_recent) if n_ctx > n_sink else 0)
    assert r.n_part == expect_n
    if n_ctx <= n_sink + n_recent:
        assert r.n_part == n_ctx
    for g in range(2):
        rows = r.rows[g]
        assert len(rows) == r.n_part
        assert np.all(np.diff(rows) > 0)                      # ascending, no duplicates
        assert set(range(min(n_sink, n_ctx))) <= set(rows)   # initial |S| rows always kept
        assert set(range(max(n_sink, n_ctx - n_recent), n_ctx)) <= set(rows)
        sel = r.sel_idx[g]
        assert len(sel) == budget
        s = sel[sel >= 0]
        assert np.all(np.diff(s) > 0) and np.all((s >= n_sink) & (s < n_ctx - n_recent))
