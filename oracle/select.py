"""Oracle for the dynamic partial-KV update (score, top-budget select, gather).

Test infrastructure only (see the package docstring).

Definition (TokenSwift summary, §3.3 "Dynamic KV Cache Management", and §2
"Challenges"): the drafting cache has a fixed budget; it always keeps the
initial |S| key/value pairs and, as generation goes on, swaps out the less
important pairs. Importance is a query-key dot product; under GQA the queries
of one KV head are grouped (keys are not replicated) and their scores summed.

Readings taken where the pages are silent:

* The score of cached position j under KV head g sums q.k over every query
  head of the group and every current query (tree node):
  sigma_g[j] = sum_{h in group g} sum_t sum_c q[h,t,c] k[g,j,c].
  No softmax, no absolute value, no pooling.
* Besides the |S| = n_sink initial rows, the n_recent most recent committed
  rows are always kept; the candidates are C = [n_sink, n_ctx - n_recent).
* The budget counts selected candidates only: B' = min(budget, |C|).
* Order is (score descending, position ascending); ties go to the earlier
  position. Selected positions are emitted ascending and padded with -1.
* Partial rows per head: sink U selected U recent, ascending.
"""

from dataclasses import dataclass

import numpy as np


@dataclass
class SelectResult:
    scores: np.ndarray   # float64 [Hkv][n_ctx]; sigma for every committed row
    sel_idx: np.ndarray  # int64 [Hkv][budget]; ascending, -1 padded
    rows: list           # per head: ascending int64 array of kept rows
    n_part: int          # rows per head in the partial cache
    cutoff: np.ndarray   # float64 [Hkv]; score of the last selected candidate (nan if none)


def candidate_range(n_ctx, n_sink, n_recent):
    lo = n_sink
    hi = n_ctx - n_recent
    return (lo, hi) if hi > lo else (lo, lo)


def partial_kv_select(q, k, n_ctx, Hkv, n_sink, budget, n_recent):
    """Scores, selected indices and the kept row set for each KV head.

    q: float [Hq][T][d]; k: float [Hkv][rows][d] with rows >= n_ctx.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Hq, T, d = q.shape
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    lo, hi = candidate_range(n_ctx, n_sink, n_recent)
    cand = np.arange(lo, hi, dtype=np.int64)
    b_eff = min(budget, len(cand))

    scores = np.zeros((Hkv, n_ctx), dtype=np.float64)
    sel = np.full((Hkv, budget), -1, dtype=np.int64)
    cutoff = np.full(Hkv, np.nan)
    rows = []
    sink = np.arange(0, min(n_sink, n_ctx), dtype=np.int64)
    recent = np.arange(max(n_sink, n_ctx - n_recent), n_ctx, dtype=np.int64)
    for g in range(Hkv):
        kg = k[g, :n_ctx]
        sig = np.zeros(n_ctx, dtype=np.float64)
        # Direct form: every (head, query) dot product, then the sum.
        for h in range(g * G, (g + 1) * G):
            sig += (kg @ q[h].T).sum(axis=1)
        scores[g] = sig
        if b_eff > 0:
            cs = sig[cand]
            order = np.lexsort((cand, -cs))      # primary: -score; then position
            chosen = cand[order[:b_eff]]
            cutoff[g] = cs[order[b_eff - 1]]
            chosen = np.sort(chosen)
            sel[g, :b_eff] = chosen
        else:
            chosen = np.zeros(0, dtype=np.int64)
        rows.append(np.concatenate([sink, chosen, recent]))
    n_part = int(len(rows[0])) if Hkv > 0 else 0
    return SelectResult(scores=scores, sel_idx=sel, rows=rows, n_part=n_part, cutoff=cutoff)


def gather_partial(k, v, rows):
    """Partial cache rows per head: k_part[g, r] = k[g, rows[g][r]]."""
    k = np.asarray(k)
    v = np.asarray(v)
    kp = np.stack([k[g, r] for g, r in enumerate(rows)])
    vp = np.stack([v[g, r] for g, r in enumerate(rows)])
    return kp, vp
