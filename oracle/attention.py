"""Oracle for tree-masked verification attention and draft attention.

Test infrastructure only (see the package docstring).

Definition (TokenSwift summary, §3.1 "Overview" with Figure 2, and Appendix E
"Tree-Based Attention"; GQA grouping from §3.3): the target model verifies the
whole draft tree in one forward pass over the FULL KV cache, each tree token
attending to the committed context and to its own predecessors in the tree.
Drafting runs the same model over a PARTIAL cache (§3.1, §3.3).

Readings taken where the pages are silent:

* Scale defaults to 1/sqrt(d).
* The tree's own keys and values sit right after the committed context, at
  rows ``n_ctx .. n_ctx+T-1`` of the same cache (node i at row n_ctx+i).
* Query head h uses KV head ``h // G`` with ``G = Hq // Hkv`` (the query heads
  of one KV head are consecutive).
* Node i sees committed rows ``0 .. n_ctx-1`` and tree rows
  ``n_ctx + a`` for every a in its ancestor set (itself included).
"""

import numpy as np

from .common import ancestor_sets


def _softmax_rows_axis0(s):
    """Softmax along axis 0; masked entries are -inf and get probability 0."""
    m = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=0, keepdims=True)


def verify_attention(q, k, v, n_ctx, parent, scale=None):
    """Tree verification attention in float64.

    q: float array [Hq][T][d] -- one query per (head, tree node).
    k, v: float arrays [Hkv][rows][d] with rows >= n_ctx + T.
    parent: length-T list, parent[0] = -1, 0 <= parent[i] < i.
    Returns O: float64 [Hq][T][d] with

        O[h,i] = sum_{j in Vis(i)} softmax_j(scale * q[h,i].k[g,j]) v[g,j],
        g = h // (Hq/Hkv),
        Vis(i) = {0..n_ctx-1} U {n_ctx + a : a ancestor-or-self of i}.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if len(parent) != T:
        raise ValueError("parent must have one entry per tree node")
    if k.shape[1] < n_ctx + T or v.shape[1] < n_ctx + T:
        raise ValueError("cache must hold n_ctx + T rows")
    G = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    anc = ancestor_sets(parent)

    # visible[r, i]: may node i see cache row r (r < n_ctx + T)?
    visible = np.zeros((n_ctx + T, T), dtype=bool)
    visible[:n_ctx, :] = True
    for i in range(T):
        for a in anc[i]:
            visible[n_ctx + a, i] = True

    out = np.empty((Hq, T, d), dtype=np.float64)
    for g in range(Hkv):
        kg = k[g, : n_ctx + T]
        vg = v[g, : n_ctx + T]
        for h in range(g * G, (g + 1) * G):
            s = scale * (kg @ q[h].T)            # [rows][T]
            s = np.where(visible, s, -np.inf)
            p = _softmax_rows_axis0(s)           # each column sums to 1
            out[h] = p.T @ vg                    # [T][d]
    return out


def draft_attention(q, k_part, v_part, n_part, scale=None):
    """Draft attention over the partial cache (TokenSwift summary, §3.1, §3.3).

    The drafting pass feeds a short chain of Tq new tokens; token t sees the
    n_part partial-cache rows and its own rows n_part .. n_part+t (causal).
    That is verification attention with the chain tree parent[t] = t-1.
    """
    Tq = np.asarray(q).shape[1]
    chain = [-1] + list(range(Tq - 1)) if Tq > 0 else []
    return verify_attention(q, k_part, v_part, n_part, chain, scale)
