"""Oracle for tree acceptance and the post-acceptance KV commit.

Test infrastructure only (see the package docstring).

Definitions: TokenSwift summary §3.1 with Figure 2 (the target model checks
the drafted tree in one pass over the full KV cache; the longest valid draft
is accepted and the caches are updated with it) and Appendix A "Lossless
Nature of Speculative Decoding" (acceptance and rejection together keep the
target model's sampling distribution).

Readings taken where the pages are silent:

* Node 0 of the tree is the root, the last committed token; its K/V row is
  written by the verification pass at cache row L = n_ctx, node i's at
  L + i. Nodes 1..T-1 are drafted tokens.
* target[i] is the target model's token at node i: a draw from its processed
  distribution there (penalty, temperature, top-p, min-p, inverse-CDF
  sampling), or the argmax for greedy decoding. A child c of node p continues
  a valid draft iff node_token[c] == target[p] ("sample, then match": every
  emitted token is the target's own draw, so the output distribution is the
  target's; with one drafted token per position this is exactly App. A's
  accept-with-probability-p / resample-the-rest rule).
* The accepted path ends at the deepest node all of whose edges from the root
  are valid; among equally deep ones, the smallest node index. Its nodes
  a_0 = 0 < a_1 < ... < a_m (a parent is listed before its children, so
  index order is depth order) are committed, and target[a_m] is the next
  token, emitted after them.
* KV commit: row L + k of the full cache receives the K/V of row L + a_k
  (k = 0..m); rows past L + m keep their contents. When a partial cache is
  given, the same m + 1 rows are appended to it at rows n_part + k.
"""

import numpy as np

from .common import ancestor_sets


def accept_path(parent, node_token, target):
    """Accepted path and next token of one verified tree.

    Returns (path, next_token): path = [a_0 = 0, a_1, ..., a_m].
    """
    parent = [int(p) for p in parent]
    ancestor_sets(parent)   # validates the tree (parent[0] = -1, parent[i] < i)
    T = len(parent)
    node_token = [int(t) for t in node_token]
    target = [int(t) for t in target]
    if len(node_token) != T or len(target) != T:
        raise ValueError("node_token and target need one entry per node")
    valid = [False] * T
    depth = [0] * T
    valid[0] = True
    for i in range(1, T):
        p = parent[i]
        valid[i] = valid[p] and node_token[i] == target[p]
        depth[i] = depth[p] + 1
    best = max((i for i in range(T) if valid[i]), key=lambda i: (depth[i], -i))
    path = []
    i = best
    while i != -1:
        path.append(i)
        i = parent[i]
    path.reverse()
    return path, target[best]


def kv_commit(k, v, n_ctx, path, k_part=None, v_part=None, n_part=0):
    """The caches after committing an accepted path (copies; inputs untouched).

    k, v: [..., Hkv, rows, d] full caches (leading axes, e.g. layers, are kept);
    k_part, v_part: partial caches of the same leading shape, or None.
    Returns (k, v, k_part, v_part).
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    src = [n_ctx + a for a in path]
    dst = [n_ctx + j for j in range(len(path))]
    moved_k = k[..., src, :].copy()
    moved_v = v[..., src, :].copy()
    k[..., dst, :] = moved_k
    v[..., dst, :] = moved_v
    if k_part is not None:
        k_part = np.array(k_part, copy=True)
        v_part = np.array(v_part, copy=True)
        rows = [n_part + j for j in range(len(path))]
        k_part[..., rows, :] = moved_k
        v_part[..., rows, :] = moved_v
    return k, v, k_part, v_part
