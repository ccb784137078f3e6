"""Shared oracle helpers: bf16 decoding and the tree's ancestor sets.

Test infrastructure only (see the package docstring).
"""

import numpy as np


def bf16_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) exactly into float64.

    A bfloat16 value is the upper half of an IEEE binary32 word, so widening
    the bits to 32 and reinterpreting is exact; binary32 -> binary64 is exact
    too.
    """
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def ancestor_sets(parent):
    """Visible tree nodes for each node of a token tree.

    TokenSwift summary, Appendix E "Tree-Based Attention": the candidate tree
    is verified in one pass and a token may attend only to the tokens that
    precede it on its own branch. Reading taken: a node sees itself and every
    ancestor up to the root (node 0); siblings and descendants are hidden.

    ``parent[0]`` must be -1 and ``0 <= parent[i] < i`` for i > 0 (a node's
    parent is listed before it). Returns a list of sorted index lists.
    """
    parent = [int(p) for p in parent]
    T = len(parent)
    if T == 0:
        return []
    if parent[0] != -1:
        raise ValueError("parent[0] must be -1 (node 0 is the root)")
    for i in range(1, T):
        if not (0 <= parent[i] < i):
            raise ValueError(f"parent[{i}]={parent[i]} must lie in [0, {i})")
    out = []
    for i in range(T):
        chain = []
        j = i
        while j != -1:
            chain.append(j)
            j = parent[j]
        out.append(sorted(chain))
    return out
