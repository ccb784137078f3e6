"""Pins for the tree-acceptance and KV-commit oracle.

The accepted path is checked against a backward walk from every node (a
formulation independent of the oracle's forward pass), the chain case's
closed form (the longest prefix of matching tokens), and hand-derived trees
for the tie rules. The commit is checked by tracking row labels.
"""

import numpy as np
import pytest

from oracle import accept_path, kv_commit
from synth import accept_inputs, random_parent, tree_parent


def _walk_back(parent, node_token, target):
    """Every node whose edges to the root all match, found by walking up."""
    out = []
    for i in range(len(parent)):
        j, ok, depth = i, True, 0
        while parent[j] != -1:
            if node_token[j] != target[parent[j]]:
                ok = False
            j, depth = parent[j], depth + 1
        if ok:
            out.append((depth, i))
    return out


@pytest.mark.parametrize("seed", range(40))
def test_matches_backward_walk(seed):
    T = 1 + seed % 64
    parent = random_parent(seed, T)
    x = accept_inputs(seed, parent, vocab=4, p_match=0.6)
    path, nxt = accept_path(parent, x["node_token"], x["target"])
    valid = _walk_back(parent, x["node_token"], x["target"])
    depth, end = min(valid, key=lambda dv: (-dv[0], dv[1]))
    assert path[-1] == end and len(path) == depth + 1
    assert nxt == x["target"][end]
    # the path is the end node's root path, in index order
    chain = [end]
    while parent[chain[-1]] != -1:
        chain.append(parent[chain[-1]])
    assert path == chain[::-1]


@pytest.mark.parametrize("seed", range(10))
def test_chain_accepts_the_longest_matching_prefix(seed):
    T = 2 + 6 * seed
    parent = tree_parent("chain", T)
    x = accept_inputs(seed, parent, vocab=3, p_match=0.8)
    eq = x["node_token"][1:] == x["target"][:-1]     # draft t matches the target's token at t-1
    n = int(np.argmin(np.append(eq, False)))          # first mismatch
    path, nxt = accept_path(parent, x["node_token"], x["target"])
    assert path == list(range(n + 1))
    assert nxt == x["target"][n]


def test_no_match_keeps_only_the_root():
    parent = tree_parent("tokenswift", 24)
    target = np.arange(24) + 100
    node = np.zeros(24, dtype=np.int32)      # never equals a target token
    assert accept_path(parent, node, target) == ([0], 100)
    assert accept_path([-1], [5], [9]) == ([0], 9)


def test_duplicate_siblings_take_the_deeper_branch():
    # nodes 1 and 2 both carry the target's token at the root; only node 2
    # has a matching child (node 3), so the path goes through node 2
    parent = [-1, 0, 0, 2, 1]
    target = [7, 8, 9, 4, 6]
    node = [0, 7, 7, 9, 1]        # node 4 needs 8 (target[1]) and has 1
    assert accept_path(parent, node, target) == ([0, 2, 3], 4)


def test_equal_depth_takes_the_smaller_end_index():
    parent = [-1, 0, 0, 1, 2]
    target = [5, 6, 7, 1, 2]
    node = [0, 5, 5, 6, 7]        # nodes 3 and 4 both valid at depth 2
    assert accept_path(parent, node, target) == ([0, 1, 3], 1)


def test_tokenswift_tree_ngram_chain_beats_shorter_head_path():
    # tree of 24: heads 1-3 under the root, 4-6 under node 1, 7-9 under node 4;
    # 4-gram chains (10, 11, 12), (13, 14, 15), ... under the root
    parent = tree_parent("tokenswift", 24)
    target = np.arange(24) + 1000
    node = np.zeros(24, dtype=np.int64)
    node[1] = target[0]; node[4] = target[1]          # head path 0-1-4: depth 2
    node[13] = target[0]; node[14] = target[13]; node[15] = target[14]   # chain: depth 3
    assert accept_path(parent, node, target) == ([0, 13, 14, 15], 1015)
    node[7] = target[4]                                # head path now depth 3 too: smaller end index 7
    assert accept_path(parent, node, target) == ([0, 1, 4, 7], 1007)


def test_bad_tree_is_rejected():
    with pytest.raises(ValueError):
        accept_path([0, 0], [1, 1], [1, 1])
    with pytest.raises(ValueError):
        accept_path([-1, 1], [1, 1], [1, 1])


@pytest.mark.parametrize("path", [[0], [0, 1, 2], [0, 2, 5], [0, 13, 14, 15], [0, 1, 4, 7]])
def test_commit_moves_labelled_rows(path):
    layers, Hkv, d, n_ctx, T, n_part, cap = 3, 2, 4, 10, 24, 5, 40
    rows = n_ctx + T + 3
    lab = np.arange(rows, dtype=np.float64)
    k = np.broadcast_to(lab[None, None, :, None], (layers, Hkv, rows, d)).copy()
    k += 1000 * np.arange(layers)[:, None, None, None] + 100000 * np.arange(Hkv)[None, :, None, None]
    v = -k
    kp = np.full((layers, Hkv, cap, d), -7.0)
    vp = np.full((layers, Hkv, cap, d), -9.0)
    k2, v2, kp2, vp2 = kv_commit(k, v, n_ctx, path, kp, vp, n_part)
    m = len(path)
    for j in range(rows):
        want = n_ctx + path[j - n_ctx] if n_ctx <= j < n_ctx + m else j
        np.testing.assert_array_equal(k2[:, :, j], k[:, :, want])
        np.testing.assert_array_equal(v2[:, :, j], v[:, :, want])
    for r in range(cap):
        if n_part <= r < n_part + m:
            np.testing.assert_array_equal(kp2[:, :, r], k[:, :, n_ctx + path[r - n_part]])
            np.testing.assert_array_equal(vp2[:, :, r], v[:, :, n_ctx + path[r - n_part]])
        else:
            assert np.all(kp2[:, :, r] == -7.0) and np.all(vp2[:, :, r] == -9.0)
    # inputs are untouched and the partial cache is optional
    assert np.all(k[..., 0, 0, n_ctx, :] == n_ctx)
    k3, v3, kp3, vp3 = kv_commit(k, v, n_ctx, path)
    np.testing.assert_array_equal(k3, k2)
    assert kp3 is None and vp3 is None
