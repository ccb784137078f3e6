"""Pins for the n-gram retrieval, random choice and tree-builder oracle.

SplitMix64 against its published outputs; retrieval against a NumPy sliding
window with np.unique; the random choice against an independent argsort and
a frequency check over many seeds; the tree against a hand-built case and
the tree shape of the workloads.
"""

import numpy as np
import pytest

from oracle import ngram_candidates, ngram_tree, splitmix64
from synth import ngram_window, tree_parent


def test_splitmix64_published_outputs():
    # first outputs of SplitMix64 started from state 0 (the generator's reference outputs)
    assert [splitmix64(0, j) for j in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def _unique_continuations(window):
    w = np.asarray(window, dtype=np.int64)
    if len(w) < 4:
        return {}
    grams = np.lib.stride_tricks.sliding_window_view(w, 4)[: len(w) - 3]
    sel = np.nonzero(grams[:, 0] == w[-1])[0]
    keys, first, counts = np.unique(grams[sel, 1:], axis=0, return_index=True, return_counts=True)
    return {tuple(int(x) for x in kk): (int(sel[f]), int(c)) for kk, f, c in zip(keys, first, counts)}


@pytest.mark.parametrize("seed", range(12))
def test_retrieval_matches_sliding_window(seed):
    W = [4, 5, 64, 300, 1024, 2000][seed % 6]
    w = ngram_window(seed, W, vocab=3 + seed % 4, repeat=0.6)
    chosen, n_distinct, n_occ = ngram_candidates(w, 10_000, seed)   # k above every count: all kept
    ref = _unique_continuations(w)
    assert n_distinct == len(ref)
    assert n_occ == sum(c for _, c in ref.values())
    assert {c[0]: (c[2], c[1]) for c in chosen} == ref
    keys = [(-c[1], c[2]) for c in chosen]
    assert keys == sorted(keys)


@pytest.mark.parametrize("seed", range(8))
def test_random_choice_is_the_k_smallest_keys(seed):
    w = ngram_window(100 + seed, 1024, vocab=5, repeat=0.2)
    k = 3 + seed
    chosen, n_distinct, _ = ngram_candidates(w, k, seed * 7919)
    ref = _unique_continuations(w)
    assert n_distinct > k
    by_first = sorted(ref.items(), key=lambda kv: kv[1][0])          # q = index in first-occurrence order
    rho = np.array([splitmix64(seed * 7919, q) for q in range(len(by_first))], dtype=np.uint64)
    keep = np.argsort(rho, kind="stable")[:k]
    assert {c[0] for c in chosen} == {by_first[q][0] for q in keep}


def test_random_choice_is_uniform_over_seeds():
    # a window with d = 8 distinct continuations of the root, k = 2: each kept with probability 1/4
    w = []
    for j in range(8):
        w += [9, 100 + j, 200 + j, 300 + j]
    w += [9]
    hits = np.zeros(8)
    for s in range(4000):
        chosen, d, _ = ngram_candidates(w, 2, s)
        assert d == 8 and len(chosen) == 2
        for c in chosen:
            hits[c[0][0] - 100] += 1
    assert np.all(np.abs(hits / 4000 - 0.25) < 0.03), hits / 4000


def test_hand_built_tree():
    w = [5, 1, 2, 3, 5, 1, 2, 3, 5, 7, 8, 9, 5]
    head = [[11, 12, 13], [21, 22, 23], [31, 32, 33]]
    r = ngram_tree(w, 20, 0, head, 24)
    assert r["parent"] == [-1, 0, 0, 0, 1, 1, 1, 4, 4, 4, 0, 10, 11, 0, 13, 14]
    assert r["node_token"] == [5, 11, 12, 13, 21, 22, 23, 31, 32, 33, 1, 2, 3, 7, 8, 9]
    assert (r["T"], r["chains"], r["distinct"], r["occurrences"]) == (16, 2, 2, 3)
    assert r["parent"] == tree_parent("tokenswift", 16)
    cut = ngram_tree(w, 20, 0, head, 12)                 # the first chain cut after two nodes
    assert cut["parent"] == [-1, 0, 0, 0, 1, 1, 1, 4, 4, 4, 0, 10]
    assert (cut["T"], cut["chains"]) == (12, 1)
    assert ngram_tree(w, 0, 0, head, 24)["T"] == 10      # k = 0: head part only
    assert ngram_tree(w, 20, 0, [], 24)["parent"] == [-1, 0, 1, 2, 0, 4, 5]


@pytest.mark.parametrize("T", [24, 64])
def test_full_window_gives_the_workload_tree_shape(T):
    w = ngram_window(3, 1024, vocab=40, repeat=0.9, n_phrases=30)
    head = [[1, 2, 3], [4, 5, 6], [7, 8, 9]]
    r = ngram_tree(w, 20, 17, head, T)
    if r["chains"] * 3 + 10 >= T:
        assert r["parent"] == tree_parent("tokenswift", T)


def test_degenerate_windows():
    assert ngram_candidates([7], 20, 0) == ([], 0, 0)
    assert ngram_candidates([7, 7, 7], 20, 0) == ([], 0, 0)            # no complete 4-gram
    chosen, d, n = ngram_candidates([7, 7, 7, 7, 7], 20, 0)            # two overlapping 4-grams, one continuation
    assert chosen == [((7, 7, 7), 2, 0)] and (d, n) == (1, 2)
    assert ngram_tree([3], 20, 0, [], 5)["parent"] == [-1]
    with pytest.raises(ValueError):
        ngram_tree([3], 20, 0, [[1, 2]], 5)
