"""GPU parity of ts_ngram_tree against the oracle: integer work, exact."""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import ngram_tree
from synth import ngram_window
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu


def _check(window, k, seed, head, T_max):
    w = torch.from_numpy(np.ascontiguousarray(window, dtype=np.int32)).to("cuda:0")
    h = None if head is None or len(head) == 0 else torch.tensor(head, dtype=torch.int32, device="cuda:0")
    parent, tok, info = ts.ngram_tree(w, k, seed, h, T_max)
    torch.cuda.synchronize()
    parent, tok, info = parent.cpu().numpy(), tok.cpu().numpy(), info.cpu().numpy()
    ref = ngram_tree(window, k, seed, head or [], T_max)
    T = ref["T"]
    assert list(info) == [T, ref["chains"], ref["distinct"], ref["occurrences"]]
    assert list(parent[:T]) == ref["parent"] and list(tok[:T]) == ref["node_token"]
    assert np.all(parent[T:] == -1) and np.all(tok[T:] == -1)


HEAD = [[11, 12, 13], [21, 22, 23], [31, 32, 33]]


@pytest.mark.parametrize("seed", range(24))
def test_random_windows(seed):
    W = [1, 3, 4, 5, 17, 256, 1024, 4096][seed % 8]
    vocab = [2, 3, 6, 50, 1000][seed % 5]
    window = ngram_window(seed, W, vocab=vocab, repeat=0.1 + 0.1 * (seed % 8))
    k = [0, 1, 3, 20, 100][seed % 5]
    levels = seed % 4
    T_max = [1, 10, 24, 64, 128][seed % 5]
    banner(f"ngram W={W} vocab={vocab} k={k} levels={levels} T_max={T_max}")
    _check(window, k, 1000 + seed, HEAD[:levels], T_max)


@pytest.mark.parametrize("seed", [0, 1, 2**63 + 5, 2**64 - 1])
def test_random_choice_many_distinct(seed):
    # vocabulary 3 and a 4096-token window: dozens of distinct continuations for k = 20
    window = ngram_window(9, 4096, vocab=3, repeat=0.0)
    _check(window, 20, seed, HEAD, 64)


def test_one_token_window_and_constant_window():
    _check(np.array([5], dtype=np.int32), 20, 0, HEAD, 24)
    _check(np.full(4096, 7, dtype=np.int32), 20, 0, HEAD, 64)      # 4093 occurrences of one continuation


def test_workload_window():
    window = ngram_window(3, 1024, vocab=128256, repeat=0.5, n_phrases=8)
    _check(window, 20, 123, HEAD, 24)
    _check(window, 20, 123, HEAD, 64)
    _check(window, 40, 123, HEAD, 128)
