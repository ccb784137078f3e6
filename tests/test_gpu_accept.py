"""GPU parity of ts_tree_accept and ts_kv_commit against the oracle.

Both are integer / byte work: the accepted path, the next token and every
cache byte must equal the oracle's exactly.
"""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from oracle import accept_path, kv_commit
from synth import accept_inputs, penalty_inputs, random_parent, tree_parent
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def _check_accept(parent, node, target):
    res = ts.tree_accept(parent, _i32(node), _i32(target))
    torch.cuda.synchronize()
    res = res.cpu().numpy()
    path, nxt = accept_path(parent, node, target)
    n = len(path)
    assert res[0] == n and res[1] == nxt, (res[:2], n, nxt)
    assert list(res[2:2 + n]) == path
    assert np.all(res[2 + n:] == -1)
    return res, path


@pytest.mark.parametrize("seed", range(40))
def test_accept_random_trees(seed):
    T = [1, 2, 3, 5, 8, 24, 37, 63, 64, 65, 100, 127, 128][seed % 13]
    parent = random_parent(seed, T)
    x = accept_inputs(seed, parent, vocab=2 + seed % 5, p_match=0.4 + 0.15 * (seed % 4))
    _check_accept(parent, x["node_token"], x["target"])


@pytest.mark.parametrize("kind,T", [("tokenswift", 24), ("tokenswift", 64), ("chain", 64), ("chain", 1),
                                    ("tiny8", 8), ("wide", 88), ("chain", 128), ("wide", 128)])
@pytest.mark.parametrize("p_match", [0.0, 0.5, 1.0])
def test_accept_tree_shapes(kind, T, p_match):
    parent = tree_parent(kind, T)
    x = accept_inputs(T + int(10 * p_match), parent, vocab=7, p_match=p_match)
    _check_accept(parent, x["node_token"], x["target"])


def _rand_bf16(shape, gen):
    return torch.randint(-32768, 32767, shape, generator=gen, device="cuda:0", dtype=torch.int16).view(torch.bfloat16)


@pytest.mark.parametrize("layers,Hkv,d,n_ctx,T,part,pad", [
    (1, 2, 128, 100, 24, True, 0), (3, 2, 64, 517, 8, True, 8), (4, 8, 128, 0, 64, False, 0),
    (2, 1, 128, 33, 1, True, 16), (5, 3, 64, 1000, 64, True, 0), (2, 2, 128, 300, 128, True, 8),
    (3, 2, 64, 99, 88, True, 0),
])
def test_commit_matches_oracle(layers, Hkv, d, n_ctx, T, part, pad):
    banner(f"commit layers={layers} Hkv={Hkv} d={d} n_ctx={n_ctx} T={T} part={part} pad={pad}")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(n_ctx + T)
    rows = n_ctx + T + 5
    kf, vf = _rand_bf16((layers, Hkv, rows, d + pad), gen), _rand_bf16((layers, Hkv, rows, d + pad), gen)
    k, v = kf[..., :d], vf[..., :d]
    parent = (tree_parent("wide", T) if T > 64 else tree_parent("tokenswift", T)) if T > 1 else [-1]
    x = accept_inputs(T, parent, vocab=3, p_match=0.8)
    res, path = _check_accept(parent, x["node_token"], x["target"])
    res_d = _i32(res)
    n_part, cap = 17, 17 + T + 2
    kp = _rand_bf16((layers, Hkv, cap, d), gen) if part else None
    vp = _rand_bf16((layers, Hkv, cap, d), gen) if part else None
    host = lambda t: None if t is None else t.view(torch.int16).cpu().numpy()
    k0, v0, kp0, vp0 = host(kf), host(vf), host(kp), host(vp)
    ts.kv_commit(res_d, T, k, v, n_ctx, kp, vp, n_part)
    torch.cuda.synchronize()
    want_k, want_v, want_kp, want_vp = kv_commit(k0[..., :d], v0[..., :d], n_ctx, path, kp0, vp0, n_part)
    np.testing.assert_array_equal(host(kf)[..., :d], want_k)
    np.testing.assert_array_equal(host(vf)[..., :d], want_v)
    np.testing.assert_array_equal(host(kf)[..., d:], k0[..., d:])   # padding channels untouched
    if part:
        np.testing.assert_array_equal(host(kp), want_kp)
        np.testing.assert_array_equal(host(vp), want_vp)


def test_commit_full_size_8b():
    """32 layers x 8 KV heads at 100K rows: the rows around the tree, every layer."""
    layers, Hkv, d, n_ctx, T = 32, 8, 128, 100_000, 24
    banner("commit full 8b")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(8)
    k, v = _rand_bf16((layers, Hkv, n_ctx + T, d), gen), _rand_bf16((layers, Hkv, n_ctx + T, d), gen)
    kp, vp = _rand_bf16((layers, Hkv, 4164 + T, d), gen), _rand_bf16((layers, Hkv, 4164 + T, d), gen)
    parent = tree_parent("tokenswift", T)
    x = accept_inputs(3, parent, vocab=2, p_match=0.9)
    res, path = _check_accept(parent, x["node_token"], x["target"])
    lo = n_ctx - 3
    win = lambda t: t[:, :, lo:].view(torch.int16).cpu().numpy()
    k0, v0 = win(k), win(v)
    kp0, vp0 = kp.view(torch.int16).cpu().numpy(), vp.view(torch.int16).cpu().numpy()
    ts.kv_commit(_i32(res), T, k, v, n_ctx, kp, vp, 4164)
    torch.cuda.synchronize()
    wk, wv, wkp, wvp = kv_commit(k0, v0, n_ctx - lo, path, kp0, vp0, 4164)
    np.testing.assert_array_equal(win(k), wk)
    np.testing.assert_array_equal(win(v), wv)
    np.testing.assert_array_equal(kp.view(torch.int16).cpu().numpy(), wkp)
    np.testing.assert_array_equal(vp.view(torch.int16).cpu().numpy(), wvp)


def test_sampled_targets_through_accept_and_commit():
    """Target tokens drawn by ts_penalty_sample for the tree's rows, drafts
    planted along two branches, then acceptance and commit."""
    T, V = 24, 1024
    banner("penalty -> accept -> commit")
    parent = tree_parent("tokenswift", T)
    x = penalty_inputs(5, T, V, 64)
    logits = torch.from_numpy(x["logits"]).to("cuda:0")
    window = torch.from_numpy(x["window"]).to("cuda:0")
    u = torch.from_numpy(x["u"]).to("cuda:0")
    _, _, _, tok = ts.penalty_sample(logits, window, 1.2, 1.0, 0.9, 0.05, u=u, want_keep=False, want_probs=False)
    target = tok.cpu().numpy()
    node = np.full(T, -5, dtype=np.int32)
    node[1], node[4] = target[0], target[1]                      # head branch, depth 2
    node[13], node[14], node[15] = target[0], target[13], target[14]   # 4-gram branch, depth 3
    res, path = _check_accept(parent, node, target)
    assert path == [0, 13, 14, 15] and res[1] == target[15]
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1)
    k, v = _rand_bf16((2, 2, 300 + T, 128), gen), _rand_bf16((2, 2, 300 + T, 128), gen)
    k0, v0 = k.view(torch.int16).cpu().numpy(), v.view(torch.int16).cpu().numpy()
    ts.kv_commit(_i32(res), T, k, v, 300)
    torch.cuda.synchronize()
    wk, wv, _, _ = kv_commit(k0, v0, 300, path)
    np.testing.assert_array_equal(k.view(torch.int16).cpu().numpy(), wk)
    np.testing.assert_array_equal(v.view(torch.int16).cpu().numpy(), wv)
