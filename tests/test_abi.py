"""C-ABI checks that need no GPU: exports, workspace queries, host validation.

Every call here is rejected by host-side validation, which runs before any
HIP call, so fake (aligned, non-null) device pointers are never dereferenced.
"""

import ctypes
import os
import re

import pytest

from long_kv_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokenswift.h")
EINVAL, ENOTSUP, EWORKSPACE = -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10002)    # misaligned (2-byte)


def _lib():
    if not os.path.exists(binding.lib_path()):
        pytest.skip("libtokenswift.so not built")
    return binding.lib()


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    syms = header_symbols()
    for name in ("ts_verify_attn", "ts_draft_attn", "ts_partial_kv_select", "ts_penalty_sample"):
        assert name in syms and name + "_workspace_size" in syms


def test_library_exports_every_header_symbol():
    L = _lib()
    missing = [s for s in header_symbols() if not hasattr(L, s)]
    assert not missing, missing
    assert L.ts_abi_version() == 107


def test_workspace_queries_depend_on_shapes_only():
    L = _lib()
    a = L.ts_verify_attn_workspace_size(100_000, 24, 32, 8, 128, 0)
    assert a > 0 and a == L.ts_verify_attn_workspace_size(100_000, 24, 32, 8, 128, 0)
    assert L.ts_verify_attn_workspace_size(100_000, 24, 32, 8, 128, 1) == 0   # one split: no partials
    forced = L.ts_verify_attn_workspace_size(100_000, 24, 32, 8, 128, 7)
    assert forced == 7 * 8 * 96 * (128 * 2 + 8)   # f16 partial outputs + (m, l) per row
    assert L.ts_verify_attn_workspace_size(100_000, 129, 32, 8, 128, 0) == 0   # unsupported -> 0
    assert L.ts_draft_attn_workspace_size(4164, 4, 32, 8, 128, 0) == L.ts_verify_attn_workspace_size(4164, 4, 32, 8, 128, 0)
    assert L.ts_partial_kv_select_workspace_size(100_000, 24, 32, 8, 128, 4096) >= 8 * 100_000 * 4
    # chunk partials plus 1024 candidate keys (8 bytes) per chunk; 28 rows -> 9 chunks per row
    assert L.ts_penalty_sample_workspace_size(28, 128256) >= 28 * 9 * 1024 * 8
    assert L.ts_penalty_sample_workspace_size(1, 262144) >= 64 * 1024 * 8


def _verify(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, s_head=128 * 200, s_pos=128, n_ctx=100, T=3, parent=[-1, 0, 1], Hq=8, Hkv=2,
             d=128, scale=0.0, out=FAKE, n_split=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    par = (ctypes.c_int32 * max(1, len(a["parent"])))(*a["parent"]) if a["parent"] is not None else None
    return L.ts_verify_attn(a["q"], a["k"], a["v"], a["s_head"], a["s_pos"], a["n_ctx"], a["T"], par, a["Hq"],
                            a["Hkv"], a["d"], a["scale"], a["out"], a["n_split"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=None), EINVAL, "null"),
    (dict(d=96), ENOTSUP, "head dim"),
    (dict(T=129, parent=[-1] + list(range(128))), ENOTSUP, "129"),
    (dict(T=0, parent=[]), EINVAL, "at least one"),
    (dict(Hq=6, Hkv=4), EINVAL, "multiple"),
    (dict(parent=[0, 0, 1]), EINVAL, "parent[0]"),
    (dict(parent=[-1, 0, 2]), EINVAL, "parent[2]"),
    (dict(parent=[-1, 1, 0]), EINVAL, "parent[1]"),
    (dict(parent=None), EINVAL, "parent"),
    (dict(s_pos=64), EINVAL, "s_pos"),
    (dict(s_pos=130), EINVAL, "s_pos"),
    (dict(s_head=0), EINVAL, "s_head"),
    (dict(k=FAKE_ODD), EINVAL, "aligned"),
    (dict(n_ctx=-1), EINVAL, "negative"),
    (dict(scale=float("nan")), EINVAL, "scale"),
    (dict(n_split=-2), EINVAL, "n_split"),
    (dict(n_ctx=100_000, n_split=0), EWORKSPACE, "workspace"),
])
def test_verify_attn_rejects(kw, code, text):
    L = _lib()
    assert _verify(L, **kw) == code
    assert text in L.ts_last_error().decode()


def _verify_scored(L, scores=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, s_head=128 * 200, s_pos=128, n_ctx=100, T=3, parent=[-1, 0, 1], Hq=8, Hkv=2,
             d=128, scale=0.0, out=FAKE, n_split=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    par = (ctypes.c_int32 * max(1, len(a["parent"])))(*a["parent"])
    return L.ts_verify_attn_scored(a["q"], a["k"], a["v"], a["s_head"], a["s_pos"], a["n_ctx"], a["T"], par, a["Hq"],
                                   a["Hkv"], a["d"], a["scale"], a["out"], scores, a["n_split"], a["ws"],
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,text", [
    (dict(scores=None), EINVAL, "scores is null"),
    (dict(scores=FAKE_ODD), EINVAL, "scores must be 4-byte aligned"),
    # 40 query heads over 8 KV heads with 64 tree nodes: 320 rows per KV head
    (dict(Hq=40, Hkv=8, T=64, parent=[-1] + list(range(63)), s_head=128 * 200), ENOTSUP, "320 query rows"),
    (dict(d=96), ENOTSUP, "head dim"),
    (dict(parent=[0, 0, 1]), EINVAL, "parent[0]"),
    (dict(n_ctx=100_000, n_split=0, s_head=128 * 200_000), EWORKSPACE, "workspace"),
])
def test_verify_attn_scored_rejects(kw, code, text):
    L = _lib()
    assert _verify_scored(L, **kw) == code
    assert text in L.ts_last_error().decode()


def test_draft_attn_rejects():
    L = _lib()
    assert L.ts_draft_attn(FAKE, FAKE, FAKE, 128 * 100, 128, 50, 129, 8, 2, 128, 0.0, FAKE, 0, None, 0, None) == ENOTSUP
    assert L.ts_draft_attn(FAKE, FAKE, None, 128 * 100, 128, 50, 4, 8, 2, 128, 0.0, FAKE, 0, None, 0, None) == EINVAL
    assert L.ts_draft_attn(FAKE, FAKE, FAKE, 128 * 100, 128, 50_000, 4, 8, 2, 128, 0.0, FAKE, 0, None, 0, None) == EWORKSPACE


def _select(L, **kw):
    a = dict(q=FAKE, T=4, k=FAKE, v=FAKE, s_head=128 * 1000, s_pos=128, n_ctx=1000, Hq=8, Hkv=2, d=128, n_sink=4,
             budget=100, n_recent=8, sel=FAKE, kp=FAKE, vp=FAKE, sp_head=128 * 112, sp_pos=128, ws=None, ws_bytes=0)
    a.update(kw)
    n_part = ctypes.c_int32(-7)
    rc = L.ts_partial_kv_select(a["q"], a["T"], a["k"], a["v"], a["s_head"], a["s_pos"], a["n_ctx"], a["Hq"], a["Hkv"],
                                a["d"], a["n_sink"], a["budget"], a["n_recent"], a["sel"], a["kp"], a["vp"],
                                a["sp_head"], a["sp_pos"], ctypes.byref(n_part), None, a["ws"], a["ws_bytes"], None)
    return rc, n_part.value


@pytest.mark.parametrize("kw,code", [
    (dict(sel=None), EINVAL), (dict(budget=-1), EINVAL), (dict(n_sink=-1), EINVAL), (dict(d=80), ENOTSUP),
    (dict(T=130), ENOTSUP), (dict(Hq=7), EINVAL), (dict(sp_head=128 * 50), EINVAL), (dict(kp=FAKE_ODD), EINVAL),
    (dict(), EWORKSPACE),
])
def test_partial_kv_select_rejects(kw, code):
    L = _lib()
    rc, n_part = _select(L, **kw)
    assert rc == code
    assert n_part == -7  # nothing written on error


def _select_scored(L, **kw):
    a = dict(scores=FAKE, k=FAKE, v=FAKE, s_head=128 * 1000, s_pos=128, n_ctx=1000, Hkv=2, d=128, n_sink=4,
             budget=100, n_recent=8, sel=FAKE, kp=FAKE, vp=FAKE, sp_head=128 * 112, sp_pos=128, ws=None, ws_bytes=0)
    a.update(kw)
    n_part = ctypes.c_int32(-7)
    rc = L.ts_partial_kv_select_scored(a["scores"], a["k"], a["v"], a["s_head"], a["s_pos"], a["n_ctx"], a["Hkv"],
                                       a["d"], a["n_sink"], a["budget"], a["n_recent"], a["sel"], a["kp"], a["vp"],
                                       a["sp_head"], a["sp_pos"], ctypes.byref(n_part), a["ws"], a["ws_bytes"], None)
    return rc, n_part.value


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), EINVAL), (dict(scores=FAKE_ODD), EINVAL), (dict(sel=None), EINVAL), (dict(budget=-1), EINVAL),
    (dict(Hkv=0), EINVAL), (dict(d=80), ENOTSUP), (dict(sp_head=128 * 50), EINVAL), (dict(kp=FAKE_ODD), EINVAL),
    (dict(), EWORKSPACE),
])
def test_partial_kv_select_scored_rejects(kw, code):
    L = _lib()
    rc, n_part = _select_scored(L, **kw)
    assert rc == code
    assert n_part == -7


def test_scored_selection_needs_less_workspace():
    L = _lib()
    full = L.ts_partial_kv_select_workspace_size(100_000, 24, 32, 8, 128, 4096)
    passes = L.ts_partial_kv_select_scored_workspace_size(100_000, 8, 128, 4096)
    # no score copy and no query sum: the full query at least adds the scores
    assert 0 < passes and passes + 8 * 100_000 * 4 <= full
    assert L.ts_partial_kv_select_scored_workspace_size(100_000, 0, 128, 4096) == 0


def _penalty(L, **kw):
    a = dict(logits=FAKE, rows=2, V=1000, window=FAKE, W=16, wstride=16, penalty=1.2, temp=1.0, top_p=0.9,
             min_p=0.05, out=FAKE, keep=FAKE, probs=FAKE, u=FAKE, token=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return L.ts_penalty_sample(a["logits"], a["rows"], a["V"], a["window"], a["W"], a["wstride"], a["penalty"],
                               a["temp"], a["top_p"], a["min_p"], a["out"], a["keep"], a["probs"], a["u"], a["token"],
                               a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), EINVAL), (dict(rows=0), EINVAL), (dict(V=0), EINVAL), (dict(V=300_000), ENOTSUP),
    (dict(W=-1), EINVAL), (dict(window=None), EINVAL), (dict(wstride=8), EINVAL), (dict(penalty=0.0), EINVAL),
    (dict(penalty=-1.2), EINVAL), (dict(temp=0.0), EINVAL), (dict(top_p=1.5), EINVAL), (dict(top_p=-0.1), EINVAL),
    (dict(min_p=float("nan")), EINVAL), (dict(u=None), EINVAL), (dict(out=FAKE_ODD), EINVAL),
    (dict(ws_bytes=1024), EWORKSPACE), (dict(ws=None), EINVAL), (dict(ws=FAKE_ODD), EINVAL),
])
def test_penalty_sample_rejects(kw, code):
    L = _lib()
    assert _penalty(L, **kw) == code


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "HERE", str(tmp_path))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def test_tree_accept_rejects():
    L = _lib()
    par = (ctypes.c_int32 * 3)(-1, 0, 1)
    assert L.ts_tree_accept(par, 3, FAKE, FAKE, None, None) == EINVAL
    assert L.ts_tree_accept(par, 0, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.ts_tree_accept(par, 129, FAKE, FAKE, FAKE, None) == ENOTSUP
    assert L.ts_tree_accept(par, 3, FAKE_ODD, FAKE, FAKE, None) == EINVAL
    bad = (ctypes.c_int32 * 3)(-1, 0, 2)
    assert L.ts_tree_accept(bad, 3, FAKE, FAKE, FAKE, None) == EINVAL
    assert "parent[2]" in L.ts_last_error().decode()


def _commit(L, **kw):
    a = dict(result=FAKE, T=24, k=FAKE, v=FAKE, s_layer=8 * 128 * 200, s_head=128 * 200, s_pos=128, layers=4, Hkv=8,
             d=128, n_ctx=100, kp=FAKE, vp=FAKE, sp_layer=8 * 128 * 64, sp_head=128 * 64, sp_pos=128, n_part=40,
             part_rows=64)
    a.update(kw)
    return L.ts_kv_commit(a["result"], a["T"], a["k"], a["v"], a["s_layer"], a["s_head"], a["s_pos"], a["layers"],
                          a["Hkv"], a["d"], a["n_ctx"], a["kp"], a["vp"], a["sp_layer"], a["sp_head"], a["sp_pos"],
                          a["n_part"], a["part_rows"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(result=None), EINVAL), (dict(T=0), EINVAL), (dict(T=129), ENOTSUP), (dict(d=96), ENOTSUP),
    (dict(layers=0), EINVAL), (dict(s_pos=64), EINVAL), (dict(s_layer=0), EINVAL), (dict(k=FAKE_ODD), EINVAL),
    (dict(vp=None), EINVAL), (dict(n_part=41), EINVAL), (dict(sp_head=0), EINVAL), (dict(n_ctx=-1), EINVAL),
])
def test_kv_commit_rejects(kw, code):
    L = _lib()
    assert _commit(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(window=None), EINVAL), (dict(W=0), EINVAL), (dict(W=4097), ENOTSUP), (dict(k=-1), EINVAL),
    (dict(levels=4), EINVAL), (dict(head=None), EINVAL), (dict(T_max=0), EINVAL), (dict(T_max=129), EINVAL),
    (dict(info=FAKE_ODD), EINVAL),
])
def test_ngram_tree_rejects(kw, code):
    L = _lib()
    a = dict(window=FAKE, W=1024, k=20, seed=7, head=FAKE, levels=3, T_max=24, parent=FAKE, tok=FAKE, info=FAKE)
    a.update(kw)
    assert L.ts_ngram_tree(a["window"], a["W"], a["k"], a["seed"], a["head"], a["levels"], a["T_max"], a["parent"],
                           a["tok"], a["info"], None) == code


@pytest.mark.parametrize("eps,alpha,code", [(0.0, 0.1, EINVAL), (1.5, 0.1, EINVAL), (float("nan"), 0.1, EINVAL),
                                            (0.1, -1.0, EINVAL), (0.1, float("inf"), EINVAL)])
def test_penalty_sample_eta_rejects(eps, alpha, code):
    L = _lib()
    rc = L.ts_penalty_sample_eta(FAKE, 2, 1000, FAKE, 16, 16, 1.2, 1.0, eps, alpha, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 40, None)
    assert rc == code
    # the shared checks still run (V beyond the supported size)
    assert L.ts_penalty_sample_eta(FAKE, 2, 300_000, FAKE, 16, 16, 1.2, 1.0, 0.1, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, 1 << 40, None) == ENOTSUP


def test_binding_checks_tensors_before_any_launch():
    """Host tensors, wrong dtypes and non-contiguous buffers are refused by
    the binding itself (a host pointer handed to a kernel would fault)."""
    import torch

    q = torch.zeros((8, 4, 64), dtype=torch.bfloat16)
    k = torch.zeros((2, 100, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        binding.verify_attn(q, k, k, 96, [-1, 0, 1, 2])
    with pytest.raises(TypeError, match="q must be"):
        binding.verify_attn(q.float(), k, k, 96, [-1, 0, 1, 2])
    with pytest.raises(ValueError, match="contiguous"):
        binding.draft_attn(q.transpose(0, 1), k, k, 96)
    logits = torch.zeros((4, 1024), dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        binding.penalty_sample(logits.t(), None, 1.2, 1.0, 0.9, 0.05)
    with pytest.raises(ValueError, match="shape"):
        binding.penalty_sample(logits, None, 1.2, 1.0, 0.9, 0.05, out=torch.zeros((4, 1000)))


def test_partial_rows_query():
    L = _lib()
    assert L.ts_partial_kv_rows(100_000, 4, 4096, 64) == 4 + 4096 + 64
    assert L.ts_partial_kv_rows(1000, 4, 5000, 8) == 1000       # budget past the candidates: every row
    assert L.ts_partial_kv_rows(70, 4, 16, 64) == 70            # fewer candidates than the budget
    assert L.ts_partial_kv_rows(3, 4, 16, 8) == 3               # shorter than the sink
    assert L.ts_partial_kv_rows(0, 4, 16, 8) == 0
    assert L.ts_partial_kv_rows(-1, 4, 16, 8) == -1
    assert binding.partial_rows(5000, 4, 1, 64) == 69


def _cpu_bf16(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_checks_extents_before_any_launch():
    """Every tensor's extent is checked against the scalars passed with it
    (the library sees only pointers: a short tensor would be read or written
    past its end). CPU tensors: the check fires before any pointer is taken."""
    import torch

    _lib()
    q = _cpu_bf16(8, 4, 64)
    k = _cpu_bf16(2, 100, 64)
    # verification: n_ctx + T rows, matching channels, one parent per node
    with pytest.raises(ValueError, match="the call needs 100"):
        binding.verify_attn(q, k[:, :99], k[:, :99], 96, [-1, 0, 1, 2])
    with pytest.raises(ValueError, match="channels"):
        binding.verify_attn(q, _cpu_bf16(2, 100, 128), _cpu_bf16(2, 100, 128), 96, [-1, 0, 1, 2])
    with pytest.raises(ValueError, match="parent has 3 entries"):
        binding.verify_attn(q, k, k, 96, [-1, 0, 1])
    with pytest.raises(ValueError, match="equal shapes"):
        binding.verify_attn(q, k, _cpu_bf16(2, 99, 64), 96, [-1, 0, 1, 2])
    with pytest.raises(ValueError, match="the call needs 100"):
        binding.verify_attn_scored(q, k[:, :99], k[:, :99], 96, [-1, 0, 1, 2])
    with pytest.raises(ValueError, match="scores must be float32"):
        binding.verify_attn_scored(q, k, k, 96, [-1, 0, 1, 2], scores=torch.zeros((2, 95)))
    # drafting: n_part + Tq rows of the partial cache
    with pytest.raises(ValueError, match="the call needs 101"):
        binding.draft_attn(q, k, k, 97)
    # selection: n_ctx rows of the full cache, n_part rows of the partial cache, the scores buffer
    kp = _cpu_bf16(2, 4 + 16 + 8, 64)
    with pytest.raises(ValueError, match="the call needs 101"):
        binding.partial_kv_select(q, k, k, 101, 4, 16, 8)
    with pytest.raises(ValueError, match="the call needs 28"):
        binding.partial_kv_select(q, k, k, 100, 4, 16, 8, k_part=kp[:, :27], v_part=kp[:, :27])
    with pytest.raises(ValueError, match="heads"):
        binding.partial_kv_select(q, k, k, 100, 4, 16, 8, k_part=_cpu_bf16(1, 28, 64), v_part=_cpu_bf16(1, 28, 64))
    with pytest.raises(ValueError, match="scores must be float32"):
        binding.partial_kv_select(q, k, k, 100, 4, 16, 8, want_scores=True, scores=torch.zeros((2, 99)))
    with pytest.raises(ValueError, match="scores must be float32"):
        binding.partial_kv_select(q, k, k, 100, 4, 16, 8, want_scores=True,
                                  scores=torch.zeros((2, 100), dtype=torch.float16))
    with pytest.raises(ValueError, match="row stride"):
        binding.partial_kv_select(q, k, k, 100, 4, 16, 8, want_scores=True, scores=torch.zeros((100, 2)).t())
    with pytest.raises(ValueError, match="the call needs 28"):
        binding.partial_kv_select_scored(torch.zeros((2, 100)), k, k, 100, 4, 16, 8, k_part=kp[:, :27],
                                         v_part=kp[:, :27])
    with pytest.raises(ValueError, match="scores must be float32"):
        binding.partial_kv_select_scored(torch.zeros((3, 100)), k, k, 100, 4, 16, 8)
    # acceptance and commit: result of T + 2 entries, the tree rows inside the caches
    tok = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="result must be"):
        binding.tree_accept([-1, 0, 1, 2], tok, tok, result=torch.zeros(5, dtype=torch.int32))
    with pytest.raises(ValueError, match="result must be"):
        binding.kv_commit(torch.zeros(5, dtype=torch.int32), 4, k, k, 96)
    with pytest.raises(ValueError, match="tree rows end at 101"):
        binding.kv_commit(torch.zeros(6, dtype=torch.int32), 4, k, k, 97)
    with pytest.raises(ValueError, match="heads and channels"):
        binding.kv_commit(torch.zeros(6, dtype=torch.int32), 4, k, k, 96, _cpu_bf16(3, 40, 64),
                          _cpu_bf16(3, 40, 64), 10)
    with pytest.raises(ValueError, match="both k_part and v_part"):
        binding.kv_commit(torch.zeros(6, dtype=torch.int32), 4, k, k, 96, _cpu_bf16(2, 40, 64), None, 10)
    # n-gram tree outputs: T_max entries (info: 4)
    win = torch.zeros(64, dtype=torch.int32)
    with pytest.raises(ValueError, match="parent must be"):
        binding.ngram_tree(win, 20, 1, T_max=24, parent=torch.zeros(23, dtype=torch.int32))
    with pytest.raises(ValueError, match="node_token must be"):
        binding.ngram_tree(win, 20, 1, T_max=24, node_token=torch.zeros(24, dtype=torch.int64))
    with pytest.raises(ValueError, match="info must be"):
        binding.ngram_tree(win, 20, 1, T_max=24, info=torch.zeros(3, dtype=torch.int32))


def test_verify_attn_noalloc_rejects_before_any_launch():
    L = _lib()
    assert L.ts_verify_attn_noalloc_max_scratch() == 32 << 20
    par = (ctypes.c_int32 * 3)(-1, 0, 1)
    # 782 forced splits of a 100K-row cache need 158 MB of partials: beyond the scratch
    par24 = (ctypes.c_int32 * 24)(-1, *range(23))
    rc = L.ts_verify_attn_noalloc(FAKE, FAKE, FAKE, 128 * 200_000, 128, 100_000, 24, par24, 32, 8, 128, 0.0, FAKE,
                                  10_000, None)
    assert rc == EWORKSPACE and "scratch" in L.ts_last_error().decode()
    assert L.ts_verify_attn_noalloc(FAKE, FAKE, FAKE, 128 * 200, 128, 100, 3, par, 8, 2, 96, 0.0, FAKE, 0,
                                    None) == ENOTSUP
    bad = (ctypes.c_int32 * 3)(-1, 0, 2)
    assert L.ts_verify_attn_noalloc(FAKE, FAKE, FAKE, 128 * 200, 128, 100, 3, bad, 8, 2, 128, 0.0, FAKE, 1,
                                    None) == EINVAL
