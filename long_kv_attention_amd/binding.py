"""ctypes binding of libtokenswift.so (argument marshalling only).

Tensors are torch tensors on the GPU; bf16 tensors are handed to the library
as their raw 16-bit patterns. Outputs and workspaces are allocated here with
torch (device memory plumbing) unless the caller passes them in.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libtokenswift.so"
TS_OK = 0
CODES = {-1: "TS_EINVAL", -2: "TS_ENOTSUP", -3: "TS_EWORKSPACE", -4: "TS_EHIP"}

_lib = None

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)

_SIGNATURES = {
    "ts_verify_attn": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32p, c_i32, c_i32, c_i32,
                               c_f32, c_vp, c_i32, c_vp, c_sz, c_vp]),
    "ts_verify_attn_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "ts_verify_attn_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32p, c_i32, c_i32, c_i32,
                                       c_f32, c_vp, c_i32, c_vp]),
    "ts_verify_attn_noalloc_max_scratch": (c_sz, []),
    "ts_verify_attn_scored": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32p, c_i32, c_i32, c_i32,
                                      c_f32, c_vp, c_vp, c_i32, c_vp, c_sz, c_vp]),
    "ts_draft_attn": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp,
                              c_i32, c_vp, c_sz, c_vp]),
    "ts_draft_attn_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "ts_partial_kv_select": (c_i32, [c_vp, c_i32, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                                     c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32p, c_vp, c_vp, c_sz,
                                     c_vp]),
    "ts_partial_kv_select_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "ts_partial_kv_rows": (c_i32, [c_i32, c_i32, c_i32, c_i32]),
    "ts_partial_kv_select_scored": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                                            c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32p, c_vp, c_sz, c_vp]),
    "ts_partial_kv_select_scored_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
    "ts_penalty_sample": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_i32, c_i64, c_f32, c_f32, c_f32, c_f32, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ts_penalty_sample_workspace_size": (c_sz, [c_i32, c_i32]),
    "ts_penalty_sample_eta": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_i32, c_i64, c_f32, c_f32, c_f32, c_f32, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ts_tree_accept": (c_i32, [c_i32p, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "ts_kv_commit": (c_i32, [c_vp, c_i32, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                             c_i64, c_i64, c_i64, c_i32, c_i32, c_vp]),
    "ts_ngram_tree": (c_i32, [c_vp, c_i32, c_i32, ctypes.c_uint64, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "ts_last_error": (ctypes.c_char_p, []),
    "ts_abi_version": (c_i32, []),
}


class TSError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {code} ({CODES.get(code, '?')}): {msg}")
        self.code = code


def lib_path():
    return os.path.join(HERE, LIB_NAME)


def lib():
    """Load libtokenswift.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m long_kv_attention_amd.build` "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != TS_OK:
        raise TSError(fn, rc, lib().ts_last_error().decode())


def _ptr(t):
    if t is None:
        return ctypes.c_void_p(0)
    if t.device.type != "cuda":   # a host pointer handed to a kernel would fault the GPU
        raise ValueError("tensors handed to the library must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _dense(t, dtype, name, shape=None):
    """t itself if it has the dtype, is contiguous and (when given) has the shape."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _out(out, shape, device, name="out"):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    return _dense(out, torch.float32, name, shape)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _cache_strides(k, v, rows=None, d=None, Hkv=None, name="k/v"):
    """Strides of a [Hkv][rows][d] cache pair, after checking that the tensors
    hold what the call will touch: at least ``rows`` rows per head, ``d``
    channels and ``Hkv`` heads (the library sees only pointers, so a short
    tensor would be read or written past its end)."""
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError(f"{name} caches must be bfloat16")
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError(f"{name} caches must be [Hkv][rows][d] of equal shapes, with contiguous channels and "
                         "equal strides")
    if Hkv is not None and k.shape[0] != Hkv:
        raise ValueError(f"{name} caches have {k.shape[0]} heads, expected {Hkv}")
    if d is not None and k.shape[2] != d:
        raise ValueError(f"{name} caches have {k.shape[2]} channels, the queries {d}")
    if rows is not None and k.shape[1] < rows:
        raise ValueError(f"{name} caches hold {k.shape[1]} rows per head, the call needs {rows}")
    return k.stride(0), k.stride(1)


def _parent_array(parent, T):
    if len(parent) != T:
        raise ValueError(f"parent has {len(parent)} entries for {T} tree nodes")
    return (ctypes.c_int32 * T)(*[int(x) for x in parent])


def _int_buffer(t, n, name):
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous int32 buffer of at least {n} entries")
    return t


def partial_rows(n_ctx, n_sink, budget, n_recent):
    """Rows of the partial cache a selection writes (ts_partial_kv_rows)."""
    n = lib().ts_partial_kv_rows(n_ctx, n_sink, budget, n_recent)
    if n < 0:
        raise ValueError("n_ctx, n_sink, budget and n_recent must be >= 0")
    return n


def _workspace(nbytes, device, ws, zeroed=False):
    """The caller's workspace (checked for size) or a new one (zero-filled when
    the call runs faster on a zero workspace: the selection's)."""
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes, need {nbytes}")
        return ws
    return (torch.zeros if zeroed else torch.empty)(nbytes, dtype=torch.uint8, device=device)


def verify_attn(q, k, v, n_ctx, parent, scale=0.0, n_split=0, out=None, ws=None, stream=None):
    """Tree verification attention (ts_verify_attn). q [Hq][T][d] bf16; k, v [Hkv][rows][d] bf16."""
    Hq, T, d = _dense(q, torch.bfloat16, "q").shape
    Hkv = k.shape[0]
    s_head, s_pos = _cache_strides(k, v, rows=n_ctx + T, d=d)
    par = _parent_array(parent, T)
    out = _out(out, (Hq, T, d), q.device)
    L = lib()
    need = L.ts_verify_attn_workspace_size(n_ctx, T, Hq, Hkv, d, n_split)
    wst = _workspace(need, q.device, ws)
    rc = L.ts_verify_attn(_ptr(q), _ptr(k), _ptr(v), s_head, s_pos, n_ctx, T, par, Hq, Hkv, d, float(scale),
                          _ptr(out), n_split, _ptr(wst), need, _stream(stream))
    _check("ts_verify_attn", rc)
    return out


def verify_attn_noalloc(q, k, v, n_ctx, parent, out, scale=0.0, n_split=0, stream=None):
    """Tree verification attention with the library's own scratch
    (ts_verify_attn_noalloc): no workspace, and ``out`` must be given, so the
    call allocates nothing."""
    Hq, T, d = _dense(q, torch.bfloat16, "q").shape
    Hkv = k.shape[0]
    s_head, s_pos = _cache_strides(k, v, rows=n_ctx + T, d=d)
    par = _parent_array(parent, T)
    _dense(out, torch.float32, "out", (Hq, T, d))
    rc = lib().ts_verify_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), s_head, s_pos, n_ctx, T, par, Hq, Hkv, d,
                                      float(scale), _ptr(out), n_split, _stream(stream))
    _check("ts_verify_attn_noalloc", rc)
    return out


def _score_buffer(scores, Hkv, n_ctx, device):
    if scores is None:
        return torch.empty((Hkv, max(n_ctx, 1)), dtype=torch.float32, device=device)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != Hkv or scores.shape[1] < n_ctx:
        raise ValueError(f"scores must be float32 [{Hkv}][{n_ctx}]")
    if n_ctx > 0 and (scores.stride(1) != 1 or (Hkv > 1 and scores.stride(0) != n_ctx)):
        raise ValueError("scores must be contiguous with row stride n_ctx")
    return scores


def verify_attn_scored(q, k, v, n_ctx, parent, scale=0.0, n_split=0, out=None, scores=None, ws=None, stream=None):
    """Verification attention plus the grouped key scores (ts_verify_attn_scored).

    Returns (out [Hq][T][d] fp32, scores [Hkv][n_ctx] fp32).
    """
    Hq, T, d = _dense(q, torch.bfloat16, "q").shape
    Hkv = k.shape[0]
    s_head, s_pos = _cache_strides(k, v, rows=n_ctx + T, d=d)
    par = _parent_array(parent, T)
    out = _out(out, (Hq, T, d), q.device)
    scores = _score_buffer(scores, Hkv, n_ctx, q.device)
    L = lib()
    need = L.ts_verify_attn_workspace_size(n_ctx, T, Hq, Hkv, d, n_split)
    wst = _workspace(need, q.device, ws)
    rc = L.ts_verify_attn_scored(_ptr(q), _ptr(k), _ptr(v), s_head, s_pos, n_ctx, T, par, Hq, Hkv, d, float(scale),
                                 _ptr(out), _ptr(scores), n_split, _ptr(wst), need, _stream(stream))
    _check("ts_verify_attn_scored", rc)
    return out, scores


def draft_attn(q, k_part, v_part, n_part, scale=0.0, n_split=0, out=None, ws=None, stream=None):
    """Draft attention over the partial cache (ts_draft_attn)."""
    Hq, Tq, d = _dense(q, torch.bfloat16, "q").shape
    Hkv = k_part.shape[0]
    s_head, s_pos = _cache_strides(k_part, v_part, rows=n_part + Tq, d=d, name="partial")
    out = _out(out, (Hq, Tq, d), q.device)
    L = lib()
    need = L.ts_draft_attn_workspace_size(n_part, Tq, Hq, Hkv, d, n_split)
    wst = _workspace(need, q.device, ws)
    rc = L.ts_draft_attn(_ptr(q), _ptr(k_part), _ptr(v_part), s_head, s_pos, n_part, Tq, Hq, Hkv, d,
                         float(scale), _ptr(out), n_split, _ptr(wst), need, _stream(stream))
    _check("ts_draft_attn", rc)
    return out


def partial_kv_select(q, k, v, n_ctx, n_sink, budget, n_recent, k_part=None, v_part=None, want_scores=False,
                      sel_idx=None, scores=None, extra_rows=0, ws=None, stream=None):
    """Score, select and gather the partial cache (ts_partial_kv_select).

    Freshly allocated partial caches hold n_sink + budget + n_recent rows plus
    ``extra_rows`` (room for the draft tokens' own keys/values).
    Returns (sel_idx [Hkv][budget] int32, k_part, v_part, n_part, scores or None).
    """
    Hq, T, d = _dense(q, torch.bfloat16, "q").shape
    Hkv = k.shape[0]
    s_head, s_pos = _cache_strides(k, v, rows=n_ctx, d=d)
    dev = q.device
    n_part_need = partial_rows(n_ctx, n_sink, budget, n_recent)
    if k_part is None:
        k_part = torch.empty((Hkv, max(n_sink + budget + n_recent + extra_rows, 1), d), dtype=torch.bfloat16,
                             device=dev)
    if v_part is None:
        v_part = torch.empty_like(k_part)
    sp_head, sp_pos = _cache_strides(k_part, v_part, rows=n_part_need, d=d, Hkv=Hkv, name="partial")
    if sel_idx is None:
        sel_idx = torch.empty((Hkv, max(budget, 1)), dtype=torch.int32, device=dev)
    else:
        _dense(sel_idx, torch.int32, "sel_idx", (Hkv, max(budget, 1)))
    scores = _score_buffer(scores, Hkv, n_ctx, dev) if want_scores else None
    L = lib()
    need = L.ts_partial_kv_select_workspace_size(n_ctx, T, Hq, Hkv, d, budget)
    wst = _workspace(need, dev, ws, zeroed=True)
    n_part = ctypes.c_int32(-1)
    rc = L.ts_partial_kv_select(_ptr(q), T, _ptr(k), _ptr(v), s_head, s_pos, n_ctx, Hq, Hkv, d, n_sink, budget,
                                n_recent, _ptr(sel_idx), _ptr(k_part), _ptr(v_part), sp_head, sp_pos,
                                ctypes.byref(n_part), _ptr(scores if want_scores else None), _ptr(wst), need,
                                _stream(stream))
    _check("ts_partial_kv_select", rc)
    return sel_idx[:, :budget], k_part, v_part, n_part.value, (scores if want_scores else None)


def partial_kv_select_scored(scores, k, v, n_ctx, n_sink, budget, n_recent, k_part=None, v_part=None,
                             sel_idx=None, extra_rows=0, ws=None, stream=None):
    """Select and gather the partial cache from given scores (ts_partial_kv_select_scored).

    scores [Hkv][n_ctx] fp32 (e.g. from verify_attn_scored). Returns
    (sel_idx [Hkv][budget] int32, k_part, v_part, n_part).
    """
    Hkv, d = k.shape[0], k.shape[2]
    s_head, s_pos = _cache_strides(k, v, rows=n_ctx)
    dev = k.device
    if scores is None:
        raise ValueError("scores are required")
    scores = _score_buffer(scores, Hkv, n_ctx, dev)
    n_part_need = partial_rows(n_ctx, n_sink, budget, n_recent)
    if k_part is None:
        k_part = torch.empty((Hkv, max(n_sink + budget + n_recent + extra_rows, 1), d), dtype=torch.bfloat16,
                             device=dev)
    if v_part is None:
        v_part = torch.empty_like(k_part)
    sp_head, sp_pos = _cache_strides(k_part, v_part, rows=n_part_need, d=d, Hkv=Hkv, name="partial")
    if sel_idx is None:
        sel_idx = torch.empty((Hkv, max(budget, 1)), dtype=torch.int32, device=dev)
    else:
        _dense(sel_idx, torch.int32, "sel_idx", (Hkv, max(budget, 1)))
    L = lib()
    need = L.ts_partial_kv_select_scored_workspace_size(n_ctx, Hkv, d, budget)
    wst = _workspace(need, dev, ws, zeroed=True)
    n_part = ctypes.c_int32(-1)
    rc = L.ts_partial_kv_select_scored(_ptr(scores), _ptr(k), _ptr(v), s_head, s_pos, n_ctx, Hkv, d, n_sink, budget,
                                       n_recent, _ptr(sel_idx), _ptr(k_part), _ptr(v_part), sp_head, sp_pos,
                                       ctypes.byref(n_part), _ptr(wst), need, _stream(stream))
    _check("ts_partial_kv_select_scored", rc)
    return sel_idx[:, :budget], k_part, v_part, n_part.value


def _penalty_call(fn, filt, logits, window, penalty, temperature, u, want_keep, want_probs, want_token, out,
                  token_out, ws, stream):
    rows, V = _dense(logits, torch.float32, "logits").shape
    dev = logits.device
    if u is not None and (_dense(u, torch.float32, "u").numel() < rows):
        raise ValueError(f"u must hold at least {rows} entries")
    if window is None or window.numel() == 0:
        W, wstride, wptr = 0, 0, None
    elif window.dim() == 1:
        W, wstride, wptr = window.shape[0], 0, window
    else:
        if window.shape[0] != rows:
            raise ValueError("window must have one row per logits row, or be 1-D (shared)")
        W, wstride, wptr = window.shape[1], window.stride(0), window
    if wptr is not None and (wptr.dtype != torch.int32 or wptr.stride(-1) != 1):
        raise ValueError("window must be int32 with contiguous rows")
    want_token = (u is not None) if want_token is None else want_token
    z = torch.empty_like(logits) if out is None else _dense(out, torch.float32, "out", (rows, V))
    keep = torch.empty((rows, V), dtype=torch.uint8, device=dev) if want_keep else None
    probs = torch.empty((rows, V), dtype=torch.float32, device=dev) if want_probs else None
    if token_out is not None:
        if token_out.dtype != torch.int32 or token_out.numel() < rows or not token_out.is_contiguous():
            raise ValueError(f"token_out must be a contiguous int32 buffer of at least {rows} entries")
        token = token_out
    else:
        token = torch.empty(rows, dtype=torch.int32, device=dev) if want_token else None
    L = lib()
    need = L.ts_penalty_sample_workspace_size(rows, V)
    wst = _workspace(need, dev, ws)
    rc = getattr(L, fn)(_ptr(logits), rows, V, _ptr(wptr), W, wstride, float(penalty), float(temperature),
                        float(filt[0]), float(filt[1]), _ptr(z), _ptr(keep), _ptr(probs), _ptr(u), _ptr(token),
                        _ptr(wst), need, _stream(stream))
    _check(fn, rc)
    return z, keep, probs, token


def penalty_sample(logits, window, penalty, temperature, top_p, min_p, u=None, want_keep=True, want_probs=True,
                   want_token=None, out=None, token_out=None, ws=None, stream=None):
    """Contextual penalty + temperature + top-p + min-p (ts_penalty_sample).

    logits [rows][V] fp32; window [rows][W] or [W] int32 (shared). Returns
    (z, keep or None, probs or None, token or None).
    """
    return _penalty_call("ts_penalty_sample", (top_p, min_p), logits, window, penalty, temperature, u, want_keep,
                         want_probs, want_token, out, token_out, ws, stream)


def penalty_sample_eta(logits, window, penalty, temperature, epsilon, alpha, u=None, want_keep=True, want_probs=True,
                       want_token=None, out=None, token_out=None, ws=None, stream=None):
    """The same pass with eta-sampling in place of top-p and min-p (ts_penalty_sample_eta)."""
    return _penalty_call("ts_penalty_sample_eta", (epsilon, alpha), logits, window, penalty, temperature, u,
                         want_keep, want_probs, want_token, out, token_out, ws, stream)


def tree_accept(parent, node_token, target, result=None, stream=None):
    """Accepted path of a verified tree (ts_tree_accept).

    node_token, target: int32 [T] on the device. Returns result int32 [T + 2]:
    (n accepted, next token, path a_0..a_{n-1}, -1 padding).
    """
    T = len(parent)
    for name, t in (("node_token", node_token), ("target", target)):
        if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != T or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 vector of {T} tokens")
    par = _parent_array(parent, T)
    if result is None:
        result = torch.empty(T + 2, dtype=torch.int32, device=node_token.device)
    else:
        _int_buffer(result, T + 2, "result")
    rc = lib().ts_tree_accept(par, T, _ptr(node_token), _ptr(target), _ptr(result), _stream(stream))
    _check("ts_tree_accept", rc)
    return result


def _layer_strides(k, v):
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("caches must be bfloat16")
    if k.dim() == 3:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    if k.dim() != 4 or k.stride() != v.stride() or k.stride(3) != 1:
        raise ValueError("caches must be [layers][Hkv][rows][d] (or [Hkv][rows][d]) with contiguous channels "
                         "and equal strides")
    return k.shape[0], k.stride(0), k.stride(1), k.stride(2)


def kv_commit(result, T, k, v, n_ctx, k_part=None, v_part=None, n_part=0, stream=None):
    """Commit an accepted path into the caches (ts_kv_commit), in place.

    k, v: [layers][Hkv][rows][d] or [Hkv][rows][d] bf16; k_part, v_part the
    partial caches of the same form (or None), n_part rows in use.
    """
    layers, s_layer, s_head, s_pos = _layer_strides(k, v)
    Hkv, d = k.shape[-3], k.shape[-1]
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if k.shape[-2] < n_ctx + T:
        raise ValueError(f"caches hold {k.shape[-2]} rows per head, the tree rows end at {n_ctx + T}")
    _int_buffer(result, T + 2, "result")
    if (k_part is None) != (v_part is None):
        raise ValueError("give both k_part and v_part or neither")
    if k_part is not None:
        pl, sp_layer, sp_head, sp_pos = _layer_strides(k_part, v_part)
        if pl != layers:
            raise ValueError("partial caches need the same number of layers")
        if k_part.shape != v_part.shape or k_part.shape[-3] != Hkv or k_part.shape[-1] != d:
            raise ValueError("partial caches must have the full caches' heads and channels, and equal shapes")
        part_rows = k_part.shape[-2]
    else:
        sp_layer = sp_head = sp_pos = 0
        part_rows = 0
    rc = lib().ts_kv_commit(_ptr(result), T, _ptr(k), _ptr(v), s_layer, s_head, s_pos, layers, Hkv, d, n_ctx,
                            _ptr(k_part), _ptr(v_part), sp_layer, sp_head, sp_pos, n_part, part_rows,
                            _stream(stream))
    _check("ts_kv_commit", rc)


def ngram_tree(window, k, seed, head_cand=None, T_max=24, parent=None, node_token=None, info=None, stream=None):
    """N-gram retrieval, random choice and draft tree (ts_ngram_tree).

    window: int32 [W] on the device (root = last token); head_cand: int32
    [levels][3] or None. Returns device tensors (parent [T_max], node_token
    [T_max], info [4] = T, chains, distinct, occurrences).
    """
    if window.dtype != torch.int32 or window.dim() != 1 or not window.is_contiguous():
        raise ValueError("window must be a contiguous int32 vector")
    dev = window.device
    levels = 0
    if head_cand is not None:
        if head_cand.dtype != torch.int32 or head_cand.dim() != 2 or head_cand.shape[1] != 3 or \
                not head_cand.is_contiguous():
            raise ValueError("head_cand must be a contiguous int32 [levels][3] tensor")
        levels = head_cand.shape[0]
    parent = torch.empty(T_max, dtype=torch.int32, device=dev) if parent is None else \
        _int_buffer(parent, T_max, "parent")
    node_token = torch.empty(T_max, dtype=torch.int32, device=dev) if node_token is None else \
        _int_buffer(node_token, T_max, "node_token")
    info = torch.empty(4, dtype=torch.int32, device=dev) if info is None else _int_buffer(info, 4, "info")
    rc = lib().ts_ngram_tree(_ptr(window), window.shape[0], int(k), int(seed) & ((1 << 64) - 1), _ptr(head_cand),
                             levels, int(T_max), _ptr(parent), _ptr(node_token), _ptr(info), _stream(stream))
    _check("ts_ngram_tree", rc)
    return parent, node_token, info
