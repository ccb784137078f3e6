"""MI355X (gfx950) hot path of TokenSwift-style ultra-long generation.

A thin ctypes binding over the C ABI of ``libtokenswift.so`` (declared in
``include/tokenswift.h``): it marshals torch tensors (device memory and the
current stream) into pointers and sizes. Every step of the computation runs in
the library's HIP kernels; nothing here computes, and there is no fallback: if
the library is missing, every call raises.
"""

from .binding import (
    TSError,
    draft_attn,
    kv_commit,
    lib,
    lib_path,
    ngram_tree,
    partial_kv_select,
    partial_kv_select_scored,
    penalty_sample,
    penalty_sample_eta,
    tree_accept,
    verify_attn,
    verify_attn_noalloc,
    verify_attn_scored,
)

__all__ = [
    "TSError",
    "lib",
    "lib_path",
    "verify_attn",
    "verify_attn_noalloc",
    "verify_attn_scored",
    "draft_attn",
    "partial_kv_select",
    "partial_kv_select_scored",
    "penalty_sample",
    "penalty_sample_eta",
    "tree_accept",
    "kv_commit",
    "ngram_tree",
]
