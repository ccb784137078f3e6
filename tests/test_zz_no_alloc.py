"""GPU check of ts_verify_attn_noalloc (no workspace argument: the split
partials live in the library's per-device scratch array) against
ts_verify_attn with a workspace: bitwise equal outputs on two calls in a row,
the second smaller than the first (the scratch keeps the first call's
contents), and the oracle's bar on both."""

import numpy as np
import pytest
import torch

import long_kv_attention_amd as ts
from long_kv_attention_amd.binding import TSError
from oracle import bf16_to_f64, verify_attention
from synth import attention_inputs, tree_parent
from tests.gpu_util import banner, dev_bf16, rel_max_err

pytestmark = pytest.mark.gpu


def _case(seed, Hq, Hkv, d, n_ctx, T, heads):
    x = attention_inputs(seed, Hq, Hkv, d, n_ctx, T)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    parent = tree_parent("tokenswift" if T > 4 else "chain", T)
    out = torch.full((Hq, T, d), float("nan"), dtype=torch.float32, device="cuda:0")
    ts.verify_attn_noalloc(q, k, v, n_ctx, parent, out)
    ref = ts.verify_attn(q, k, v, n_ctx, parent)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    G = Hq // Hkv
    got = out.cpu().numpy()
    for g in heads:
        o = verify_attention(bf16_to_f64(x["q"][g * G:(g + 1) * G]), bf16_to_f64(x["k"][g:g + 1]),
                             bf16_to_f64(x["v"][g:g + 1]), n_ctx, parent)
        assert rel_max_err(got[g * G:(g + 1) * G], o) <= 2e-3


def test_two_calls_second_smaller():
    banner("noalloc verify: 8B-class 100K rows, then 12q/2kv 20K rows")
    _case(71, 32, 8, 128, 100_000, 24, heads=[0, 7])     # 6.2 MiB of split partials
    _case(72, 12, 2, 128, 20_000, 8, heads=[1])          # smaller: different grid and partial layout


def test_single_split_needs_no_scratch():
    banner("noalloc verify: one split")
    _case(73, 8, 2, 64, 300, 4, heads=[0, 1])


def test_beyond_the_scratch_is_refused():
    x = attention_inputs(74, 32, 8, 128, 100_000, 24)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out = torch.empty((32, 24, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(TSError, match="TS_EWORKSPACE"):   # 782 splits of partials: 158 MB
        ts.verify_attn_noalloc(q, k, v, 100_000, tree_parent("tokenswift", 24), out, n_split=10_000)
