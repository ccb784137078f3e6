"""Helpers for the GPU parity tests (moving seeded inputs to the device, error metrics)."""

import numpy as np
import torch


def dev_bf16(bits):
    """uint16 bfloat16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def rel_max_err(got, ref):
    """max |got - ref| / max |ref| (the attention parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
