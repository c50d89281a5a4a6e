"""Parity helpers shared by the GPU tests and the benchmark's sampled checks.

Criteria (fixed once here):
  fp32 inputs:  max |x - ref| <= 1e-4 on o and on the final state;
  bf16 inputs:  max |x - ref| / rms(ref) <= 2e-2 on o and on the final state
                (o is produced in fp32; the state is always fp32).
"""
from __future__ import annotations

import numpy as np
import torch

TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def max_abs(a, ref):
    a, ref = to_np(a), to_np(ref)
    return float(np.max(np.abs(a - ref))) if ref.size else 0.0


def rel_rms(a, ref):
    a, ref = to_np(a), to_np(ref)
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(a - ref))) / max(rms, 1e-30)


def assert_parity(a, ref, in_dtype, what=""):
    if in_dtype == torch.float32:
        e = max_abs(a, ref)
        assert e <= TOL_F32_ABS, f"{what}: max-abs {e:.3e} > {TOL_F32_ABS}"
    else:
        e = rel_rms(a, ref)
        assert e <= TOL_BF16_REL, f"{what}: max|d|/rms {e:.3e} > {TOL_BF16_REL}"
    return e
