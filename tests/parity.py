"""Parity metrics and small drivers shared by the GPU tests.

Tolerances (fp32 state, bf16 q/k/v, fp64 oracle fed the same bf16/fp32 values):

* fp32 tensors (states, checkpoints): ``rel(x, r) = max|x - r| / max|r| <= 2e-3``.
* bf16 outputs o: storing a value in bf16 alone moves it by up to half an ulp (relative
  2^-8 near a power of two), which on its own can exceed 2e-3 of max|r|. So o is scored on
  the error beyond that mandatory rounding:
  ``rel_bf16(x, r) = max(max(0, |x - r| - ulp_bf16(r) / 2)) / max|r| <= 2e-3``;
  a kernel whose fp32 result is exact scores 0.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = 2e-3


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel(x, r) -> float:
    x, r = f64(x), f64(r)
    den = np.max(np.abs(r)) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - r)) / den)


def half_ulp_bf16(r: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(r))            # |r| = m 2^e, m in [0.5, 1): ulp_bf16 = 2^(e-8)
    h = np.ldexp(1.0, e - 9)
    return np.where(r == 0, 0.0, h)


def rel_bf16(x, r) -> float:
    x, r = f64(x), f64(r)
    den = np.max(np.abs(r)) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    excess = np.maximum(0.0, np.abs(x - r) - half_ulp_bf16(r))
    return float(np.max(excess) / den)


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def meta_equal(gpu_meta: np.ndarray, oracle_meta: np.ndarray, slots) -> None:
    slots = list(slots)
    np.testing.assert_array_equal(gpu_meta[slots], oracle_meta[slots])
