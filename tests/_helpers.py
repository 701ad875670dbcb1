"""Shared helpers for the parity tests: tolerances and oracle/device plumbing.

Tolerances (the pages give none; the workload definitions do):
  fp32: per-row normwise relative error  max_i ||Y_i - Y*_i||_inf / ||Y*_i||_inf <= 1e-5
        (elementwise relative error is not attainable by any fp32 evaluation:
        some outputs are ~1e-5 in magnitude while their row is O(1)).
  bf16: elementwise absolute error max |Y - Y*| <= 2e-2, Y upcast to fp64.
"""
from __future__ import annotations

import numpy as np
import torch

F32_ROW_RTOL = 1e-5
BF16_ATOL = 2e-2


def row_normwise_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||y - ref||_inf / ||ref||_inf (rows = last axis)."""
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)
    return float(np.max(num / den))


def max_abs_err(y: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(y - ref)))


def assert_parity(y: np.ndarray, ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if dtype == torch.float32:
        err = row_normwise_err(y, ref)
        assert err <= F32_ROW_RTOL, f"{what}: fp32 row-normwise error {err:.3e} > {F32_ROW_RTOL}"
    else:
        err = max_abs_err(y, ref)
        assert err <= BF16_ATOL, f"{what}: bf16 max abs error {err:.3e} > {BF16_ATOL}"
    return err


def to_dev(*ts, device="cuda"):
    return [t.to(device).contiguous() for t in ts]


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
