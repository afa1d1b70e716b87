"""Comparison rules for GPU results against the fp64 oracle.

Floating-point outputs: per element e, err_e = |gpu_e - ref_e| / scale_e with
scale_e = sum_i a_i |V_i[d]| the condition scale of the convex combination
(>= |ref_e|); where scale_e == 0 the GPU value must be exactly 0. The bar is
max err <= 1e-5 for fp32 outputs and <= 1e-2 for bf16 outputs. Statistics
(m, lse) pass when |gpu - ref| <= 1e-5 (1 + |ref|). Integer and bit-level
results (block sums, the plan, single-source aggregates) must be identical.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 1e-2}
STATS_TOL = 1e-5


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy: bf16 as uint16 bit patterns, fp32 as float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def scaled_error(gpu: np.ndarray, ref: np.ndarray, scale: np.ndarray) -> float:
    g = widen(gpu)
    diff = np.abs(g - ref)
    zero = scale == 0
    if np.any(zero) and np.any(g[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(zero, 0.0, diff / np.where(zero, 1.0, scale))
    return float(err.max()) if err.size else 0.0


def assert_close_scaled(gpu: np.ndarray, ref: np.ndarray, scale: np.ndarray, dtype: str, what=""):
    err = scaled_error(gpu, ref, scale)
    assert err <= TOL[dtype], f"{what}: max scaled error {err:.3e} > {TOL[dtype]:.0e} ({dtype})"
    return err


def assert_stats(gpu: np.ndarray, ref: np.ndarray, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    bad = np.abs(g - ref) > STATS_TOL * (1.0 + np.abs(ref))
    assert not bad.any(), (f"{what}: {bad.sum()} stats outside 1e-5(1+|ref|); "
                           f"worst |d| = {np.abs(g - ref).max():.3e}")


def sample_rows(R: int, count: int, seed: int = 0) -> np.ndarray:
    """Row 0, row R-1 and count-2 further distinct rows drawn with ``seed``."""
    if count >= R:
        return np.arange(R, dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, R - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, R - 1], mid])).astype(np.int64)
