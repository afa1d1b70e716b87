"""Seeded synthetic inputs for tests and benchmarks -- no AttnRes arithmetic.

Two implementations of one counter-based generator (defined in gen.hip's
header comment): the HIP fill kernels of ``libattnres_inputs.so`` for large
device tensors, and the numpy twin below for small host tensors (queries,
gains, per-layer scales) and for checking the device generator.

Workload recipes mirror the five synthetic configurations of the benchmark
(single aggregate; Full stack; Block prefill; Block decode; long-context
Block); see WORKLOADS.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PKG = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(PKG, "libattnres_inputs.so")

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

# generator roles (stream identifiers)
ROLE_X, ROLE_V, ROLE_W, ROLE_GAMMA, ROLE_SCALE, ROLE_SRC, ROLE_AUX = 1, 2, 3, 4, 5, 6, 7


# ----------------------------------------------------------------------------
# numpy twin of the generator
# ----------------------------------------------------------------------------

def mix64(z: int) -> int:
    z &= M64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(0xBF58476D1CE4E5B9)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, role: int, layer: int) -> int:
    return mix64((seed * GOLDEN + mix64((role << 32) | layer)) & M64)


def _bits(key: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GOLDEN))


def normal(seed: int, role: int, layer: int, idx) -> np.ndarray:
    """Standard normals (fp64) at element indices ``idx`` (Box-Muller)."""
    b = _bits(stream_key(seed, role, layer), idx)
    u1 = ((b >> np.uint64(40)) + np.uint64(1)).astype(np.float64) * 2.0 ** -24
    u2 = ((b >> np.uint64(16)) & np.uint64(0xFFFFFF)).astype(np.float64) * 2.0 ** -24
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(6.283185307179586 * u2)


def uniform(seed: int, role: int, layer: int, idx) -> np.ndarray:
    """Uniforms in [0, 1) (fp64, 53 bits) at element indices ``idx``."""
    b = _bits(stream_key(seed, role, layer), idx)
    return (b >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of fp64 values (normal range)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    b = x.view(np.uint64)
    sign = b >> np.uint64(63)
    mag = b & np.uint64(0x7FFFFFFFFFFFFFFF)
    mag = mag + np.uint64((1 << 44) - 1) + ((mag >> np.uint64(45)) & np.uint64(1))
    e = (mag >> np.uint64(52)).astype(np.int64) - 1023 + 127
    mant = ((mag >> np.uint64(45)) & np.uint64(0x7F)).astype(np.int64)
    out = (sign.astype(np.int64) << 15) | (e << 7) | mant
    out = np.where(x == 0.0, sign.astype(np.int64) << 15, out)
    return out.astype(np.uint16)


def tensor_rows(seed: int, role: int, layer: int, rows, D: int, scale: float, dtype: str) -> np.ndarray:
    """Host copy of generated rows (global row indices ``rows``) of a [*, D] tensor:
    uint16 bf16 patterns or float32, exactly what the device fill writes."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = (rows[:, None] * D + np.arange(D, dtype=np.int64)[None, :]).astype(np.uint64)
    v = scale * normal(seed, role, layer, idx)
    return bf16_bits(v) if dtype == "bf16" else v.astype(np.float32)


def queries(seed: int, L1: int, D: int, sigma: float = 0.02) -> np.ndarray:
    """[L1, D] fp32 pseudo-queries ~ N(0, sigma^2)."""
    idx = np.arange(L1 * D, dtype=np.uint64)
    return (sigma * normal(seed, ROLE_W, 0, idx)).astype(np.float32).reshape(L1, D)


def gains(seed: int, D: int, lo: float = 0.5, hi: float = 1.5, layer: int = 0) -> np.ndarray:
    """[D] fp32 RMSNorm gains ~ U(lo, hi)."""
    return (lo + (hi - lo) * uniform(seed, ROLE_GAMMA, layer, np.arange(D))).astype(np.float32)


def layer_scales(seed: int, L: int, lo: float = 0.1, hi: float = 5.0) -> np.ndarray:
    """Per-sublayer output scales c_l ~ U(lo, hi), l = 1..L (fp64)."""
    return lo + (hi - lo) * uniform(seed, ROLE_SCALE, 0, np.arange(1, L + 1))


# ----------------------------------------------------------------------------
# workload recipes
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    kind: str                 # "aggregate" or "stack"
    B: int
    T: int
    D: int
    dtype: str                # "f32" or "bf16"
    L: int = 0
    S: int = 0
    n: int = 0
    x_sigma: float = 1.0
    v_scale: str = "uniform"  # "uniform" (c_l ~ U(0.1,5)), "const", "depth"
    v_sigma: float = 1.0
    ring: bool = False        # generate v_l per sublayer into a 3-slot ring
    src_sigmas: List[float] = field(default_factory=list)
    seed: int = 0
    description: str = ""

    @property
    def R(self) -> int:
        return self.B * self.T

    def scales(self) -> np.ndarray:
        if self.v_scale == "uniform":
            return layer_scales(self.seed, self.L)
        if self.v_scale == "depth":
            return 1.0 + np.arange(1, self.L + 1, dtype=np.float64) / 50.0
        return np.full(self.L, self.v_sigma, dtype=np.float64)


WORKLOADS = {
    "aggregate_n4": Workload(
        "aggregate_n4", "aggregate", B=2, T=64, D=256, dtype="f32", n=4,
        src_sigmas=[1.0, 3.0, 0.3, 10.0],
        description="single aggregate, n=4 sources N(0,s^2) s in {1,3,0.3,10}, fp32, "
                    "gain U(0.5,1.5), query N(0,0.02^2) and an all-zero run"),
    "full_L16": Workload(
        "full_L16", "stack", B=4, T=512, D=1024, dtype="bf16", L=16, S=1,
        description="Full AttnRes stack (S=1), 16 sublayers + embedding, bf16"),
    "full_L16_D4096": Workload(
        "full_L16_D4096", "stack", B=8, T=2048, D=4096, dtype="bf16", L=16, S=1,
        description="Full AttnRes stack at the Block config's token count and width "
                    "(16 sublayers + embedding, 17 sources of 128 MiB): the HBM-bound case "
                    "for the two-phase Full schedule"),
    "block_L48_S8": Workload(
        "block_L48_S8", "stack", B=8, T=2048, D=4096, dtype="bf16", L=48, S=8,
        description="Block AttnRes two-phase prefill, L=48, S=8 (6 blocks), bf16"),
    "decode_L96_S12": Workload(
        "decode_L96_S12", "stack", B=128, T=1, D=7168, dtype="bf16", L=96, S=12,
        x_sigma=2.0, v_scale="const", v_sigma=(4.0 / 12.0) ** 0.5,
        description="Block AttnRes decode regime, L=96, S=12, 128 rows, bf16; "
                    "x ~ N(0,4), v_l ~ N(0,4/12) so completed block sums are N(0,4)"),
    "long_L186_S24": Workload(
        "long_L186_S24", "stack", B=1, T=131072, D=7168, dtype="bf16", L=186, S=24,
        v_scale="depth", ring=True,
        description="long-context Block AttnRes, L=186, S=24 (7x24+18), 131072 rows, bf16; "
                    "v_l = (1 + l/50) N(0,1) generated per sublayer"),
}


# ----------------------------------------------------------------------------
# device side (libattnres_inputs.so)
# ----------------------------------------------------------------------------

class RingCtx(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("role", ctypes.c_uint32), ("dtype", ctypes.c_int32),
                ("R", ctypes.c_int64), ("D", ctypes.c_int64), ("L", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("scales", ctypes.c_void_p),
                ("slots", ctypes.c_void_p * 3)]


class RecorderCtx(ctypes.Structure):
    _fields_ = [("inner", ctypes.c_void_p), ("inner_ctx", ctypes.c_void_p), ("rec", ctypes.c_void_p),
                ("rows", ctypes.c_void_p), ("nrows", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("L", ctypes.c_int32), ("pad", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (binds the library to torch's HIP runtime)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build with "
                               "`python -m depth_wise_attention_rms_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.attnres_inputs_fill_normal.argtypes = [P, I, I64, I64, P, ctypes.c_uint64,
                                                 ctypes.c_uint32, ctypes.c_uint32,
                                                 ctypes.c_double, P]
        L.attnres_inputs_gather_rows.argtypes = [P, P, P, I64, I64, P]
        for f in ("attnres_inputs_fill_normal", "attnres_inputs_gather_rows"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fill_normal(dst, seed: int, role: int, layer: int, scale: float, row_ids=None, stream=None):
    """Fill device tensor ``dst`` [rows, D] (bf16 or fp32) with scale * N(0,1);
    with ``row_ids`` (device int64 [rows]) row r holds generated row row_ids[r]."""
    import torch
    D = dst.shape[-1]
    rows = dst.numel() // D
    dt = 1 if dst.dtype == torch.bfloat16 else 0
    ids = None if row_ids is None else ctypes.c_void_p(row_ids.data_ptr())
    rc = lib().attnres_inputs_fill_normal(ctypes.c_void_p(dst.data_ptr()), dt, rows, D, ids,
                                          seed, role, layer, float(scale), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"attnres_inputs_fill_normal failed ({rc})")
    return dst


def gather_rows(dst, src, row_ids, stream=None):
    rc = lib().attnres_inputs_gather_rows(ctypes.c_void_p(dst.data_ptr()),
                                          ctypes.c_void_p(src.data_ptr()),
                                          ctypes.c_void_p(row_ids.data_ptr()), row_ids.numel(),
                                          src.shape[-1] * src.element_size(), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"attnres_inputs_gather_rows failed ({rc})")
    return dst


def fn_ptr(name: str) -> int:
    return ctypes.cast(getattr(lib(), name), ctypes.c_void_p).value
