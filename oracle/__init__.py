"""Python access to the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

Arrays cross the boundary as numpy arrays: bf16 tensors as ``uint16`` bit
patterns, fp32 tensors as ``float32``, every result as ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1

GCC_FLAGS = ["-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-pthread"]


def compile_oracle(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile an oracle source with gcc: fp64, no contraction, no fast-math."""
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", out + ".tmp", "-lm"], check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> str:
    return compile_oracle()


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are bf16 bit patterns (uint16) or float32, got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ptr_array(arrs: Sequence[np.ndarray]):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def _sources(sources):
    srcs = [np.ascontiguousarray(s) for s in sources]
    dt = _dtype_code(srcs[0])
    rows, D = srcs[0].shape
    for s in srcs:
        if s.shape != (rows, D) or _dtype_code(s) != dt:
            raise ValueError("sources must share shape [rows, D] and dtype")
    return srcs, dt, rows, D


class Oracle:
    """One loaded oracle library (the real one, or a test's mutant build)."""

    def __init__(self, path: str = LIBRARY):
        L = ctypes.CDLL(path)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_aggregate.argtypes = [I64, I64, I, I, P, P, P, D, P, P, P, P, P, I]
        L.oracle_phase1.argtypes = [I64, I64, I, I, P, I, P, P, D, P, P, P, P, I]
        L.oracle_phase2.argtypes = [I64, I64, I, P, P, P, P, D, P, P, P, P, P, I]
        L.oracle_block_plan.argtypes = [I, I, P, P]
        L.oracle_atomic_block_size.argtypes = [I, I]
        L.oracle_block_stack.argtypes = [I64, I64, I, I, I, P, P, P, P, D,
                                         P, P, P, P, P, P, P, P, P, I]
        L.oracle_rmsnorm.argtypes = [I64, I64, I, P, P, D, P, P, I]
        L.oracle_merge.argtypes = [I64, I64, I, P, P, I, P, P, P, D, P, P, P, P, I]
        L.oracle_aggregate_backward.argtypes = [I64, I64, I, I, P, P, P, D, P, P, P, P, I]
        L.oracle_round.argtypes = [D, I]
        L.oracle_round.restype = D
        L.oracle_store_rounded.argtypes = [P, I64, I, P]
        L.oracle_store_rounded.restype = None
        for f in ("oracle_aggregate", "oracle_phase1", "oracle_phase2", "oracle_block_plan",
                  "oracle_atomic_block_size", "oracle_block_stack", "oracle_rmsnorm", "oracle_merge",
                  "oracle_aggregate_backward",
                  "oracle_max_sources"):
            getattr(L, f).restype = ctypes.c_int
        self.lib = L
        self.path = path

    def aggregate(self, sources, w, gamma=None, eps=1e-8, nthreads=None, want_alpha=False):
        """AGG over ``sources`` (list of [rows, D]) with query ``w`` [D] and gain ``gamma``."""
        srcs, dt, rows, D = _sources(sources)
        n = len(srcs)
        w, gamma = _f32(w), _f32(gamma)
        h = np.empty((rows, D)); sc = np.empty((rows, D))
        m = np.empty(rows); lse = np.empty(rows)
        alpha = np.empty((rows, n)) if want_alpha else None
        keep = _ptr_array(srcs)
        rc = self.lib.oracle_aggregate(rows, D, dt, n, keep, _ptr(w), _ptr(gamma), eps, _ptr(h),
                                       _ptr(sc), _ptr(m), _ptr(lse), _ptr(alpha),
                                       nthreads or default_threads())
        _check(rc, "oracle_aggregate")
        out = {"h": h, "scale": sc, "m": m, "lse": lse}
        if want_alpha:
            out["alpha"] = alpha
        return out

    def phase1(self, blocks, W, Gamma=None, eps=1e-8, nthreads=None):
        """Phase 1: the S queries (rows of ``W`` [S, D]) over the fixed block list."""
        srcs, dt, rows, D = _sources(blocks)
        W, Gamma = _f32(W), _f32(Gamma)
        S = W.shape[0]
        o = np.empty((S, rows, D)); sc = np.empty((S, rows, D))
        m = np.empty((S, rows)); lse = np.empty((S, rows))
        keep = _ptr_array(srcs)
        rc = self.lib.oracle_phase1(rows, D, dt, len(srcs), keep, S, _ptr(W), _ptr(Gamma), eps,
                                    _ptr(o), _ptr(sc), _ptr(m), _ptr(lse),
                                    nthreads or default_threads())
        _check(rc, "oracle_phase1")
        return {"o": o, "scale": sc, "m": m, "lse": lse}

    def phase2(self, o, lse, w, p_prev, v_prev, gamma=None, eps=1e-8, nthreads=None):
        """Phase 2 for one sublayer; ``p_prev`` None is the first merge (p = v_prev)."""
        o = np.ascontiguousarray(o); v_prev = np.ascontiguousarray(v_prev)
        dt = _dtype_code(o)
        rows, D = o.shape
        lse = np.ascontiguousarray(lse, dtype=np.float32)
        w, gamma = _f32(w), _f32(gamma)
        pp = None if p_prev is None else np.ascontiguousarray(p_prev)
        p_out = np.empty_like(v_prev)
        h = np.empty((rows, D)); sc = np.empty((rows, D))
        rc = self.lib.oracle_phase2(rows, D, dt, _ptr(o), _ptr(lse), _ptr(w), _ptr(gamma), eps,
                                    _ptr(pp), _ptr(v_prev), _ptr(p_out), _ptr(h), _ptr(sc),
                                    nthreads or default_threads())
        _check(rc, "oracle_phase2")
        return {"p": p_out, "h": h, "scale": sc}

    def aggregate_backward(self, sources, w, dh, gamma=None, eps=1e-8, nthreads=None):
        """Gradients of one aggregate for upstream dh [rows, D]: dV [n, rows, D],
        dw [D] and dgamma [D] (None without a gain), all float64."""
        srcs, dt, rows, D = _sources(sources)
        dh = np.ascontiguousarray(dh)
        w, gamma = _f32(w), _f32(gamma)
        dV = np.empty((len(srcs), rows, D)); dw = np.empty(D)
        dg = np.empty(D) if gamma is not None else None
        rc = self.lib.oracle_aggregate_backward(rows, D, dt, len(srcs), _ptr_array(srcs), _ptr(w),
                                                _ptr(gamma), eps, _ptr(dh), _ptr(dV), _ptr(dw),
                                                _ptr(dg), nthreads or default_threads())
        _check(rc, "oracle_aggregate_backward")
        return {"dV": dV, "dw": dw, "dgamma": dg}

    def merge(self, o, lse, sources, w, gamma=None, eps=1e-8, nthreads=None):
        """Merge a normalised group (o [rows, D], lse [rows]) with more sources."""
        o = np.ascontiguousarray(o)
        srcs = [np.ascontiguousarray(a) for a in sources]
        dt = _dtype_code(o)
        rows, D = o.shape
        lse = np.ascontiguousarray(lse, dtype=np.float32)
        w, gamma = _f32(w), _f32(gamma)
        h = np.empty((rows, D)); sc = np.empty((rows, D)); m = np.empty(rows); ls = np.empty(rows)
        rc = self.lib.oracle_merge(rows, D, dt, _ptr(o), _ptr(lse), len(srcs), _ptr_array(srcs), _ptr(w),
                                   _ptr(gamma), eps, _ptr(h), _ptr(sc), _ptr(m), _ptr(ls),
                                   nthreads or default_threads())
        _check(rc, "oracle_merge")
        return {"h": h, "scale": sc, "m": m, "lse": ls}

    def rmsnorm(self, x, gamma=None, eps=1e-6, nthreads=None):
        """RMSNorm of the rows of ``x`` (fp32 or bf16 bit patterns): fp64 outputs and per-row rms."""
        x = np.ascontiguousarray(x)
        dt = _dtype_code(x)
        rows, D = x.shape
        gamma = _f32(gamma)
        out = np.empty((rows, D)); rms = np.empty(rows)
        rc = self.lib.oracle_rmsnorm(rows, D, dt, _ptr(x), _ptr(gamma), eps, _ptr(out), _ptr(rms),
                                     nthreads or default_threads())
        _check(rc, "oracle_rmsnorm")
        return {"out": out, "rms": rms}

    def block_plan(self, L: int, S: int):
        """(nb, block_start[nb+1], n_sources[L+1]) of the naive Block forward."""
        bs = np.zeros(L + 2, dtype=np.int32)
        ns = np.zeros(L + 1, dtype=np.int32)
        nb = self.lib.oracle_block_plan(L, S, _ptr(bs), _ptr(ns))
        _check(0 if nb > 0 else nb, "oracle_block_plan")
        return nb, bs[: nb + 1].copy(), ns

    def atomic_block_size(self, num_hidden_layers: int, layers_per_block=None) -> int:
        return self.lib.oracle_atomic_block_size(
            num_hidden_layers, 0 if layers_per_block is None else int(layers_per_block))

    def round_to(self, x, dtype: str) -> np.ndarray:
        """Round float64 values to the dtype (nearest-even): bf16 bit patterns or float32."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
        self.lib.oracle_store_rounded(_ptr(x), x.size, BF16 if dtype == "bf16" else F32, _ptr(out))
        return out

    def block_stack(self, x, v, W, S, Gamma=None, eps=1e-8, want_h=True, nthreads=None):
        """Naive Block stack forward over the rows of ``x`` [rows, D] with sublayer
        outputs ``v`` (L arrays [rows, D]) and queries ``W`` [L+1, D]."""
        x = np.ascontiguousarray(x)
        dt = _dtype_code(x)
        rows, D = x.shape
        L = len(v)
        vs = [np.ascontiguousarray(a) for a in v]
        for a in vs:
            if a.shape != (rows, D) or _dtype_code(a) != dt:
                raise ValueError("v_l must match x")
        W, Gamma = _f32(W), _f32(Gamma)
        if W.shape != (L + 1, D):
            raise ValueError("W must be [L+1, D]")
        nb = self.lib.oracle_block_plan(L, S, None, None)
        h = np.empty((L, rows, D)) if want_h else None
        hs = np.empty((L, rows, D)) if want_h else None
        hm = np.empty((L, rows)); hl = np.empty((L, rows))
        y = np.empty((rows, D)); ys = np.empty((rows, D)); ym = np.empty(rows); yl = np.empty(rows)
        bsums = np.empty((nb, rows, D), dtype=x.dtype)
        keep = _ptr_array(vs)
        rc = self.lib.oracle_block_stack(rows, D, dt, L, S, _ptr(x), keep, _ptr(W), _ptr(Gamma),
                                         eps, _ptr(h), _ptr(hs), _ptr(hm), _ptr(hl), _ptr(y),
                                         _ptr(ys), _ptr(ym), _ptr(yl), _ptr(bsums),
                                         nthreads or default_threads())
        _check(rc, "oracle_block_stack")
        return {"h": h, "h_scale": hs, "h_m": hm, "h_lse": hl, "y": y, "y_scale": ys, "y_m": ym,
                "y_lse": yl, "block_sums": bsums, "nb": nb}


    def block_stack_backward(self, x, v, W, S, dh, dy, Gamma=None, eps=1e-8, agg_fn=None, nthreads=None):
        """Gradients of L = sum_l <dh_l, h_l> + <dy, y> through the naive Block
        stack forward (K3 9.3 forward_naive, final aggregate of K3 9.1): the
        aggregate backward of every aggregate, composed over the sources
        forward_naive gives it. Sublayer l of block k aggregates the embedding
        x, the completed block sums b_1..b_k and (from its block's second
        sublayer on) the partial, the rounded left fold of the block's earlier
        outputs; y aggregates x and every block sum. A block sum's gradient
        goes to each output of its block and a partial's to each output it
        sums (rounding to the I/O dtype taken as the identity). Returns dx
        [rows, D], dv [L, rows, D], dW [L+1, D] and dGamma [L+1, D] (None
        without gains), float64. ``agg_fn(srcs, w, dh, gamma, eps)`` may
        replace the aggregate backward (same result keys) to compose other
        per-aggregate quantities the same way."""
        x = np.ascontiguousarray(x)
        v = [np.ascontiguousarray(a) for a in v]
        L = len(v)
        rows, D = x.shape
        dt = "bf16" if _dtype_code(x) == BF16 else "f32"
        W = _f32(W)
        Gamma = _f32(Gamma)
        if agg_fn is None:
            agg_fn = lambda srcs, w, d, g, e: self.aggregate_backward(srcs, w, d, g, eps=e, nthreads=nthreads)
        st = self.block_stack(x, v, W, S, Gamma, eps, want_h=False, nthreads=nthreads)
        bsums = list(st["block_sums"])
        nb = st["nb"]
        dx = np.zeros((rows, D))
        dv = np.zeros((L, rows, D))
        db = np.zeros((nb + 1, rows, D))
        dW = np.zeros((L + 1, D))
        dG = np.zeros((L + 1, D)) if Gamma is not None else None
        wide = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) \
            if a.dtype == np.uint16 else a.astype(np.float64)
        for l in range(1, L + 1):
            k, j = (l - 1) // S, (l - 1) % S
            start = k * S + 1
            srcs = [x] + bsums[:k]
            if j >= 1:
                part = v[start - 1]
                for t in range(start + 1, l):
                    part = self.round_to(wide(part) + wide(v[t - 1]), dt)
                srcs = srcs + [part]
            out = agg_fn(srcs, W[l - 1], dh[l - 1], None if Gamma is None else Gamma[l - 1], eps)
            dx += out["dV"][0]
            for i in range(1, k + 1):
                db[i] += out["dV"][i]
            if j >= 1:
                for t in range(start, l):  # the partial sums outputs start .. l-1
                    dv[t - 1] += out["dV"][-1]
            dW[l - 1] = out["dw"]
            if dG is not None:
                dG[l - 1] = out["dgamma"]
        out = agg_fn([x] + bsums, W[L], dy, None if Gamma is None else Gamma[L], eps)
        dx += out["dV"][0]
        for i in range(1, nb + 1):
            db[i] += out["dV"][i]
        dW[L] = out["dw"]
        if dG is not None:
            dG[L] = out["dgamma"]
        for i in range(1, nb + 1):  # block sum b_i sums the outputs of block i-1
            for t in range((i - 1) * S + 1, min(i * S, L) + 1):
                dv[t - 1] += db[i]
        return {"dx": dx, "dv": dv, "dW": dW, "dGamma": dG}


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def aggregate(*a, **k):
    return default().aggregate(*a, **k)


def phase1(*a, **k):
    return default().phase1(*a, **k)


def phase2(*a, **k):
    return default().phase2(*a, **k)


def aggregate_backward(*a, **k):
    return default().aggregate_backward(*a, **k)


def merge(*a, **k):
    return default().merge(*a, **k)


def rmsnorm(*a, **k):
    return default().rmsnorm(*a, **k)


def block_plan(*a, **k):
    return default().block_plan(*a, **k)


def atomic_block_size(*a, **k):
    return default().atomic_block_size(*a, **k)


def round_to(*a, **k):
    return default().round_to(*a, **k)


def block_stack(*a, **k):
    return default().block_stack(*a, **k)


def block_stack_backward(*a, **k):
    return default().block_stack_backward(*a, **k)
