"""Thin Python binding of libattnres (include/attnres.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch supplies device memory and the current HIP stream. Functions
carry the C names; optional outputs may be passed as None to have them
allocated with torch.empty.

The library is loaded from this package directory (built by
``python -m depth_wise_attention_rms_amd.build``). There is no fallback: if it
is missing, or no GPU is present for a compute call, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Sequence, Union

import torch  # loads the HIP runtime that the library then binds to (same soname)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattnres.so")

ATTNRES_F32, ATTNRES_BF16 = 0, 1
STATUS = {0: "ok", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP", -5: "ECALLBACK"}
TIMING_KINDS = {"phase1": 0, "phase2": 1, "aggregate": 2, "close": 3, "fold": 4, "norm": 5,
                "backward": 6, "backward_reduce": 7, "phase1_stats": 8}

EXPORTS = (
    "attnres_aggregate", "attnres_phase1_batched", "attnres_phase2_merge",
    "attnres_phase2_merge_norm", "attnres_rmsnorm", "attnres_table_sublayer",
    "attnres_stack_workspace_bytes", "attnres_block_stack_forward",
    "attnres_block_stack_forward_norm", "attnres_stack_overlap_workspace_bytes",
    "attnres_block_stack_forward_overlap", "attnres_merge_sources", "attnres_full_workspace_bytes",
    "attnres_full_stack_forward", "attnres_aggregate_backward_workspace_bytes",
    "attnres_aggregate_backward", "attnres_aggregate_backward_noalloc",
    "attnres_table_sublayer_bwd", "attnres_stack_backward_workspace_bytes", "attnres_block_stack_backward",
    "attnres_noalloc_scratch_bytes", "attnres_block_layout",
    "attnres_atomic_block_size", "attnres_status_string", "attnres_last_error",
    "attnres_timing_enable", "attnres_timing_pause", "attnres_timing_reset", "attnres_timing_read",
    "attnres_timing_kernels", "attnres_timing_trace",
)

SUBLAYER_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                               ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p)


class AttnResError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({code}): {detail}")
        self.code = code
        self.detail = detail


_lib = None


def lib():
    """The loaded libattnres (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m depth_wise_attention_rms_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, D, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                               ctypes.c_double, ctypes.c_size_t)
        L.attnres_aggregate.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P, P]
        L.attnres_phase1_batched.argtypes = [P, I, I64, I64, I, P, P, I, F, P, P, P, P]
        L.attnres_phase2_merge.argtypes = [P, P, P, P, F, P, P, P, P, I64, I64, I, P]
        L.attnres_phase2_merge_norm.argtypes = [P, P, P, P, F, P, P, P, P, P, F, P, I64, I64, I, P]
        L.attnres_rmsnorm.argtypes = [P, I64, I64, I, P, F, P, P]
        L.attnres_table_sublayer.argtypes = [P, I, P, ctypes.POINTER(P), P]
        L.attnres_stack_workspace_bytes.argtypes = [I, I, I64, I64, I]
        L.attnres_stack_workspace_bytes.restype = SZ
        L.attnres_block_stack_forward.argtypes = [P, I, I, I64, I64, I, P, P, F, P, P, P, P, P, SZ, P]
        L.attnres_block_stack_forward_norm.argtypes = [P, I, I, I64, I64, I, P, P, F, P, F, P, P, P, P,
                                                       P, SZ, P]
        L.attnres_stack_overlap_workspace_bytes.argtypes = [I, I, I64, I64, I]
        L.attnres_stack_overlap_workspace_bytes.restype = SZ
        L.attnres_block_stack_forward_overlap.argtypes = [P, I, I, I64, I64, I, P, P, F, I, P, F, P, P, P,
                                                          P, P, SZ, P, P]
        L.attnres_merge_sources.argtypes = [P, P, P, I, I64, I64, I, P, P, F, P, P, P, P]
        L.attnres_full_workspace_bytes.argtypes = [I, I, I64, I64, I]
        L.attnres_full_workspace_bytes.restype = SZ
        L.attnres_full_stack_forward.argtypes = [P, I, I, I64, I64, I, P, P, F, P, P, P, P, SZ, P]
        L.attnres_aggregate_backward_workspace_bytes.argtypes = [I64, I64, I]
        L.attnres_aggregate_backward_workspace_bytes.restype = SZ
        L.attnres_aggregate_backward.argtypes = [P, I, I64, I64, I, P, P, F, P, P, I, P, P, P, SZ, P]
        L.attnres_aggregate_backward_noalloc.argtypes = [P, I, I64, I64, I, P, P, F, P, P, I, P, P, P]
        L.attnres_table_sublayer_bwd.argtypes = [P, I, P, ctypes.POINTER(P), P]
        L.attnres_stack_backward_workspace_bytes.argtypes = [I, I, I64, I64, I]
        L.attnres_stack_backward_workspace_bytes.restype = SZ
        L.attnres_block_stack_backward.argtypes = [P, P, I, I, I64, I64, I, P, P, F, P, P, P, P, P, P, P,
                                                   P, P, SZ, P]
        L.attnres_noalloc_scratch_bytes.argtypes = []
        L.attnres_noalloc_scratch_bytes.restype = SZ
        L.attnres_block_layout.argtypes = [I, I, P, P]
        L.attnres_atomic_block_size.argtypes = [I, I]
        L.attnres_status_string.argtypes = [I]
        L.attnres_status_string.restype = ctypes.c_char_p
        L.attnres_last_error.argtypes = []
        L.attnres_last_error.restype = ctypes.c_char_p
        L.attnres_timing_enable.argtypes = [I]
        L.attnres_timing_pause.argtypes = [I]
        L.attnres_timing_reset.argtypes = []
        L.attnres_timing_read.argtypes = [I, ctypes.POINTER(I64), ctypes.POINTER(D), ctypes.POINTER(D)]
        L.attnres_timing_trace.argtypes = [I, P, P, P, P]
        L.attnres_timing_trace.restype = I
        L.attnres_timing_kernels.argtypes = [I]
        L.attnres_timing_kernels.restype = ctypes.c_char_p
        for f in ("attnres_aggregate", "attnres_phase1_batched", "attnres_phase2_merge",
                  "attnres_phase2_merge_norm", "attnres_rmsnorm", "attnres_block_stack_forward_norm",
                  "attnres_merge_sources", "attnres_full_stack_forward", "attnres_aggregate_backward",
                  "attnres_aggregate_backward_noalloc", "attnres_table_sublayer",
                  "attnres_table_sublayer_bwd", "attnres_block_stack_backward", "attnres_block_stack_forward", "attnres_block_layout",
                  "attnres_block_stack_forward_overlap",
                  "attnres_atomic_block_size", "attnres_timing_enable", "attnres_timing_pause",
                  "attnres_timing_reset", "attnres_timing_read"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnResError(fn, rc, lib().attnres_last_error().decode())
    return rc


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return ATTNRES_BF16
    if t == torch.float32:
        return ATTNRES_F32
    raise TypeError(f"AttnRes I/O dtype must be bfloat16 or float32, not {t}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _rows(t: torch.Tensor):
    D = t.shape[-1]
    return t.numel() // D if D else 0, D


def _ptr_array(ts: Sequence[torch.Tensor]):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def attnres_aggregate(sources: Sequence[torch.Tensor], w: torch.Tensor, gamma=None, eps=1e-8,
                      out=None, m_out=None, lse_out=None, stream=None):
    """AGG over ``sources`` (each [..., D]); returns (out, m_out, lse_out)."""
    x0 = sources[0]
    R, D = _rows(x0)
    if out is None:
        out = torch.empty_like(x0)
    arr = _ptr_array(sources)
    _check("attnres_aggregate", lib().attnres_aggregate(
        arr, len(sources), R, D, dtype_code(x0.dtype), _ptr(w), _ptr(gamma), eps, _ptr(out),
        _ptr(m_out), _ptr(lse_out), _stream(stream)))
    return out, m_out, lse_out


def attnres_phase1_batched(blocks: Sequence[torch.Tensor], W: torch.Tensor, Gamma=None, eps=1e-8,
                           out=None, m_out=None, lse_out=None, stream=None):
    """Phase 1 for the S = W.shape[0] queries; returns (out [S,R,D], m [S,R], lse [S,R])."""
    x0 = blocks[0]
    R, D = _rows(x0)
    S = W.shape[0]
    if out is None:
        out = torch.empty((S, R, D), dtype=x0.dtype, device=x0.device)
    if lse_out is None:
        lse_out = torch.empty((S, R), dtype=torch.float32, device=x0.device)
    arr = _ptr_array(blocks)
    _check("attnres_phase1_batched", lib().attnres_phase1_batched(
        arr, len(blocks), R, D, dtype_code(x0.dtype), _ptr(W), _ptr(Gamma), S, eps, _ptr(out),
        _ptr(m_out), _ptr(lse_out), _stream(stream)))
    return out, m_out, lse_out


def attnres_phase2_merge(o, lse, w, v_prev, p_prev=None, gamma=None, eps=1e-8, p_out=None,
                         h_out=None, stream=None):
    """One Phase-2 merge; returns (h_out, p_out). p_out is allocated when p_prev is given."""
    R, D = _rows(o)
    if h_out is None:
        h_out = torch.empty_like(o)
    if p_prev is not None and p_out is None:
        p_out = torch.empty_like(o)
    _check("attnres_phase2_merge", lib().attnres_phase2_merge(
        _ptr(o), _ptr(lse), _ptr(w), _ptr(gamma), eps, _ptr(p_prev), _ptr(v_prev), _ptr(p_out),
        _ptr(h_out), R, D, dtype_code(o.dtype), _stream(stream)))
    return h_out, p_out


def attnres_phase2_merge_norm(o, lse, w, v_prev, gamma_f=None, eps_f=1e-6, p_prev=None, gamma=None,
                              eps=1e-8, p_out=None, h_out=None, hn_out=None, want_h=False, stream=None):
    """Phase-2 merge with the sublayer's input norm fused in; returns (hn_out, h_out, p_out).
    h_out is written only when given or ``want_h``."""
    R, D = _rows(o)
    if hn_out is None:
        hn_out = torch.empty_like(o)
    if h_out is None and want_h:
        h_out = torch.empty_like(o)
    if p_prev is not None and p_out is None:
        p_out = torch.empty_like(o)
    _check("attnres_phase2_merge_norm", lib().attnres_phase2_merge_norm(
        _ptr(o), _ptr(lse), _ptr(w), _ptr(gamma), eps, _ptr(p_prev), _ptr(v_prev), _ptr(p_out),
        _ptr(h_out), _ptr(gamma_f), eps_f, _ptr(hn_out), R, D, dtype_code(o.dtype), _stream(stream)))
    return hn_out, h_out, p_out


def attnres_rmsnorm(x, gamma=None, eps=1e-6, out=None, stream=None):
    """out = RMSNorm(x) * gamma over the last axis (out may be x)."""
    R, D = _rows(x)
    if out is None:
        out = torch.empty_like(x)
    _check("attnres_rmsnorm", lib().attnres_rmsnorm(_ptr(x), R, D, dtype_code(x.dtype), _ptr(gamma),
                                                    eps, _ptr(out), _stream(stream)))
    return out


def attnres_stack_workspace_bytes(L: int, S: int, R: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().attnres_stack_workspace_bytes(L, S, R, D, dtype_code(dtype)))


def attnres_block_layout(L: int, S: int):
    """(nb, block_start[nb+1], n_sources[L+1]) as Python lists."""
    bs = (ctypes.c_int * (L + 2))()
    ns = (ctypes.c_int * (L + 1))()
    nb = lib().attnres_block_layout(L, S, bs, ns)
    if nb < 0:
        _check("attnres_block_layout", nb)
    return nb, list(bs)[: nb + 1], list(ns)


def attnres_atomic_block_size(num_decoder_layers: int, layers_per_block: Optional[int] = None) -> int:
    rc = lib().attnres_atomic_block_size(num_decoder_layers, layers_per_block or 0)
    if rc < 0:
        _check("attnres_atomic_block_size", rc)
    return rc


class NativeSublayer:
    """A C sublayer callback (function pointer + context) from another library."""

    def __init__(self, fn_ptr: int, ctx, keepalive=()):
        self.fn_ptr = fn_ptr
        self.ctx = ctx
        self.keepalive = keepalive


Sublayer = Union[Sequence[torch.Tensor], NativeSublayer, Callable[[int, int], torch.Tensor]]


def _sublayer_fn(sublayer: Sublayer):
    """(function pointer, context, objects to keep alive) of a sublayer argument."""
    keep = []
    if isinstance(sublayer, NativeSublayer):
        return ctypes.c_void_p(sublayer.fn_ptr), sublayer.ctx, keep
    if isinstance(sublayer, (list, tuple)):
        table = _ptr_array(sublayer)
        keep.append(table)
        return (ctypes.cast(lib().attnres_table_sublayer, ctypes.c_void_p),
                ctypes.cast(table, ctypes.c_void_p), keep)
    if callable(sublayer):
        outs = []

        def tramp(_ctx, l, h, v_out, _stream):
            try:
                v = sublayer(l, h)
                outs.append(v)
                v_out[0] = v.data_ptr()
                return 0
            except Exception:  # noqa: BLE001 -- reported to the library as a callback failure
                return 1
        cfn = SUBLAYER_FN(tramp)
        keep += [cfn, outs]
        return ctypes.cast(cfn, ctypes.c_void_p), None, keep
    raise TypeError("sublayer must be a tensor list, a NativeSublayer or a callable")


def attnres_block_stack_forward(x: torch.Tensor, W: torch.Tensor, S: int, sublayer: Sublayer,
                                Gamma=None, eps=1e-8, block_sums=None, y=None, workspace=None,
                                stream=None, norm=None, keep_sources=None):
    """Block AttnRes stack forward (Full when S == 1). ``sublayer`` is a list of
    L pre-computed outputs, a NativeSublayer, or a Python callable
    ``f(l, h_ptr) -> tensor v_l``. Returns (y, block_sums). With
    ``norm=(Gamma_f, eps_f)`` (Gamma_f an [L, D] fp32 tensor or None) the
    sublayers receive RMSNorm(h_l) * Gamma_f[l-1] instead of h_l
    (attnres_block_stack_forward_norm). ``keep_sources`` (S == 1 only): the
    sublayer outputs stay valid for the whole call, so they serve as the
    sources themselves and no block sums are formed (default: True for a
    list of outputs)."""
    R, D = _rows(x)
    L = W.shape[0] - 1
    dt = dtype_code(x.dtype)
    nb = attnres_block_layout(L, S)[0]
    if y is None:
        y = torch.empty_like(x)
    if keep_sources is None:
        keep_sources = isinstance(sublayer, (list, tuple))
    if block_sums is None and not (S == 1 and keep_sources):
        block_sums = [torch.empty_like(x) for _ in range(nb)]
    need = attnres_stack_workspace_bytes(L, S, R, D, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    fn, ctx, keep = _sublayer_fn(sublayer)
    bs = _ptr_array(block_sums) if block_sums is not None else None
    if norm is None:
        _check("attnres_block_stack_forward", lib().attnres_block_stack_forward(
            _ptr(x), L, S, R, D, dt, _ptr(W), _ptr(Gamma), eps, fn, ctx, bs, _ptr(y),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    else:
        Gamma_f, eps_f = norm
        _check("attnres_block_stack_forward_norm", lib().attnres_block_stack_forward_norm(
            _ptr(x), L, S, R, D, dt, _ptr(W), _ptr(Gamma), eps, _ptr(Gamma_f), eps_f, fn, ctx, bs,
            _ptr(y), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    return y, block_sums


def attnres_stack_overlap_workspace_bytes(L: int, S: int, R: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().attnres_stack_overlap_workspace_bytes(L, S, R, D, dtype_code(dtype)))


def attnres_block_stack_forward_overlap(x: torch.Tensor, W: torch.Tensor, S: int, sublayer: Sublayer,
                                        side_stream, Gamma=None, eps=1e-8, block_sums=None, y=None,
                                        workspace=None, stream=None, norm=None):
    """The stack forward with the decode schedule: each block's Phase 1 runs on
    ``side_stream`` during the previous block (a torch.cuda.Stream of the same
    device). Arguments and result as attnres_block_stack_forward; block sums
    are always produced."""
    R, D = _rows(x)
    L = W.shape[0] - 1
    dt = dtype_code(x.dtype)
    nb = attnres_block_layout(L, S)[0]
    if y is None:
        y = torch.empty_like(x)
    if block_sums is None:
        block_sums = [torch.empty_like(x) for _ in range(nb)]
    need = attnres_stack_overlap_workspace_bytes(L, S, R, D, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    fn, ctx, keep = _sublayer_fn(sublayer)
    Gamma_f, eps_f = norm if norm is not None else (None, 0.0)
    _check("attnres_block_stack_forward_overlap", lib().attnres_block_stack_forward_overlap(
        _ptr(x), L, S, R, D, dt, _ptr(W), _ptr(Gamma), eps, 1 if norm is not None else 0,
        _ptr(Gamma_f), eps_f, fn, ctx, _ptr_array(block_sums), _ptr(y),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream), _stream(side_stream)))
    del keep
    return y, block_sums


def attnres_merge_sources(o, lse, sources, w, gamma=None, eps=1e-8, out=None, m_out=None, lse_out=None,
                          stream=None):
    """Merge a normalised group (o, lse) with more sources; returns (out, m_out, lse_out)."""
    R, D = _rows(o)
    if out is None:
        out = torch.empty_like(o)
    table = _ptr_array(sources)
    _check("attnres_merge_sources", lib().attnres_merge_sources(
        _ptr(o), _ptr(lse), table, len(sources), R, D, dtype_code(o.dtype), _ptr(w), _ptr(gamma), eps,
        _ptr(out), _ptr(m_out), _ptr(lse_out), _stream(stream)))
    return out, m_out, lse_out


def attnres_full_workspace_bytes(L: int, C: int, R: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().attnres_full_workspace_bytes(L, C, R, D, dtype_code(dtype)))


def attnres_full_stack_forward(x: torch.Tensor, W: torch.Tensor, C: int, sublayer: Sublayer, Gamma=None,
                               eps=1e-8, y=None, workspace=None, stream=None):
    """Full AttnRes stack forward with schedule block size C (C = 1: naive). Returns y."""
    R, D = _rows(x)
    L = W.shape[0] - 1
    if y is None:
        y = torch.empty_like(x)
    need = attnres_full_workspace_bytes(L, C, R, D, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    fn, ctx, keep = _sublayer_fn(sublayer)
    _check("attnres_full_stack_forward", lib().attnres_full_stack_forward(
        _ptr(x), L, C, R, D, dtype_code(x.dtype), _ptr(W), _ptr(Gamma), eps, fn, ctx, _ptr(y),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    del keep
    return y


def attnres_aggregate_backward_workspace_bytes(R: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().attnres_aggregate_backward_workspace_bytes(R, D, dtype_code(dtype)))


def attnres_aggregate_backward(sources: Sequence[torch.Tensor], w: torch.Tensor, dh: torch.Tensor,
                               gamma=None, eps=1e-8, dV=None, dw=None, dgamma=None,
                               accumulate=False, want_dgamma=None, workspace=None, stream=None):
    """Gradients of AGG(sources) for upstream ``dh``; returns (dV list of fp32
    [..., D], dw [D], dgamma [D] or None). dgamma is produced when
    ``want_dgamma`` (default: a gain is given) or a buffer is passed."""
    x0 = sources[0]
    R, D = _rows(x0)
    dev = x0.device
    if dV is None:
        dV = [torch.empty(x0.shape, dtype=torch.float32, device=dev) for _ in sources]
    if dw is None:
        dw = torch.empty(D, dtype=torch.float32, device=dev)
    if want_dgamma is None:
        want_dgamma = gamma is not None
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(D, dtype=torch.float32, device=dev)
    need = attnres_aggregate_backward_workspace_bytes(R, D, x0.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("attnres_aggregate_backward", lib().attnres_aggregate_backward(
        _ptr_array(sources), len(sources), R, D, dtype_code(x0.dtype), _ptr(w), _ptr(gamma), eps,
        _ptr(dh), _ptr_array(dV), 1 if accumulate else 0, _ptr(dw), _ptr(dgamma),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    return dV, dw, dgamma


def attnres_stack_backward_workspace_bytes(L: int, S: int, R: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().attnres_stack_backward_workspace_bytes(L, S, R, D, dtype_code(dtype)))


def attnres_block_stack_backward(x: torch.Tensor, v: Sequence[torch.Tensor], W: torch.Tensor, S: int,
                                 dy: torch.Tensor, dh: Sequence[torch.Tensor], block_sums=None,
                                 Gamma=None, eps=1e-8, dx=None, dv=None, dW=None, dGamma=None,
                                 want_dgamma=None, workspace=None, stream=None):
    """Gradients of the Block stack forward for upstream gradients dh_l (a list
    of L tensors, served by the built-in table callback) and dy. Returns
    (dx, dv list, dW, dGamma or None), all fp32."""
    R, D = _rows(x)
    L = W.shape[0] - 1
    dev = x.device
    if dx is None:
        dx = torch.empty((R, D), dtype=torch.float32, device=dev)
    if dv is None:
        dv = [torch.empty((R, D), dtype=torch.float32, device=dev) for _ in range(L)]
    if dW is None:
        dW = torch.empty((L + 1, D), dtype=torch.float32, device=dev)
    if want_dgamma is None:
        want_dgamma = Gamma is not None
    if dGamma is None and want_dgamma:
        dGamma = torch.empty((L + 1, D), dtype=torch.float32, device=dev)
    need = attnres_stack_backward_workspace_bytes(L, S, R, D, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    table = _ptr_array(dh)
    vt = _ptr_array(v)
    bs = _ptr_array(block_sums) if block_sums is not None else None
    _check("attnres_block_stack_backward", lib().attnres_block_stack_backward(
        _ptr(x), vt, L, S, R, D, dtype_code(x.dtype), _ptr(W), _ptr(Gamma), eps, bs, _ptr(dy),
        ctypes.cast(lib().attnres_table_sublayer_bwd, ctypes.c_void_p), ctypes.cast(table, ctypes.c_void_p),
        _ptr(dx), _ptr_array(dv), _ptr(dW), _ptr(dGamma), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel(), _stream(stream)))
    return dx, dv, dW, dGamma


def attnres_noalloc_scratch_bytes() -> int:
    return int(lib().attnres_noalloc_scratch_bytes())


def attnres_aggregate_backward_noalloc(sources: Sequence[torch.Tensor], w: torch.Tensor,
                                       dh: torch.Tensor, dV: Sequence[torch.Tensor], dw: torch.Tensor,
                                       gamma=None, eps=1e-8, dgamma=None, accumulate=False,
                                       stream=None):
    """attnres_aggregate_backward with the library's fixed scratch instead of a
    workspace. Every output buffer is the caller's (nothing is allocated here
    either); returns (dV, dw, dgamma)."""
    x0 = sources[0]
    R, D = _rows(x0)
    _check("attnres_aggregate_backward_noalloc", lib().attnres_aggregate_backward_noalloc(
        _ptr_array(sources), len(sources), R, D, dtype_code(x0.dtype), _ptr(w), _ptr(gamma), eps,
        _ptr(dh), _ptr_array(dV), 1 if accumulate else 0, _ptr(dw), _ptr(dgamma), _stream(stream)))
    return dV, dw, dgamma


def attnres_timing_enable(capacity: int):
    _check("attnres_timing_enable", lib().attnres_timing_enable(capacity))


def attnres_timing_pause(paused: bool):
    _check("attnres_timing_pause", lib().attnres_timing_pause(1 if paused else 0))


def attnres_timing_reset():
    _check("attnres_timing_reset", lib().attnres_timing_reset())


def attnres_timing_read(kind: str):
    """(launches, total_ms, total_algorithmic_bytes) recorded for a kernel kind."""
    n = ctypes.c_int64(); ms = ctypes.c_double(); b = ctypes.c_double()
    _check("attnres_timing_read", lib().attnres_timing_read(TIMING_KINDS[kind], ctypes.byref(n),
                                                            ctypes.byref(ms), ctypes.byref(b)))
    return n.value, ms.value, b.value


def attnres_timing_trace(max_launches: int = 4096):
    """[(kind name, stream handle, start ms, end ms)] of the timed launches, in
    enqueue order, relative to the first one's start."""
    import numpy as np
    kinds = np.zeros(max_launches, np.int32)
    streams = np.zeros(max_launches, np.uint64)
    t0 = np.zeros(max_launches, np.float64)
    t1 = np.zeros(max_launches, np.float64)
    n = lib().attnres_timing_trace(max_launches, kinds.ctypes.data, streams.ctypes.data, t0.ctypes.data,
                                   t1.ctypes.data)
    if n < 0:
        _check("attnres_timing_trace", n)
    names = {v: k for k, v in TIMING_KINDS.items()}
    return [(names.get(int(kinds[i]), str(kinds[i])), int(streams[i]), float(t0[i]), float(t1[i]))
            for i in range(n)]


def attnres_timing_kernels(kind: str) -> str:
    """Comma-separated names of the kernels the timed launches of a kind ran."""
    return lib().attnres_timing_kernels(TIMING_KINDS[kind]).decode()
