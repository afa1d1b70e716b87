"""Device-resident synthetic workloads for tests and the benchmark.

Builds a workload's inputs on the GPU with the seeded generator
(``inputs``): the embedding x, the sublayer outputs v_1..v_L (a resident table
or a 3-slot ring regenerated per sublayer), the fp32 pseudo-queries, the
block-sum outputs, y and the workspace, then runs
``attnres_block_stack_forward``. Optionally records chosen token rows of every
h_l. No AttnRes arithmetic lives here.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import binding, inputs

EPS = float(np.float32(1e-8))  # the eps every configuration uses, as the fp32 the kernels see


def torch_dtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


class DeviceStack:
    def __init__(self, wl: inputs.Workload, device="cuda", W_host: Optional[np.ndarray] = None,
                 gains: bool = False):
        """``gains``: give every query its own RMSNorm gain [L+1, D] ~ U(0.5, 1.5)
        (self.Gamma_host) instead of ones."""
        assert wl.kind == "stack"
        self.wl = wl
        self.device = device
        R, D, L, S = wl.R, wl.D, wl.L, wl.S
        self.dt = torch_dtype(wl.dtype)
        self.W_host = W_host if W_host is not None else inputs.queries(wl.seed, L + 1, D)
        self.W = torch.from_numpy(self.W_host).to(device)
        self.Gamma_host = (np.stack([inputs.gains(wl.seed + 7, D, layer=l) for l in range(L + 1)])
                           .astype(np.float32) if gains else None)
        self.Gamma = None if self.Gamma_host is None else torch.from_numpy(self.Gamma_host).to(device)
        self.x = torch.empty((R, D), dtype=self.dt, device=device)
        inputs.fill_normal(self.x, wl.seed, inputs.ROLE_X, 0, wl.x_sigma)
        self.scales = wl.scales()
        self._keep = []
        if wl.ring:
            self.slots = [torch.empty((R, D), dtype=self.dt, device=device) for _ in range(3)]
            self._scales_c = (ctypes.c_double * L)(*self.scales.tolist())
            ctx = inputs.RingCtx()
            ctx.seed, ctx.role, ctx.dtype = wl.seed, inputs.ROLE_V, 1 if wl.dtype == "bf16" else 0
            ctx.R, ctx.D, ctx.L = R, D, L
            ctx.scales = ctypes.cast(self._scales_c, ctypes.c_void_p)
            for i in range(3):
                ctx.slots[i] = self.slots[i].data_ptr()
            self._ring_ctx = ctx
            self.v = None
            self.sublayer = binding.NativeSublayer(
                inputs.fn_ptr("attnres_inputs_ring_sublayer"), ctypes.cast(ctypes.pointer(ctx), ctypes.c_void_p))
        else:
            self.v = []
            for l in range(1, L + 1):
                t = torch.empty((R, D), dtype=self.dt, device=device)
                inputs.fill_normal(t, wl.seed, inputs.ROLE_V, l, float(self.scales[l - 1]))
                self.v.append(t)
            self._table = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.v])
            self.sublayer = binding.NativeSublayer(
                ctypes.cast(binding.lib().attnres_table_sublayer, ctypes.c_void_p).value,
                ctypes.cast(self._table, ctypes.c_void_p))
        self.nb = binding.attnres_block_layout(L, S)[0]
        self.block_sums = None if S == 1 and not wl.ring else [
            torch.empty((R, D), dtype=self.dt, device=device) for _ in range(self.nb)]
        self.y = torch.empty((R, D), dtype=self.dt, device=device)
        need = binding.attnres_stack_workspace_bytes(L, S, R, D, self.dt)
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        self.overlap_workspace = None

    def recorder(self, rows: np.ndarray):
        """A sublayer callback that records token rows ``rows`` of every h_l
        (into self.rec [L, len(rows), D]) and then defers to self.sublayer."""
        wl = self.wl
        self.rec_rows = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(self.device)
        self.rec = torch.empty((wl.L, len(rows), wl.D), dtype=self.dt, device=self.device)
        ctx = inputs.RecorderCtx()
        ctx.inner = self.sublayer.fn_ptr
        ctx.inner_ctx = self.sublayer.ctx
        ctx.rec = self.rec.data_ptr()
        ctx.rows = self.rec_rows.data_ptr()
        ctx.nrows = len(rows)
        ctx.row_bytes = wl.D * self.rec.element_size()
        ctx.L = wl.L
        self._rec_ctx = ctx
        return binding.NativeSublayer(inputs.fn_ptr("attnres_inputs_record_sublayer"),
                                      ctypes.cast(ctypes.pointer(ctx), ctypes.c_void_p))

    def forward(self, sublayer=None, stream=None, norm=None, side_stream=None):
        """One stack forward; ``norm=(Gamma_f, eps_f)`` hands the sublayers
        RMSNorm(h_l) * Gamma_f[l-1] instead of h_l. With ``side_stream`` the
        forward runs the decode schedule (attnres_block_stack_forward_overlap),
        each block's Phase 1 on that stream."""
        wl = self.wl
        if side_stream is not None:
            if self.block_sums is None:
                self.block_sums = [torch.empty((wl.R, wl.D), dtype=self.dt, device=self.device)
                                   for _ in range(self.nb)]
            if self.overlap_workspace is None:
                need = binding.attnres_stack_overlap_workspace_bytes(wl.L, wl.S, wl.R, wl.D, self.dt)
                self.overlap_workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            return binding.attnres_block_stack_forward_overlap(
                self.x, self.W, wl.S, sublayer or self.sublayer, side_stream, Gamma=self.Gamma, eps=EPS,
                block_sums=self.block_sums, y=self.y, workspace=self.overlap_workspace, stream=stream,
                norm=norm)
        return binding.attnres_block_stack_forward(
            self.x, self.W, wl.S, sublayer or self.sublayer, Gamma=self.Gamma, eps=EPS,
            block_sums=self.block_sums, y=self.y, workspace=self.workspace, stream=stream, norm=norm,
            keep_sources=not wl.ring)

    def host_rows(self, rows: np.ndarray):
        """The generated inputs at token rows ``rows``, copied to the host:
        (x_rows, [v_1 rows, ..., v_L rows]) as uint16 bf16 patterns or float32."""
        from_dev = _to_host
        ids = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(self.device)
        wl = self.wl
        buf = torch.empty((len(rows), wl.D), dtype=self.dt, device=self.device)
        inputs.fill_normal(buf, wl.seed, inputs.ROLE_X, 0, wl.x_sigma, row_ids=ids)
        xr = from_dev(buf)
        vr = []
        for l in range(1, wl.L + 1):
            inputs.fill_normal(buf, wl.seed, inputs.ROLE_V, l, float(self.scales[l - 1]), row_ids=ids)
            vr.append(from_dev(buf))
        return xr, vr


def _to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
