"""GPU parity of the sublayer input norm: attnres_rmsnorm, the norm fused into
the Phase-2 merge, and the stack forward that hands each sublayer
RMSNorm(h_l) * Gamma_f[l-1] (attnres_block_stack_forward_norm).

References come from the oracle alone: its own aggregate h, rounded to the
I/O dtype by the oracle, then its fp64 RMSNorm. The GPU normalises its own
rounded h, which may sit one rounding step away from the oracle's, so the
norm's scaled error uses scale |gamma_f[d]| * (scale_h[d] + |h[d]|) / rms(h):
an error of e * scale_h in h, a relative error d in the row's rms and the
final rounding (2^-9 |hn| for bf16) stay below max(e, d + 2^-9) of it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from depth_wise_attention_rms_amd.workload import EPS, DeviceStack
from tests.stack_check import norm_reference
from tests.parity import assert_close_scaled, sample_rows, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()
    inputs.lib()
    yield
    torch.cuda.synchronize()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


NORM_CASES = [
    # (R, D, dtype, gain, eps, inplace)
    (37, 4096, "bf16", True, 1e-6, False), (130, 1000, "bf16", False, 1e-8, True),
    (5, 7168, "bf16", True, 0.25, False), (1, 8, "bf16", True, 1e-6, False),
    (3, 16384, "bf16", True, 1e-6, True), (65, 4096, "f32", True, 1e-6, True),
    (9, 1028, "f32", False, 0.0, False),
]


@pytest.mark.parametrize("R,D,dtype,gain,eps_f,inplace", NORM_CASES)
def test_rmsnorm_matches_oracle(R, D, dtype, gain, eps_f, inplace):
    announce(f"rmsnorm R={R} D={D} {dtype} gain={gain} eps={eps_f} inplace={inplace}")
    x = inputs.tensor_rows(41, inputs.ROLE_AUX, 5, np.arange(R), D, 2.5, dtype)
    g = inputs.gains(41, D) if gain else None
    xd = to_device(x)
    out = b.attnres_rmsnorm(xd, None if g is None else torch.from_numpy(g).cuda(), eps=eps_f,
                            out=xd if inplace else None)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x, g, eps=eps_f)["out"]
    assert_close_scaled(to_host(out), ref, np.abs(ref), dtype, "rmsnorm")


def test_rmsnorm_zero_rows_and_validation():
    announce("rmsnorm edge cases")
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    out = b.attnres_rmsnorm(x, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0, "a zero row normalises to zeros"
    b.attnres_rmsnorm(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), eps=1e-6)
    with pytest.raises(b.AttnResError):
        b.attnres_rmsnorm(x, eps=-1.0)


PH2N_CASES = [
    # (R, D, dtype, has_prev, want_h)
    (65, 4096, "bf16", True, False), (65, 4096, "bf16", False, True), (37, 7168, "bf16", True, True),
    (130, 1000, "bf16", True, False), (1, 8, "bf16", False, False), (65, 4096, "f32", True, True),
]


@pytest.mark.parametrize("R,D,dtype,has_prev,want_h", PH2N_CASES)
def test_phase2_merge_norm(R, D, dtype, has_prev, want_h):
    announce(f"phase2 norm R={R} D={D} {dtype} prev={has_prev} want_h={want_h}")
    o = inputs.tensor_rows(51, inputs.ROLE_AUX, 1, np.arange(R), D, 1.0, dtype)
    v = inputs.tensor_rows(51, inputs.ROLE_AUX, 2, np.arange(R), D, 3.0, dtype)
    p = inputs.tensor_rows(51, inputs.ROLE_AUX, 3, np.arange(R), D, 2.0, dtype) if has_prev else None
    lse = (2.0 * inputs.normal(51, inputs.ROLE_AUX, 4, np.arange(R))).astype(np.float32)
    w = inputs.queries(51, 1, D, sigma=0.3 / math.sqrt(D / 64))[0]
    gf = inputs.gains(52, D)
    eps_f = 1e-6
    hn, h, p_res = b.attnres_phase2_merge_norm(
        to_device(o), torch.from_numpy(lse).cuda(), torch.from_numpy(w).cuda(), to_device(v),
        gamma_f=torch.from_numpy(gf).cuda(), eps_f=eps_f,
        p_prev=None if p is None else to_device(p), eps=EPS, want_h=want_h)
    torch.cuda.synchronize()
    ref = oracle.phase2(o, lse, w, p, v, None, eps=EPS)
    hn_ref, scale = norm_reference(ref["h"], ref["scale"], dtype, gf, eps_f)
    assert_close_scaled(to_host(hn), hn_ref, scale, dtype, "phase2 hn")
    if want_h:
        assert_close_scaled(to_host(h), ref["h"], ref["scale"], dtype, "phase2 h")
    if has_prev:
        assert np.array_equal(to_host(p_res), ref["p"]), "partial p must be bit-exact"


STACK_NORM = [
    # Block with the matrix-core Phase 1, several rows per workgroup
    inputs.Workload("norm_block", "stack", B=2, T=150, D=1024, dtype="bf16", L=12, S=4, seed=3),
    # Full AttnRes (S = 1): every sublayer's h is an aggregate normalised in place
    inputs.Workload("norm_full", "stack", B=1, T=64, D=256, dtype="bf16", L=6, S=1, seed=4),
    # S > 8: the vector-ALU Phase 1, and a short last block
    inputs.Workload("norm_wide", "stack", B=4, T=10, D=512, dtype="bf16", L=14, S=12, seed=5),
    inputs.Workload("norm_f32", "stack", B=1, T=5, D=64, dtype="f32", L=7, S=3, seed=6),
    # the register-tile Phase 1 writing output 0's norm itself, at D = 4096 with
    # 2..7 sources (8 sources there take the separate norm pass) and D = 3072;
    # more rows than workgroups, ragged
    inputs.Workload("norm_block_4096", "stack", B=1, T=600, D=4096, dtype="bf16", L=32, S=4, seed=7),
    inputs.Workload("norm_block_3072", "stack", B=3, T=100, D=3072, dtype="bf16", L=18, S=6, seed=8),
    # 8 queries per block (two full query tiles, as config 3) and 3 (an odd
    # count: the last query pair's upper half is empty)
    inputs.Workload("norm_block_S8", "stack", B=1, T=270, D=2048, dtype="bf16", L=21, S=8, seed=10),
    inputs.Workload("norm_block_S3", "stack", B=1, T=333, D=4096, dtype="bf16", L=11, S=3, seed=11),
]


@pytest.mark.parametrize("wl", STACK_NORM, ids=[w.name for w in STACK_NORM])
def test_stack_forward_norm(wl):
    """Every sublayer receives RMSNorm(h_l) * Gamma_f[l-1]; y and the block sums
    are bit-identical to the forward without the norm."""
    announce(wl.name)
    ds = DeviceStack(wl)
    Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
    eps_f = 1e-6
    ds.forward()
    torch.cuda.synchronize()
    y_plain = to_host(ds.y)
    bs_plain = None if ds.block_sums is None else [to_host(t) for t in ds.block_sums]
    rows = np.arange(wl.R)
    ds.forward(ds.recorder(rows), norm=(torch.from_numpy(Gf).cuda(), eps_f))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ds.y), y_plain), "the norm must not change y"
    if bs_plain is not None:
        for k, t in enumerate(ds.block_sums):
            assert np.array_equal(to_host(t), bs_plain[k]), f"the norm must not change b_{k + 1}"
    rec = to_host(ds.rec)
    xr, vr = ds.host_rows(rows)
    ref = oracle.block_stack(xr, vr, ds.W_host, wl.S, eps=EPS)
    for l in range(wl.L):
        hn_ref, scale = norm_reference(ref["h"][l], ref["h_scale"][l], wl.dtype, Gf[l], eps_f)
        assert_close_scaled(rec[l], hn_ref, scale, wl.dtype, f"{wl.name} hn_{l + 1}")


def test_stack_forward_norm_without_gains():
    """Gamma_f = NULL (a gain of one): the matrix-core Phase 1 then stages ones
    as its gain, and the merges and the statistics pass skip theirs. 300 rows
    of 4096, blocks of 4 (Phase 1 over 2 and 3 sources)."""
    wl = inputs.Workload("norm_nogain_4096", "stack", B=1, T=300, D=4096, dtype="bf16", L=12, S=4, seed=9)
    announce(wl.name)
    ds = DeviceStack(wl)
    eps_f = 1e-6
    rows = np.arange(wl.R)
    ds.forward(ds.recorder(rows), norm=(None, eps_f))
    torch.cuda.synchronize()
    rec = to_host(ds.rec)
    xr, vr = ds.host_rows(rows)
    ref = oracle.block_stack(xr, vr, ds.W_host, wl.S, eps=EPS)
    for l in range(wl.L):
        hn_ref, scale = norm_reference(ref["h"][l], ref["h_scale"][l], wl.dtype, None, eps_f)
        assert_close_scaled(rec[l], hn_ref, scale, wl.dtype, f"{wl.name} hn_{l + 1}")


def test_stack_forward_norm_benchmark_shape():
    """The normed stack at the benchmark's shape and launch configuration
    (config 3's stack, 16384 rows of 4096, the gains and eps of the normed
    benchmark): 128 sampled rows of every hn_l against the oracle; y and the
    block sums bit-identical to the forward without the norm."""
    wl = inputs.WORKLOADS["block_L48_S8"]
    announce(f"{wl.name} normed")
    ds = DeviceStack(wl)
    Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
    eps_f = 1e-6
    ds.forward()
    torch.cuda.synchronize()
    y_plain = to_host(ds.y)
    bs_plain = [to_host(t) for t in ds.block_sums]
    rows = sample_rows(wl.R, 128, seed=5)
    ds.forward(ds.recorder(rows), norm=(torch.from_numpy(Gf).cuda(), eps_f))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ds.y), y_plain), "the norm must not change y"
    for k, t in enumerate(ds.block_sums):
        assert np.array_equal(to_host(t), bs_plain[k]), f"the norm must not change b_{k + 1}"
    rec = to_host(ds.rec)
    xr, vr = ds.host_rows(rows)
    ref = oracle.block_stack(xr, vr, ds.W_host, wl.S, eps=EPS)
    for l in range(wl.L):
        hn_ref, scale = norm_reference(ref["h"][l], ref["h_scale"][l], wl.dtype, Gf[l], eps_f)
        assert_close_scaled(rec[l], hn_ref, scale, wl.dtype, f"{wl.name} hn_{l + 1}")
    del ds
    torch.cuda.empty_cache()


def test_stack_forward_norm_scores_pass():
    """The normed stack whose Phase 1 runs as the matrix-core scores pass and
    the outputs pass (4096 rows of 7168, 12 queries, a short last block):
    sampled rows of every hn_l against the oracle; y and the block sums
    bit-identical to the forward without the norm."""
    wl = inputs.Workload("norm_gemm", "stack", B=1, T=4096, D=7168, dtype="bf16", L=27, S=12, seed=12)
    announce(wl.name)
    ds = DeviceStack(wl)
    Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
    eps_f = 1e-6
    ds.forward()
    torch.cuda.synchronize()
    y_plain = to_host(ds.y)
    bs_plain = [to_host(t) for t in ds.block_sums]
    rows = sample_rows(wl.R, 128)
    ds.forward(ds.recorder(rows), norm=(torch.from_numpy(Gf).cuda(), eps_f))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ds.y), y_plain), "the norm must not change y"
    for k, t in enumerate(ds.block_sums):
        assert np.array_equal(to_host(t), bs_plain[k]), f"the norm must not change b_{k + 1}"
    rec = to_host(ds.rec)
    xr, vr = ds.host_rows(rows)
    ref = oracle.block_stack(xr, vr, ds.W_host, wl.S, eps=EPS)
    for l in range(wl.L):
        hn_ref, scale = norm_reference(ref["h"][l], ref["h_scale"][l], wl.dtype, Gf[l], eps_f)
        assert_close_scaled(rec[l], hn_ref, scale, wl.dtype, f"{wl.name} hn_{l + 1}")
    del ds
    torch.cuda.empty_cache()


@pytest.mark.parametrize("norm", [False, True])
def test_phase2_merge_large_rows_nontemporal(norm):
    """Phase 2 on [R, D] tensors above 1 GiB (R = 75000, D = 7168, bf16),
    where p, h and hn are written with non-temporal stores: sampled rows
    against the oracle, p bit-exact."""
    R, D, dtype = 75000, 7168, "bf16"
    announce(f"phase2 large R={R} D={D} norm={norm}")
    dev = []
    for layer, sigma in ((1, 1.0), (2, 3.0), (3, 2.0)):
        t = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        dev.append(inputs.fill_normal(t, 53, inputs.ROLE_AUX, layer, sigma))
    o_d, v_d, p_d = dev
    lse = (2.0 * inputs.normal(53, inputs.ROLE_AUX, 4, np.arange(R))).astype(np.float32)
    w = inputs.queries(53, 1, D, sigma=0.3 / math.sqrt(D / 64))[0]
    gf = inputs.gains(54, D)
    eps_f = 1e-6
    lse_d, w_d = torch.from_numpy(lse).cuda(), torch.from_numpy(w).cuda()
    if norm:
        hn, h, p_res = b.attnres_phase2_merge_norm(o_d, lse_d, w_d, v_d, gamma_f=torch.from_numpy(gf).cuda(),
                                                   eps_f=eps_f, p_prev=p_d, eps=EPS, want_h=True)
    else:
        h, p_res = b.attnres_phase2_merge(o_d, lse_d, w_d, v_d, p_prev=p_d, eps=EPS)
    torch.cuda.synchronize()
    rows = sample_rows(R, 512)
    ids = torch.from_numpy(rows).cuda()
    o, v, p = (inputs.tensor_rows(53, inputs.ROLE_AUX, k, rows, D, s, dtype)
               for k, s in ((1, 1.0), (2, 3.0), (3, 2.0)))
    ref = oracle.phase2(o, lse[rows], w, p, v, None, eps=EPS)
    assert_close_scaled(to_host(h[ids]), ref["h"], ref["scale"], dtype, "phase2 h (large)")
    assert np.array_equal(to_host(p_res[ids]), ref["p"]), "partial p must be bit-exact"
    if norm:
        hn_ref, scale = norm_reference(ref["h"], ref["scale"], dtype, gf, eps_f)
        assert_close_scaled(to_host(hn[ids]), hn_ref, scale, dtype, "phase2 hn (large)")
    del dev, o_d, v_d, p_d, h, p_res
    torch.cuda.empty_cache()
