"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every comparison uses the rule of tests/parity.py (scaled error <= 1e-5 for
fp32 and 1e-2 for bf16 outputs; stats within 1e-5 (1+|ref|); block sums, the
single-source aggregate and h_1 bit-exact). Inputs come from the seeded
generator (device fill kernels or the numpy twin); the oracle reads exactly
the bits the GPU read. Full-size workloads are checked on sampled rows
(row 0, row R-1 and seeded others) in the launch configuration the benchmark
times.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from depth_wise_attention_rms_amd.workload import EPS, DeviceStack
from tests.parity import (assert_close_scaled, assert_stats, sample_rows, to_device, to_host,
                          widen)
from tests.stack_check import check_stack as _check_stack

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


def host_src(seed, role, layer, rows, D, sigma, dtype):
    return inputs.tensor_rows(seed, role, layer, np.arange(rows), D, sigma, dtype)


# ----------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------

def test_generator_device_matches_twin():
    announce("generator")
    for dtype, rows, D, scale in (("bf16", 64, 1024, 1.0), ("bf16", 7, 7168, 3.7), ("f32", 32, 256, 10.0)):
        t = torch.empty((rows, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        inputs.fill_normal(t, 0, inputs.ROLE_V, 5, scale)
        assert np.array_equal(to_host(t), inputs.tensor_rows(0, inputs.ROLE_V, 5, np.arange(rows), D, scale, dtype))
    # row-id fill equals the same rows of a full fill
    full = torch.empty((300, 512), dtype=torch.bfloat16, device="cuda")
    inputs.fill_normal(full, 3, inputs.ROLE_X, 0, 2.0)
    ids = torch.tensor([0, 17, 299, 150], dtype=torch.int64, device="cuda")
    part = torch.empty((4, 512), dtype=torch.bfloat16, device="cuda")
    inputs.fill_normal(part, 3, inputs.ROLE_X, 0, 2.0, row_ids=ids)
    assert torch.equal(part, full[ids])


# ----------------------------------------------------------------------------
# aggregate
# ----------------------------------------------------------------------------

def _run_aggregate(srcs_host, w, gamma, dtype):
    srcs = [to_device(s) for s in srcs_host]
    R = srcs_host[0].shape[0]
    m = torch.empty(R, dtype=torch.float32, device="cuda")
    lse = torch.empty(R, dtype=torch.float32, device="cuda")
    out, _, _ = b.attnres_aggregate(srcs, torch.from_numpy(w).cuda(),
                                    None if gamma is None else torch.from_numpy(gamma).cuda(),
                                    eps=EPS, m_out=m, lse_out=lse)
    torch.cuda.synchronize()
    return to_host(out), to_host(m), to_host(lse)


@pytest.mark.parametrize("zero_query", [False, True])
def test_aggregate_single_config(zero_query):
    """Single aggregate workload: n = 4 sources N(0, s^2), s in {1, 3, 0.3, 10},
    B = 2, T = 64, D = 256, fp32, gain U(0.5, 1.5), query N(0, 0.02^2) and an
    all-zero run."""
    wl = inputs.WORKLOADS["aggregate_n4"]
    announce(f"aggregate_n4 zero_query={zero_query}")
    R, D = wl.R, wl.D
    srcs = []
    for i, s in enumerate(wl.src_sigmas):
        t = torch.empty((R, D), dtype=torch.float32, device="cuda")
        inputs.fill_normal(t, wl.seed, inputs.ROLE_SRC, i, s)
        srcs.append(to_host(t))
    w = np.zeros(D, np.float32) if zero_query else inputs.queries(wl.seed, 1, D)[0]
    gamma = inputs.gains(wl.seed, D)
    h, m, lse = _run_aggregate(srcs, w, gamma, "f32")
    ref = oracle.aggregate(srcs, w, gamma, eps=EPS)
    assert_close_scaled(h, ref["h"], ref["scale"], "f32", "aggregate h")
    assert_stats(m, ref["m"], "aggregate m")
    assert_stats(lse, ref["lse"], "aggregate lse")
    if zero_query:
        mean = np.mean([widen(s) for s in srcs], axis=0)
        assert np.max(np.abs(h - mean) / ref["scale"]) <= 1e-5


AGG_CASES = [
    # (n, R, D, dtype)
    (1, 37, 520, "bf16"), (2, 37, 520, "bf16"), (3, 300, 1024, "bf16"), (5, 130, 4096, "bf16"),
    (8, 65, 7168, "bf16"), (9, 65, 4096, "bf16"), (17, 130, 1024, "bf16"), (33, 9, 2048, "bf16"),
    (64, 5, 264, "bf16"), (4, 3, 12288, "bf16"), (11, 3, 16384, "bf16"), (1, 1, 8, "bf16"),
    (2, 37, 516, "f32"), (7, 130, 4096, "f32"), (17, 33, 1024, "f32"), (3, 5, 8188, "f32"),
    (1, 37, 516, "f32"), (1, 3, 8188, "f32"),
]


@pytest.mark.parametrize("n,R,D,dtype", AGG_CASES)
def test_aggregate_sweep(n, R, D, dtype):
    announce(f"aggregate n={n} R={R} D={D} {dtype}")
    rng_sig = [0.1 + 0.7 * i for i in range(n)]
    srcs = [host_src(11, inputs.ROLE_SRC, i, R, D, rng_sig[i], dtype) for i in range(n)]
    w = inputs.queries(11 + n, 1, D, sigma=0.05)[0]
    gamma = inputs.gains(11, D) if n % 2 else None
    h, m, lse = _run_aggregate(srcs, w, gamma, dtype)
    ref = oracle.aggregate(srcs, w, gamma, eps=EPS)
    assert_close_scaled(h, ref["h"], ref["scale"], dtype, f"aggregate n={n}")
    assert_stats(m, ref["m"], "m")
    assert_stats(lse, ref["lse"], "lse")
    if n == 1:
        assert np.array_equal(h, srcs[0]), "a one-source aggregate must return the source bit for bit"


# ----------------------------------------------------------------------------
# Phase 1 and Phase 2 in isolation
# ----------------------------------------------------------------------------

PH1_CASES = [
    # (n, S, R, D, dtype)
    (1, 8, 37, 4096, "bf16"), (2, 8, 37, 264, "bf16"), (3, 5, 130, 1024, "bf16"),
    (4, 12, 65, 7168, "bf16"), (5, 8, 65, 4096, "bf16"), (6, 8, 130, 4096, "bf16"),
    (7, 3, 33, 7168, "bf16"), (8, 24, 17, 7168, "bf16"), (9, 4, 17, 1024, "bf16"),
    (12, 12, 9, 4096, "bf16"), (16, 2, 9, 4096, "bf16"), (20, 3, 5, 2048, "bf16"),
    (6, 8, 3, 16384, "bf16"), (3, 1, 1, 8, "bf16"),
    (2, 8, 37, 516, "f32"), (6, 8, 65, 4096, "f32"), (8, 5, 9, 2048, "f32"), (13, 4, 9, 1024, "f32"),
    (1, 5, 37, 1028, "f32"), (1, 3, 9, 8, "f32"),
    # the matrix-core path (bf16, S <= 8, n <= 8, D in {1024, 2048, 3072, 4096}):
    # one A tile for S <= 4, two above; R above the CU count gives each
    # workgroup several rows, so the LDS ring wraps
    (7, 8, 300, 2048, "bf16"), (8, 3, 513, 1024, "bf16"), (2, 1, 260, 3072, "bf16"),
    (4, 4, 1000, 4096, "bf16"), (5, 5, 1000, 4096, "bf16"), (8, 8, 37, 4096, "bf16"),
    (6, 8, 700, 4096, "bf16"), (1, 6, 300, 1024, "bf16"), (3, 7, 777, 3072, "bf16"),
    # everything else takes the streamed kernel (S = 9, 10 with n <= 8, more
    # than 8 sources, fp32, other widths): query tiles of 2, 4 or 8 at 8
    # elements per lane (bf16 D <= 4096, fp32 D <= 2048), 1, 2 or 4 at 16,
    # 2 (bf16) or 1 (fp32) at 32, in passes when S exceeds the tile; R well above the 512-workgroup grid makes every workgroup walk
    # many rows with the next source group in flight across row ends
    (7, 10, 300, 2048, "bf16"), (4, 9, 1000, 4096, "bf16"),
    (12, 8, 2000, 4096, "bf16"), (10, 24, 1500, 7168, "bf16"), (64, 3, 40, 1024, "bf16"),
    (9, 5, 777, 1000, "bf16"), (3, 3, 300, 8192, "f32"), (11, 17, 600, 2048, "f32"),
    (33, 6, 1100, 256, "bf16"), (12, 1, 200, 7168, "bf16"), (9, 2, 300, 7168, "bf16"),
]


@pytest.mark.parametrize("n,S,R,D,dtype", PH1_CASES)
def test_phase1_sweep(n, S, R, D, dtype):
    announce(f"phase1 n={n} S={S} R={R} D={D} {dtype}")
    srcs = [host_src(21, inputs.ROLE_SRC, i, R, D, 1.0 + 0.5 * i, dtype) for i in range(n)]
    W = inputs.queries(21 + S, S, D, sigma=0.05)
    G = np.stack([inputs.gains(21, D, layer=s) for s in range(S)]) if n % 2 == 0 else None
    out, m, lse = b.attnres_phase1_batched(
        [to_device(s) for s in srcs], torch.from_numpy(W).cuda(),
        None if G is None else torch.from_numpy(G).cuda(), eps=EPS,
        m_out=torch.empty((S, R), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.phase1(srcs, W, G, eps=EPS)
    o_h, m_h, l_h = to_host(out), to_host(m), to_host(lse)
    for s in range(S):
        assert_close_scaled(o_h[s], ref["o"][s], ref["scale"][s], dtype, f"phase1 o[{s}]")
    assert_stats(m_h, ref["m"], "phase1 m")
    assert_stats(l_h, ref["lse"], "phase1 lse")
    if n == 1:
        for s in range(S):
            assert np.array_equal(o_h[s], srcs[0]), "one source: every query returns it bit for bit"


PH2_CASES = [
    # (R, D, dtype, has_prev, inplace)
    (65, 4096, "bf16", False, False), (65, 4096, "bf16", True, False), (65, 4096, "bf16", True, True),
    (37, 7168, "bf16", True, True), (130, 1000, "bf16", True, False), (3, 16384, "bf16", True, True),
    (1, 8, "bf16", True, False), (300, 520, "bf16", False, False),
    (65, 4096, "f32", True, True), (37, 1028, "f32", False, False),
]


@pytest.mark.parametrize("R,D,dtype,has_prev,inplace", PH2_CASES)
def test_phase2_sweep(R, D, dtype, has_prev, inplace):
    announce(f"phase2 R={R} D={D} {dtype} prev={has_prev} inplace={inplace}")
    o = host_src(31, inputs.ROLE_AUX, 1, R, D, 1.0, dtype)
    v = host_src(31, inputs.ROLE_AUX, 2, R, D, 3.0, dtype)
    p = host_src(31, inputs.ROLE_AUX, 3, R, D, 2.0, dtype) if has_prev else None
    lse = (2.0 * inputs.normal(31, inputs.ROLE_AUX, 4, np.arange(R))).astype(np.float32)
    w = inputs.queries(31, 1, D, sigma=0.3 / math.sqrt(D / 64))[0]
    gamma = inputs.gains(31, D)
    o_d, v_d = to_device(o), to_device(v)
    p_d = None if p is None else to_device(p)
    p_out = p_d if (inplace and p_d is not None) else None
    h, p_res = b.attnres_phase2_merge(o_d, torch.from_numpy(lse).cuda(), torch.from_numpy(w).cuda(),
                                      v_d, p_prev=p_d, gamma=torch.from_numpy(gamma).cuda(), eps=EPS,
                                      p_out=p_out)
    torch.cuda.synchronize()
    ref = oracle.phase2(o, lse, w, p, v, gamma, eps=EPS)
    assert_close_scaled(to_host(h), ref["h"], ref["scale"], dtype, "phase2 h")
    if has_prev:
        assert np.array_equal(to_host(p_res), ref["p"]), "partial p must be bit-exact"


# ----------------------------------------------------------------------------
# stack forward
# ----------------------------------------------------------------------------

def test_stack_bruteforce_grid():
    """Every L <= 7 and S <= L+1 on 3 rows, D in {8, 16, 64} (and 1024 for bf16,
    which takes the matrix-core Phase 1), both dtypes."""
    for dtype in ("bf16", "f32"):
        for D in ((8, 16, 64, 1024) if dtype == "bf16" else (8, 16, 64)):
            for L in range(1, 8):
                for S in range(1, L + 2):
                    wl = inputs.Workload(f"grid_L{L}_S{S}_D{D}_{dtype}", "stack", B=1, T=3, D=D,
                                         dtype=dtype, L=L, S=S, seed=L * 100 + S)
                    ds = DeviceStack(wl, W_host=inputs.queries(L, L + 1, D, sigma=0.4))
                    _check_stack(ds, np.arange(3))


@pytest.mark.parametrize("B,T,D,L,S", [(2, 300, 2048, 20, 6), (1, 601, 4096, 13, 3), (1, 333, 3072, 9, 2)])
def test_stack_matrix_core_many_rows(B, T, D, L, S):
    """Block stacks whose Phase 1 runs on the matrix cores with several token
    rows per workgroup and fused block closes, bf16, all rows. Phase 1 writes
    output 0 into the sublayer-input buffer and output 1 into the partial
    buffer that its own fused close reads (blocks of 3 and 6); blocks of 2
    have no partial buffer."""
    wl = inputs.Workload(f"mfma_rows_D{D}_S{S}", "stack", B=B, T=T, D=D, dtype="bf16", L=L, S=S, seed=7 + S)
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, np.arange(wl.R), chunk=300)


def test_stack_full_config():
    """Full AttnRes stack: 16 sublayers + embedding, B = 4, T = 512, D = 1024, bf16; all rows."""
    wl = inputs.WORKLOADS["full_L16"]
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, np.arange(wl.R), chunk=512)


def test_stack_block_prefill_config():
    """Block two-phase prefill: L = 48, S = 8, B = 8, T = 2048, D = 4096, bf16;
    512 sampled rows, in the benchmark's launch configuration."""
    wl = inputs.WORKLOADS["block_L48_S8"]
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, sample_rows(wl.R, 512), chunk=128)


def test_stack_decode_config():
    """Block decode regime: L = 96, S = 12, 128 rows, D = 7168, bf16; all rows."""
    wl = inputs.WORKLOADS["decode_L96_S12"]
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, np.arange(wl.R), chunk=64)


@pytest.mark.parametrize("B,T,S,dtype", [(1, 200, 24, "bf16"), (2, 100, 12, "bf16"), (1, 40, 24, "bf16"),
                                          (1, 200, 24, "f32"), (1, 40, 12, "f32")])
def test_stack_streamed_phase1_passes(B, T, S, dtype):
    """Streamed Phase 1 with more queries than one register tile at D = 7168
    (4 per pass in bf16, fewer in fp32), with fused block closes: at 200
    rows two passes run side by side per launch and the later launches read
    the stored block sum; at 40 rows all the passes share one launch.
    L = 2 S + 3: block 2 runs all S queries over two sources, one of them
    closed on the fly, and block 3 is short."""
    L = 2 * S + 3
    wl = inputs.Workload(f"p1_passes_R{B * T}_S{S}_{dtype}", "stack", B=B, T=T, D=7168, dtype=dtype, L=L, S=S,
                         seed=S + T)
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, np.arange(wl.R), chunk=100)


GEMM_STACKS = [
    # (B, T, D, S, L): Phase 1 on the matrix-core scores pass and the outputs
    # pass (bf16, more than 8 queries or a width outside the register-tile
    # kernel, at least 4096 rows); ragged row tiles; 24 queries (3 Qp tiles)
    # then a 5-query block; sources 2..8 with S = 12, then 9 sources (16
    # columns per row, the packed outputs pass); 32 queries (4 tiles) at
    # D = 1024; 9 queries at D = 4096; 16 blocks of 4 at D = 1024 (the
    # register-tile Phase 1 up to 8 sources, then 9..16 on the scores pass);
    # 15 blocks of 3 queries at D = 7168 (every column count, odd query
    # count in the packed outputs pass)
    (1, 4100, 7168, 24, 53),
    (2, 2048, 7168, 12, 99),
    (4, 2048, 1024, 32, 71),
    (1, 4096, 4096, 9, 20),
    (1, 4100, 1024, 4, 64),
    (1, 4096, 7168, 3, 45),
]


@pytest.mark.parametrize("B,T,D,S,L", GEMM_STACKS)
def test_stack_gemm_phase1(B, T, D, S, L):
    """Block stacks whose Phase 1 runs as the scores/outputs passes, with the
    block close as its own launch: sampled rows of every h_l, y and the block
    sums against the oracle's naive forward."""
    wl = inputs.Workload(f"gemm_p1_R{B * T}_D{D}_S{S}_L{L}", "stack", B=B, T=T, D=D, dtype="bf16", L=L, S=S,
                         seed=L + S)
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, sample_rows(wl.R, 192), chunk=64)
    del ds
    torch.cuda.empty_cache()


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("T,L,S,D", [(4100, 12, 12, 7168), (4100, 24, 12, 7168), (4100, 30, 12, 7168),
                                     (4100, 54, 12, 7168), (4100, 39, 4, 1024), (4100, 62, 4, 1024),
                                     (128, 24, 12, 7168), (128, 90, 12, 7168), (77, 40, 10, 512)])
def test_scores_pass_statistics(T, L, S, D):
    """Phase 1's fp32 statistics at the 1e-5 bar: a stack of T rows whose last
    block's Phase 1 has nb sources. At 4100 rows, on the matrix-core scores
    pass: with 12 queries of 7168, L // 12 + 1 (1: statistics only, one
    column per row; 2, 3 and 5: two, four and eight columns per row; the
    short last blocks hold 6 queries); with 4 queries of 1024, 10 and 16
    (sixteen columns per row). With fewer rows, on the streamed kernel: 2 and
    8 sources at decode's shape, and 4 sources over 77 rows of 512. After the
    forward the workspace holds that block's m and lse [Sk, R] at the
    offsets of the header's layout (folded queries, outputs, m, lse),
    compared on every row with the oracle's Phase 1 over the block sums the
    GPU stored."""
    wl = inputs.Workload(f"scores_stats_T{T}_L{L}_S{S}_D{D}", "stack", B=1, T=T, D=D, dtype="bf16", L=L, S=S,
                         seed=L + 5)
    announce(wl.name)
    ds = DeviceStack(wl)
    ds.forward()
    torch.cuda.synchronize()
    R, nb = wl.R, ds.nb
    start = (nb - 1) * S + 1
    Sk = L - start + 1
    Skw = min(S, L)
    off_m = _a256((L + 1) * D * 4) + _a256(Skw * R * D * 2 if Skw > 1 else 0)
    off_lse = off_m + _a256(Skw * R * 4)
    ws = ds.workspace
    m = ws[off_m:off_m + Sk * R * 4].view(torch.float32).view(Sk, R)
    lse = ws[off_lse:off_lse + Sk * R * 4].view(torch.float32).view(Sk, R)
    blocks = [to_host(ds.x)] + [to_host(t) for t in ds.block_sums[:nb - 1]]
    ref = oracle.phase1(blocks, ds.W_host[start - 1:L], eps=EPS)
    assert_stats(to_host(m), ref["m"], f"{wl.name} m")
    assert_stats(to_host(lse), ref["lse"], f"{wl.name} lse")
    del ds
    torch.cuda.empty_cache()


def test_stack_long_context_config():
    """Long-context Block: L = 186, S = 24, T = 131072, D = 7168, bf16, sublayer
    outputs generated per sublayer into a ring; 512 sampled rows."""
    wl = inputs.WORKLOADS["long_L186_S24"]
    announce(wl.name)
    ds = DeviceStack(wl)
    _check_stack(ds, sample_rows(wl.R, 512), chunk=64)
    del ds
    torch.cuda.empty_cache()


GAIN_STACKS = [
    # (B, T, D, S, L): every query with its own RMSNorm gain, folded on the
    # GPU once per forward; the matrix-core Phase 1, the streamed Phase 1 at
    # D = 7168 with S > 8, and the matrix-core scores pass
    (2, 300, 2048, 6, 20),
    (1, 40, 7168, 12, 25),
    (1, 4096, 7168, 12, 15),
]


@pytest.mark.parametrize("B,T,D,S,L", GAIN_STACKS)
def test_stack_with_gains(B, T, D, S, L):
    """Block stacks with non-unit gains: sampled rows of every h_l, y and the
    block sums against the oracle's naive forward with the same gains."""
    wl = inputs.Workload(f"gain_R{B * T}_D{D}_S{S}_L{L}", "stack", B=B, T=T, D=D, dtype="bf16", L=L, S=S,
                         seed=L + 2 * S)
    announce(wl.name)
    ds = DeviceStack(wl, gains=True)
    _check_stack(ds, sample_rows(wl.R, 192), chunk=64)
    del ds
    torch.cuda.empty_cache()


def test_stack_is_deterministic():
    wl = inputs.Workload("det", "stack", B=2, T=1000, D=4096, dtype="bf16", L=20, S=6)
    announce("determinism")
    ds = DeviceStack(wl)
    ds.forward()
    y1 = ds.y.clone()
    b1 = [t.clone() for t in ds.block_sums]
    ds.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1, ds.y)
    assert all(torch.equal(a, c) for a, c in zip(b1, ds.block_sums))


def test_stack_zero_rows_and_callback_failure():
    wl = inputs.Workload("small", "stack", B=1, T=5, D=64, dtype="bf16", L=6, S=3)
    announce("callback failure")
    ds = DeviceStack(wl)

    def failing(l, h):
        if l == 3:
            raise RuntimeError("planted failure")
        return ds.v[l - 1]
    with pytest.raises(b.AttnResError) as e:
        b.attnres_block_stack_forward(ds.x, ds.W, 3, failing, eps=EPS, block_sums=ds.block_sums,
                                      y=ds.y, workspace=ds.workspace)
    assert e.value.code == -5 and "l = 3" in e.value.detail
    torch.cuda.synchronize()
    # R == 0 is a no-op
    x0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y0, _ = b.attnres_block_stack_forward(x0, ds.W, 3, [x0] * 6, eps=EPS)
    assert y0.shape == (0, 64)
