"""GPU parity of the Full AttnRes two-phase schedule: attnres_merge_sources
against the oracle's merge, and attnres_full_stack_forward (schedule block
size C) against the oracle's naive Full forward (Block with S = 1), on every
row and every sublayer."""
import math

import numpy as np
import pytest
import torch

import oracle
from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from depth_wise_attention_rms_amd.workload import EPS, DeviceStack
from tests.parity import assert_close_scaled, assert_stats, sample_rows, to_device, to_host

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


MERGE_CASES = [
    # (R, D, dtype, n)
    (65, 4096, "bf16", 1), (65, 4096, "bf16", 3), (37, 7168, "bf16", 5), (130, 1000, "bf16", 9),
    (1, 8, "bf16", 2), (300, 520, "bf16", 17), (65, 4096, "f32", 4),
]


@pytest.mark.parametrize("R,D,dtype,n", MERGE_CASES)
def test_merge_sources(R, D, dtype, n):
    announce(f"merge R={R} D={D} {dtype} n={n}")
    rows = np.arange(R)
    o = inputs.tensor_rows(61, inputs.ROLE_AUX, 1, rows, D, 1.0, dtype)
    srcs = [inputs.tensor_rows(61, inputs.ROLE_SRC, i, rows, D, 0.5 + i, dtype) for i in range(n)]
    lse = (2.0 * inputs.normal(61, inputs.ROLE_AUX, 4, rows)).astype(np.float32)
    w = inputs.queries(61, 1, D, sigma=0.3 / math.sqrt(D / 64))[0]
    g = inputs.gains(61, D)
    m_out = torch.empty(R, dtype=torch.float32, device="cuda")
    lse_out = torch.empty(R, dtype=torch.float32, device="cuda")
    out, _, _ = b.attnres_merge_sources(to_device(o), torch.from_numpy(lse).cuda(),
                                        [to_device(a) for a in srcs], torch.from_numpy(w).cuda(),
                                        gamma=torch.from_numpy(g).cuda(), eps=EPS, m_out=m_out,
                                        lse_out=lse_out)
    torch.cuda.synchronize()
    ref = oracle.merge(o, lse, srcs, w, g, eps=EPS)
    assert_close_scaled(to_host(out), ref["h"], ref["scale"], dtype, "merge h")
    assert_stats(to_host(lse_out), ref["lse"], "merge lse")
    assert_stats(to_host(m_out), ref["m"], "merge m")


FULL_CASES = [
    # (name, L, C, B, T, D, dtype): C = 1 is the naive schedule; ragged last
    # chunks; a chunk whose Phase 1 sees 16 sources (vector-ALU limit) and one
    # that sees 17 (per-query aggregates)
    ("full_L16_C4", 16, 4, 4, 512, 1024, "bf16"),
    ("full_L7_C3_f32", 7, 3, 1, 5, 64, "f32"),
    ("full_L10_C4", 10, 4, 2, 150, 1024, "bf16"),
    ("full_L20_C5", 20, 5, 1, 64, 512, "bf16"),
    ("full_L24_C8", 24, 8, 1, 40, 256, "bf16"),
    ("full_L9_C1", 9, 1, 1, 50, 256, "bf16"),
    ("full_L5_C16", 5, 16, 1, 33, 128, "bf16"),
    ("full_L12_C4_gains", 12, 4, 2, 100, 1024, "bf16"),
    # at least 4096 rows: chunks of 9..16 sources on the matrix-core scores
    # pass and the packed outputs pass (odd query counts included), beside
    # the register-tile Phase 1 for the first chunks; D = 7168 takes the
    # scores pass for every chunk
    ("full_L16_C4_scores", 16, 4, 1, 4100, 1024, "bf16"),
    ("full_L20_C5_scores_gains", 20, 5, 1, 4096, 2048, "bf16"),
    ("full_L12_C3_D7168", 12, 3, 1, 4096, 7168, "bf16"),
]


@pytest.mark.parametrize("name,L,C,B,T,D,dtype", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_full_two_phase_matches_naive(name, L, C, B, T, D, dtype):
    announce(name)
    wl = inputs.Workload(name, "stack", B=B, T=T, D=D, dtype=dtype, L=L, S=1, seed=L * 10 + C)
    ds = DeviceStack(wl, gains=name.endswith("_gains"))
    rows = np.arange(wl.R)
    rec = ds.recorder(rows)
    y = b.attnres_full_stack_forward(ds.x, ds.W, C, rec, Gamma=ds.Gamma, eps=EPS)
    torch.cuda.synchronize()
    xr, vr = ds.host_rows(rows)
    for c0 in range(0, wl.R, 512):
        sl = slice(c0, c0 + 512)
        ref = oracle.block_stack(xr[sl], [a[sl] for a in vr], ds.W_host, 1, Gamma=ds.Gamma_host, eps=EPS)
        recs = to_host(ds.rec[:, sl])
        for l in range(L):
            assert_close_scaled(recs[l], ref["h"][l], ref["h_scale"][l], dtype, f"{name} h_{l + 1}")
        assert_close_scaled(to_host(y[sl]), ref["y"], ref["y_scale"], dtype, f"{name} y")
        assert np.array_equal(recs[0], xr[sl]), "h_1 must equal the embedding bit for bit"


@pytest.mark.parametrize("C", [4, 8])
def test_full_schedule_benchmark_shape(C):
    """The Full two-phase schedule at the benchmark's shape and launch
    configuration (16384 rows of 4096, L = 16, bf16; schedule block sizes 4 and
    8, the measured ones): 128 sampled rows of every h_l and y against the
    oracle's naive Full forward."""
    wl = inputs.WORKLOADS["full_L16_D4096"]
    name = f"{wl.name}_C{C}"
    announce(name)
    ds = DeviceStack(wl)
    rows = sample_rows(wl.R, 128, seed=C)
    rec = ds.recorder(rows)
    y = b.attnres_full_stack_forward(ds.x, ds.W, C, rec, Gamma=ds.Gamma, eps=EPS)
    torch.cuda.synchronize()
    xr, vr = ds.host_rows(rows)
    ref = oracle.block_stack(xr, vr, ds.W_host, 1, Gamma=ds.Gamma_host, eps=EPS)
    recs = to_host(ds.rec)
    for l in range(wl.L):
        assert_close_scaled(recs[l], ref["h"][l], ref["h_scale"][l], wl.dtype, f"{name} h_{l + 1}")
    ids = torch.from_numpy(rows).to("cuda")
    assert_close_scaled(to_host(y[ids]), ref["y"], ref["y_scale"], wl.dtype, f"{name} y")
    assert np.array_equal(recs[0], xr), "h_1 must equal the embedding bit for bit"
    del ds, y
    torch.cuda.empty_cache()
