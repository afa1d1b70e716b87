"""GPU parity of the decode schedule (attnres_block_stack_forward_overlap):
each block's Phase 1 runs on a side stream during the previous block, over
the sources that exist when that block starts, and the block sum the previous
block closes with joins later as one more single-source term (K3 course notes
section 9.4, eq. OS2: the merge of source groups is exact).

Every h_l, y and block sum is compared with the oracle's naive forward (the
same rule as every stack test: scaled error <= 1e-2 for bf16 and 1e-5 for
fp32, block sums bit-exact). y and the block sums must also equal the plain
forward's bit for bit: the final aggregate and the closes do not depend on
the schedule. Graph capture of both streams is replayed and checked.
"""
import numpy as np
import pytest
import torch

from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from depth_wise_attention_rms_amd.workload import EPS, DeviceStack
from tests.parity import sample_rows, to_host
from tests.stack_check import check_stack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()
    inputs.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def side():
    return torch.cuda.Stream()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _plain_outputs(ds):
    ds.forward()
    torch.cuda.synchronize()
    return to_host(ds.y), [to_host(t) for t in ds.block_sums]


def _same_as_plain(ds, plain):
    y, bs = plain
    assert np.array_equal(to_host(ds.y), y), "y differs from the plain schedule's"
    for k, t in enumerate(ds.block_sums):
        assert np.array_equal(to_host(t), bs[k]), f"b_{k + 1} differs from the plain schedule's"


def test_overlap_decode_config(side):
    """Decode regime: L = 96, S = 12, 128 rows, D = 7168, bf16; all rows and
    every sublayer."""
    wl = inputs.WORKLOADS["decode_L96_S12"]
    announce(f"overlap {wl.name}")
    ds = DeviceStack(wl)
    plain = _plain_outputs(ds)
    check_stack(ds, np.arange(wl.R), chunk=64, side_stream=side)
    _same_as_plain(ds, plain)


def test_overlap_bruteforce_grid(side):
    """Every L <= 7 and S <= L+1 on 3 rows: one-sublayer blocks (S = 1 and
    short last blocks), first blocks whose Phase 1 sees only the embedding,
    both dtypes, D in {8, 64} (and 1024 for bf16, the matrix-core Phase 1),
    with and without gains."""
    for dtype in ("bf16", "f32"):
        for D in ((8, 64, 1024) if dtype == "bf16" else (8, 64)):
            for L in range(1, 8):
                for S in range(1, L + 2):
                    wl = inputs.Workload(f"ovl_L{L}_S{S}_D{D}_{dtype}", "stack", B=1, T=3, D=D,
                                         dtype=dtype, L=L, S=S, seed=L * 100 + S + 7)
                    ds = DeviceStack(wl, W_host=inputs.queries(L + 3, L + 1, D, sigma=0.4),
                                     gains=(L + S) % 2 == 0)
                    check_stack(ds, np.arange(3), side_stream=side)


OVERLAP_SHAPES = [
    # (B, T, D, S, L, dtype, gains): the streamed Phase 1 with S > 8 at
    # D = 7168 and a one-sublayer last block; the matrix-core Phase 1 with
    # several rows per workgroup; Full (S = 1); fp32
    (1, 40, 7168, 12, 25, "bf16", True),
    (2, 300, 2048, 6, 20, "bf16", False),
    (1, 64, 256, 1, 6, "bf16", True),
    (1, 33, 1024, 5, 13, "f32", True),
]


@pytest.mark.parametrize("B,T,D,S,L,dtype,gains", OVERLAP_SHAPES)
def test_overlap_shapes(side, B, T, D, S, L, dtype, gains):
    wl = inputs.Workload(f"ovl_R{B * T}_D{D}_S{S}_L{L}_{dtype}", "stack", B=B, T=T, D=D, dtype=dtype,
                         L=L, S=S, seed=L + S + D)
    announce(f"overlap {wl.name} gains={gains}")
    ds = DeviceStack(wl, gains=gains)
    check_stack(ds, np.arange(wl.R), chunk=150, side_stream=side)
    y = to_host(ds.y)
    bs = [to_host(t) for t in ds.block_sums]
    ds.forward()
    torch.cuda.synchronize()
    _same_as_plain(ds, (y, bs))


def test_overlap_scores_pass(side):
    """4100 rows of 7168 with 12 queries: the side stream's Phase 1 runs the
    query split, the matrix-core scores pass and the outputs pass; sampled
    rows."""
    wl = inputs.Workload("ovl_gemm", "stack", B=1, T=4100, D=7168, dtype="bf16", L=27, S=12, seed=29)
    announce(f"overlap {wl.name}")
    ds = DeviceStack(wl)
    check_stack(ds, sample_rows(wl.R, 128), chunk=64, side_stream=side)
    del ds
    torch.cuda.empty_cache()


def test_overlap_norm(side):
    """The normed decode schedule: sublayer l receives RMSNorm(h_l) *
    Gamma_f[l-1]; every input against the oracle, y and the block sums
    bit-identical to the plain forward's."""
    wl = inputs.Workload("ovl_norm", "stack", B=4, T=10, D=7168, dtype="bf16", L=30, S=12, seed=31)
    announce(f"overlap {wl.name}")
    ds = DeviceStack(wl)
    plain = _plain_outputs(ds)
    Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
    check_stack(ds, np.arange(wl.R), side_stream=side, norm=(torch.from_numpy(Gf).cuda(), 1e-6))
    _same_as_plain(ds, plain)


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
def test_overlap_graph_replay(norm):
    """The decode workload's overlapped forward captured (both streams) into a
    HIP graph: three replays, with eager forwards and host synchronisations
    between them, each bit-identical to the eager result."""
    wl = inputs.WORKLOADS["decode_L96_S12"]
    announce(f"overlap graph {wl.name} norm={norm}")
    ds = DeviceStack(wl)
    nrm = None
    if norm:
        Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
        nrm = (torch.from_numpy(Gf).cuda(), 1e-6)
    side = torch.cuda.Stream()
    rows = np.arange(wl.R)
    rec_fn = ds.recorder(rows)
    ds.forward(rec_fn, norm=nrm, side_stream=side)
    torch.cuda.synchronize()
    y_ref = to_host(ds.y)
    rec_ref = to_host(ds.rec)
    bs_ref = [to_host(t) for t in ds.block_sums]

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ds.forward(rec_fn, stream=cap, norm=nrm, side_stream=side)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.forward(rec_fn, stream=torch.cuda.current_stream(), norm=nrm, side_stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.y.zero_()
        ds.rec.zero_()
        for t in ds.block_sums:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ds.y), y_ref), f"replay {rep}: y differs from eager"
        assert np.array_equal(to_host(ds.rec), rec_ref), f"replay {rep}: a sublayer input differs"
        for k, t in enumerate(ds.block_sums):
            assert np.array_equal(to_host(t), bs_ref[k]), f"replay {rep}: b_{k + 1} differs"
        ds.forward(rec_fn, norm=nrm, side_stream=side)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ds.y), y_ref), f"eager after replay {rep} differs"


def test_overlap_rejects_bad_streams():
    wl = inputs.Workload("ovl_small", "stack", B=1, T=5, D=64, dtype="bf16", L=6, S=3, seed=3)
    announce("overlap argument checks")
    ds = DeviceStack(wl)
    cur = torch.cuda.current_stream()
    with pytest.raises(b.AttnResError) as e:
        ds.forward(side_stream=cur, stream=cur)
    assert e.value.code == -1 and "side_stream" in e.value.detail
    torch.cuda.synchronize()
