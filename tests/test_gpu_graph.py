"""The stack forward captured into a HIP graph (through torch.cuda.graph) and
replayed: every replay must reproduce the eager forward bit for bit.

The forward enqueues kernels only (no allocation, synchronisation or memset),
so it is capturable as a whole; the decode regime (few token rows, many
sublayers) is launch-bound and is the case a graph is for. Replays alternate
with eager work and host synchronisations, and each is checked.
"""
import numpy as np
import pytest
import torch

from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from depth_wise_attention_rms_amd.workload import DeviceStack
from tests.parity import to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()
    inputs.lib()
    yield
    torch.cuda.synchronize()


GRAPH_CASES = [
    inputs.WORKLOADS["decode_L96_S12"],
    inputs.Workload("graph_block", "stack", B=2, T=64, D=1024, dtype="bf16", L=16, S=4, seed=9),
    inputs.Workload("graph_full", "stack", B=1, T=32, D=256, dtype="bf16", L=5, S=1, seed=10),
    # 4096 rows of 7168 with 12 queries: Phase 1 as the query split, the
    # matrix-core scores pass and the outputs pass, with a separate close
    inputs.Workload("graph_gemm", "stack", B=1, T=4096, D=7168, dtype="bf16", L=15, S=12, seed=11),
]


@pytest.mark.parametrize("wl", GRAPH_CASES, ids=[w.name for w in GRAPH_CASES])
@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
def test_stack_graph_replay_matches_eager(wl, norm):
    print(f"[gpu-case] graph {wl.name} norm={norm}", flush=True)
    ds = DeviceStack(wl)
    nrm = None
    if norm:
        Gf = np.stack([inputs.gains(wl.seed + 100, wl.D, layer=l) for l in range(wl.L)]).astype(np.float32)
        nrm = (torch.from_numpy(Gf).cuda(), 1e-6)
    ds.forward(norm=nrm)
    torch.cuda.synchronize()
    y_ref = to_host(ds.y)
    bs_ref = None if ds.block_sums is None else [to_host(t) for t in ds.block_sums]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ds.forward(stream=side, norm=nrm)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.forward(stream=torch.cuda.current_stream(), norm=nrm)
    torch.cuda.synchronize()

    for rep in range(3):
        ds.y.zero_()
        if ds.block_sums is not None:
            for t in ds.block_sums:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ds.y), y_ref), f"replay {rep}: y differs from eager"
        if bs_ref is not None:
            for k, t in enumerate(ds.block_sums):
                assert np.array_equal(to_host(t), bs_ref[k]), f"replay {rep}: b_{k + 1} differs"
        ds.forward(norm=nrm)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ds.y), y_ref), f"eager after replay {rep} differs"
