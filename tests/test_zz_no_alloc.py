"""The no-allocation aggregate backward (attnres_aggregate_backward_noalloc)
against the workspace entry point (attnres_aggregate_backward) it shares its
kernels with, through the C ABI.

Both run the same kernels with the same launch plan, and the backward's sum
over rows runs in a fixed order, so the results must agree bit for bit. Two
calls in a row share the library's fixed scratch: the second, smaller call
must not see anything the first one left there.
"""
import math

import numpy as np
import pytest
import torch

from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()
    inputs.lib()
    yield
    torch.cuda.synchronize()


def _case(seed, R, D, dtype, n, with_gamma):
    rows = np.arange(R)
    srcs = [inputs.tensor_rows(seed, inputs.ROLE_SRC, i, rows, D, 0.5 + 0.37 * i, dtype) for i in range(n)]
    dh = inputs.tensor_rows(seed, inputs.ROLE_AUX, 9, rows, D, 1.0, dtype)
    w = inputs.queries(seed, 1, D, sigma=0.3 / math.sqrt(max(D, 64) / 64))[0]
    g = inputs.gains(seed, D) if with_gamma else None
    dev = torch.device("cuda:0")
    to = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if dtype == "bf16":
        tod = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        tod = to
    return [tod(s) for s in srcs], tod(dh), to(w), to(g)


def _run_both(srcs, dh, w, g, accumulate):
    dev = dh.device
    R, D = dh.shape
    n = len(srcs)
    seed_dv = [torch.full((R, D), 0.25 * (i + 1), dtype=torch.float32, device=dev) for i in range(n)]
    seed_dw = torch.full((D,), -0.5, dtype=torch.float32, device=dev)
    outs = []
    for noalloc in (False, True):
        dV = [t.clone() for t in seed_dv]
        dw = seed_dw.clone()
        dg = seed_dw.clone() if g is not None else None
        if noalloc:
            b.attnres_aggregate_backward_noalloc(srcs, w, dh, dV, dw, gamma=g, dgamma=dg,
                                                 accumulate=accumulate)
        else:
            b.attnres_aggregate_backward(srcs, w, dh, gamma=g, dV=dV, dw=dw, dgamma=dg,
                                         accumulate=accumulate)
        torch.cuda.synchronize()
        outs.append((dV, dw, dg))
    return outs


def _assert_same(ref, got, what):
    for i, (a, c) in enumerate(zip(ref[0], got[0])):
        assert torch.equal(a, c), f"{what}: dV[{i}] differs"
    assert torch.equal(ref[1], got[1]), f"{what}: dw differs"
    if ref[2] is not None:
        assert torch.equal(ref[2], got[2]), f"{what}: dgamma differs"


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 5000 rows of 4096 bf16, 7 sources -- a grid at its
    # workgroup cap with a two-stage row sum, so the scratch fills widely
    print("[gpu-case] noalloc backward R=5000 D=4096 bf16 n=7", flush=True)
    big = _case(71, 5000, 4096, "bf16", 7, with_gamma=False)
    ref, got = _run_both(*big, accumulate=False)
    _assert_same(ref, got, "first call")
    assert torch.count_nonzero(ref[1]) > 0
    # second call, smaller: 300 rows of 1024 fp32, 3 sources, with a gain and
    # accumulation into seeded gradients
    print("[gpu-case] noalloc backward R=300 D=1024 f32 n=3 accumulate", flush=True)
    small = _case(72, 300, 1024, "f32", 3, with_gamma=True)
    ref, got = _run_both(*small, accumulate=True)
    _assert_same(ref, got, "second call")


def test_noalloc_rejects_rows_beyond_the_scratch():
    print("[gpu-case] noalloc backward rejects bf16 R=4096 D=8200", flush=True)
    dev = torch.device("cuda:0")
    R, D = 4096, 8200
    srcs = [torch.zeros((R, D), dtype=torch.bfloat16, device=dev)]
    dV = [torch.zeros((R, D), dtype=torch.float32, device=dev)]
    dw = torch.zeros(D, dtype=torch.float32, device=dev)
    w = torch.zeros(D, dtype=torch.float32, device=dev)
    with pytest.raises(b.AttnResError) as e:
        b.attnres_aggregate_backward_noalloc(srcs, w, srcs[0], dV, dw)
    assert e.value.code == -2 and "scratch" in e.value.detail
