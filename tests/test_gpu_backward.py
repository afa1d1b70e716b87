"""GPU parity of the aggregate backward (attnres_aggregate_backward) against
the oracle's fp64 gradients on the same inputs.

Tolerance. The gradients are fp32 results of fp32 arithmetic on exactly
widened inputs, so the bar is the fp32 one, 1e-5, relative to a condition
scale built from magnitudes (numpy, fp64, from the inputs alone):
  |g|_i   = sum_d |dh_d V_id|          (magnitude behind g_i = dh . V_i)
  S_i     = sum_d |q~_d V_id| / r_i    (magnitude behind the score s_i)
  DS_i    = |ds_i| + a_i (|g|_i + sum_j a_j |g|_j)
            + 2 a_i (|g_i| + 2 sum_j a_j |g_j|) max_j S_j
            (rounding of g, and of the scores through the softmax)
  dV_i[d] : a_i |dh_d| + DS_i (|q~_d| / r_i + |s_i| |V_id| / (D r_i^2))
  dq~[d]  : sum_rows sum_i DS_i |V_id| / r_i;  dw: * |gamma|, dgamma: * |w|
A rounding error of u per operation, summed over the at most ~100 sequential
steps of any of these sums, stays well below 1e-5 of the scale.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs
from tests.bwd_scale import bwd_scales
from tests.parity import to_device, to_host, widen

pytestmark = pytest.mark.gpu

TOL = 1e-5


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


def scaled_err(got, ref, scale):
    diff = np.abs(got.astype(np.float64) - ref)
    zero = scale == 0
    assert not np.any(diff[zero]), "nonzero where the scale is zero"
    return float(np.max(diff[~zero] / scale[~zero], initial=0.0))


def make_case(seed, R, D, dtype, n, with_gamma, sigma=0.3):
    rows = np.arange(R)
    srcs = [inputs.tensor_rows(seed, inputs.ROLE_SRC, i, rows, D, 0.5 + 0.37 * i, dtype) for i in range(n)]
    dh = inputs.tensor_rows(seed, inputs.ROLE_AUX, 9, rows, D, 1.0, dtype)
    w = inputs.queries(seed, 1, D, sigma=sigma / math.sqrt(max(D, 64) / 64))[0]
    g = inputs.gains(seed, D) if with_gamma else None
    return srcs, dh, w, g


def host_values(a, dtype):
    return widen(a) if dtype == "bf16" else a.astype(np.float64)


def check_backward(srcs, dh, w, g, eps, dtype, dV, dw, dgamma, base=None, what=""):
    """Compare GPU gradients with the oracle's (plus `base`, the values the
    GPU accumulated onto, when given)."""
    ref = oracle.aggregate_backward(srcs, w, dh, g, eps=eps)
    V = np.stack([host_values(a, dtype) for a in srcs])
    q = (w * g).astype(np.float32).astype(np.float64) if g is not None else w.astype(np.float64)
    sc_dV, sc_dq = bwd_scales(V, q, host_values(dh, dtype), eps)
    ref_dV, ref_dw = ref["dV"], ref["dw"]
    ref_dg = ref["dgamma"] if g is not None else None
    if base is not None:
        ref_dV = ref_dV + base["dV"]
        ref_dw = ref_dw + base["dw"]
        if ref_dg is not None:
            ref_dg = ref_dg + base["dgamma"]
        # accumulating adds one rounding of the sum
        sc_dV = sc_dV + np.abs(base["dV"]) * 2 ** -23 / TOL
    worst = 0.0
    for i in range(len(srcs)):
        e = scaled_err(to_host(dV[i]), ref_dV[i], sc_dV[i])
        assert e <= TOL, f"{what} dV[{i}] scaled error {e:.3e}"
        worst = max(worst, e)
    gam = np.abs(g.astype(np.float64)) if g is not None else np.ones_like(sc_dq)
    sc_dw = sc_dq * gam + (np.abs(base["dw"]) * 2 ** -23 / TOL if base is not None else 0)
    e = scaled_err(to_host(dw), ref_dw, sc_dw)
    assert e <= TOL, f"{what} dw scaled error {e:.3e}"
    if ref_dg is not None:
        sc_dg = sc_dq * np.abs(w.astype(np.float64)) + (
            np.abs(base["dgamma"]) * 2 ** -23 / TOL if base is not None else 0)
        e = scaled_err(to_host(dgamma), ref_dg, sc_dg)
        assert e <= TOL, f"{what} dgamma scaled error {e:.3e}"
    return worst


BWD_CASES = [
    # (R, D, dtype, n, gamma, eps): resident groups of 2/4/8/16 sources, the
    # streamed form (n > 16; wide rows with n > 4), ragged rows (D = 1000),
    # several waves per row (D = 7168: 7 waves), four vectors per lane
    # (bf16 D = 16384, fp32 D = 8192), tiny rows, and a grid that exceeds the
    # workgroup cap (R = 5000 rows of D = 256: 4 rows per workgroup)
    (65, 4096, "bf16", 8, True, 1e-6),
    (65, 4096, "bf16", 1, True, 1e-6),
    (33, 4096, "bf16", 2, False, 1e-8),
    (40, 1000, "bf16", 3, True, 1e-6),
    (37, 7168, "bf16", 5, True, 1e-6),
    (20, 2048, "bf16", 13, True, 1e-6),
    (20, 1024, "bf16", 16, True, 1e-6),
    (17, 1024, "bf16", 17, True, 1e-6),
    (9, 512, "bf16", 40, True, 1e-6),
    (5, 16384, "bf16", 3, True, 1e-6),
    (5, 16384, "bf16", 7, True, 1e-6),
    (1, 8, "bf16", 3, True, 0.5),
    (5000, 256, "bf16", 3, True, 1e-6),
    (65, 4096, "f32", 6, True, 1e-6),
    (9, 8192, "f32", 5, False, 1e-6),
    (30, 4, "f32", 2, True, 1e-3),
]


@pytest.mark.parametrize("R,D,dtype,n,with_gamma,eps", BWD_CASES)
def test_backward_matches_oracle(R, D, dtype, n, with_gamma, eps):
    announce(f"backward R={R} D={D} {dtype} n={n} gamma={with_gamma} eps={eps}")
    srcs, dh, w, g = make_case(R + n, R, D, dtype, n, with_gamma)
    dV, dw, dgamma = b.attnres_aggregate_backward(
        [to_device(a) for a in srcs], torch.from_numpy(w).cuda(), to_device(dh),
        gamma=None if g is None else torch.from_numpy(g).cuda(), eps=eps)
    torch.cuda.synchronize()
    check_backward(srcs, dh, w, g, eps, dtype, dV, dw, dgamma, what=f"n={n} D={D}")


def test_backward_single_source_is_identity():
    """One source: dV = dh exactly (widened), and the query gets no gradient."""
    announce("backward n=1 exact")
    srcs, dh, w, g = make_case(5, 30, 1024, "bf16", 1, True)
    dV, dw, dgamma = b.attnres_aggregate_backward(
        [to_device(srcs[0])], torch.from_numpy(w).cuda(), to_device(dh),
        gamma=torch.from_numpy(g).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dV[0]).astype(np.float64), widen(dh))
    assert not np.any(to_host(dw)) and not np.any(to_host(dgamma))


@pytest.mark.parametrize("n", [4, 20])
def test_backward_accumulate(n):
    """accumulate != 0 adds to dV, dw and dgamma; two calls in a row with
    different inputs sum both gradients; the result is deterministic."""
    announce(f"backward accumulate n={n}")
    R, D = 50, 1024
    srcs, dh, w, g = make_case(71, R, D, "bf16", n, True)
    rng = np.random.default_rng(3)
    base = {"dV": rng.standard_normal((n, R, D)).astype(np.float32),
            "dw": rng.standard_normal(D).astype(np.float32),
            "dgamma": rng.standard_normal(D).astype(np.float32)}
    dV = [torch.from_numpy(base["dV"][i].copy()).cuda() for i in range(n)]
    dw = torch.from_numpy(base["dw"].copy()).cuda()
    dgamma = torch.from_numpy(base["dgamma"].copy()).cuda()
    args = ([to_device(a) for a in srcs], torch.from_numpy(w).cuda(), to_device(dh))
    b.attnres_aggregate_backward(*args, gamma=torch.from_numpy(g).cuda(), eps=1e-6, dV=dV, dw=dw,
                                 dgamma=dgamma, accumulate=True)
    torch.cuda.synchronize()
    base64 = {k: v.astype(np.float64) for k, v in base.items()}
    check_backward(srcs, dh, w, g, 1e-6, "bf16", dV, dw, dgamma, base=base64, what="accumulate")
    # determinism: a fresh (non-accumulating) call twice gives identical bits
    o1 = b.attnres_aggregate_backward(*args, gamma=torch.from_numpy(g).cuda(), eps=1e-6)
    o2 = b.attnres_aggregate_backward(*args, gamma=torch.from_numpy(g).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    for x, y in zip(o1[0] + [o1[1], o1[2]], o2[0] + [o2[1], o2[2]]):
        assert torch.equal(x, y), "the backward must be deterministic"


def test_backward_large_rows_sampled():
    """The bench-scale shape (R = 16384 rows of D = 4096, n = 8): every dV row
    of a sample against the oracle on those rows; dw and dgamma, sums over
    all rows, against the oracle on all rows is too slow, so they are checked
    for the sampled rows by a second call restricted to those rows."""
    announce("backward R=16384 D=4096 n=8 sampled rows")
    R, D, n = 16384, 4096, 8
    wl_seed = 29
    w = inputs.queries(wl_seed, 1, D, sigma=0.3 / math.sqrt(D / 64))[0]
    g = inputs.gains(wl_seed, D)
    def dev(role, layer, scale):
        t = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        return inputs.fill_normal(t, wl_seed, role, layer, scale)

    dev_src = [dev(inputs.ROLE_SRC, i, 0.5 + 0.37 * i) for i in range(n)]
    dev_dh = dev(inputs.ROLE_AUX, 9, 1.0)
    wt, gt = torch.from_numpy(w).cuda(), torch.from_numpy(g).cuda()
    dV, dw, dgamma = b.attnres_aggregate_backward(dev_src, wt, dev_dh, gamma=gt, eps=1e-6)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(1).integers(0, R, 14)]))
    srcs = [inputs.tensor_rows(wl_seed, inputs.ROLE_SRC, i, rows, D, 0.5 + 0.37 * i, "bf16")
            for i in range(n)]
    dh = inputs.tensor_rows(wl_seed, inputs.ROLE_AUX, 9, rows, D, 1.0, "bf16")
    idx = torch.from_numpy(rows).cuda()
    dV_rows = [t.index_select(0, idx) for t in dV]
    # the host copies must be the rows the GPU used
    for i in range(n):
        assert np.array_equal(to_host(dev_src[i].index_select(0, idx)), srcs[i])
    # dw / dgamma for the sampled rows only, through a call on those rows
    sub = b.attnres_aggregate_backward([s.index_select(0, idx) for s in dev_src], wt,
                                       dev_dh.index_select(0, idx), gamma=gt, eps=1e-6)
    torch.cuda.synchronize()
    check_backward(srcs, dh, w, g, 1e-6, "bf16", dV_rows, sub[1], sub[2], what="R=16384 rows")
    # and the full-R dw is the column sum: finite and deterministic
    again = b.attnres_aggregate_backward(dev_src, wt, dev_dh, gamma=gt, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(again[1], dw) and torch.equal(again[2], dgamma)
    assert torch.isfinite(dw).all()


def test_backward_edge_cases_and_validation():
    announce("backward edge cases")
    D = 256
    w = torch.zeros(D, dtype=torch.float32, device="cuda")
    dw = torch.full((D,), 7.0, device="cuda")
    dg = torch.full((D,), 7.0, device="cuda")
    empty = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    # R = 0: dw and dgamma are zeroed, or left as they are when accumulating
    b.attnres_aggregate_backward([empty, empty], w, empty, dV=[torch.empty((0, D), device="cuda")] * 2,
                                 dw=dw, dgamma=dg)
    torch.cuda.synchronize()
    assert not torch.any(dw) and not torch.any(dg)
    dw.fill_(7.0)
    b.attnres_aggregate_backward([empty], w, empty, dV=[torch.empty((0, D), device="cuda")], dw=dw,
                                 accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dw == 7.0)
    x = torch.randn((4, D), device="cuda").to(torch.bfloat16)
    dV = [torch.empty((4, D), device="cuda") for _ in range(2)]
    with pytest.raises(b.AttnResError):  # dV aliasing each other
        b.attnres_aggregate_backward([x, x], w, x, dV=[dV[0], dV[0]], dw=dw)
    with pytest.raises(b.AttnResError):  # workspace too small
        b.attnres_aggregate_backward([x, x], w, x, dV=dV, dw=dw,
                                     workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    rc = b.lib().attnres_aggregate_backward(None, 0, 4, D, 1, b._ptr(w), None, 1e-6, b._ptr(x), None,
                                            0, b._ptr(dw), None, None, 0, None)
    assert rc == -1, "n = 0 must be rejected"
