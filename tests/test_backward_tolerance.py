"""The aggregate backward's parity bar (tests/bwd_scale.py) checked in both
directions on the CPU, against the fp64 oracle:

- not too tight: an independent fp32 evaluation of the gradient formula
  (numpy float32, its own summation order) stays within 1e-5 of the scale;
- not too loose: the same evaluation with one planted mistake -- a dropped
  term, an uncentred softmax Jacobian, a missing 1/r, scores on raw sources,
  the gain where w belongs, eps dropped -- fails it by orders of magnitude.

So a GPU backward that passes the bar has none of these mistakes.
"""
import numpy as np
import pytest

import oracle
from tests.bwd_scale import bwd_scales
from tests.oracle_pins import bf16_normal, bf16_to_f64

TOL = 1e-5


def _case(eps):
    rng = np.random.default_rng(91)
    n, rows, D = 5, 48, 512
    V = [bf16_normal(rng, (rows, D), s) for s in (1.0, 3.0, 0.4, 2.0, 0.8)]
    dh = bf16_normal(rng, (rows, D), 1.0)
    w = (rng.standard_normal(D) * 0.3 / np.sqrt(D / 64)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return V, dh, w, g, eps


def _fp32_backward(V, dh, w, g, eps, mistake=None):
    """dV [n, rows, D], dw [D], dgamma [D] in float32 arithmetic."""
    f = np.float32
    Vf = np.stack([bf16_to_f64(a).astype(f) for a in V])
    dhf = bf16_to_f64(dh).astype(f)
    q = (w * g).astype(f)
    D = Vf.shape[-1]
    ms = (Vf * Vf).mean(-1, dtype=f)
    r = np.sqrt(ms + (f(0) if mistake == "eps_dropped" else f(eps))).astype(f)
    dot = (Vf @ q).astype(f)
    s = dot if mistake == "scores_on_raw" else (dot / r).astype(f)
    a = np.exp(s - s.max(0)).astype(f)
    a = (a / a.sum(0, dtype=f)).astype(f)
    gi = (Vf * dhf[None]).sum(-1, dtype=f)
    gh = (a * gi).sum(0, dtype=f)
    ds = (a * gi) if mistake == "uncentred_softmax" else (a * (gi - gh)).astype(f)
    rms_term = (s / (f(D) * r * r))[..., None] * Vf
    if mistake == "drop_rms_term":
        rms_term = np.zeros_like(rms_term)
    dV = a[..., None] * dhf[None] + ds[..., None] * (q[None, None] / r[..., None] - rms_term)
    dq_rows = (ds / (f(1) if mistake == "dq_raw_sources" else r))[..., None] * Vf
    dq = dq_rows.sum((0, 1), dtype=f)
    dw = dq * (w if mistake == "dw_takes_w" else g)
    dgamma = dq * w
    return dV.astype(np.float64), dw.astype(np.float64), dgamma.astype(np.float64)


def _worst(V, dh, w, g, eps, got):
    ref = oracle.aggregate_backward(V, w, dh, g, eps=eps)
    Vd = np.stack([bf16_to_f64(a) for a in V])
    q = (w * g).astype(np.float32).astype(np.float64)
    sc_dV, sc_dq = bwd_scales(Vd, q, bf16_to_f64(dh), eps)
    errs = [np.max(np.abs(got[0] - ref["dV"]) / sc_dV),
            np.max(np.abs(got[1] - ref["dw"]) / (sc_dq * np.abs(g.astype(np.float64)))),
            np.max(np.abs(got[2] - ref["dgamma"]) / (sc_dq * np.abs(w.astype(np.float64))))]
    return max(errs)


@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_fp32_evaluation_passes(eps):
    V, dh, w, g, eps = _case(eps)
    worst = _worst(V, dh, w, g, eps, _fp32_backward(V, dh, w, g, eps))
    assert worst <= TOL, f"an fp32 evaluation fails the bar: {worst:.3e}"


@pytest.mark.parametrize("mistake,eps", [
    ("drop_rms_term", 1e-6), ("uncentred_softmax", 1e-6), ("dq_raw_sources", 1e-6),
    ("scores_on_raw", 1e-6), ("dw_takes_w", 1e-6), ("eps_dropped", 0.25),
])
def test_planted_mistake_fails(mistake, eps):
    V, dh, w, g, eps = _case(eps)
    worst = _worst(V, dh, w, g, eps, _fp32_backward(V, dh, w, g, eps, mistake))
    assert worst > 100 * TOL, f"the bar lets {mistake} pass (worst scaled error {worst:.3e})"
