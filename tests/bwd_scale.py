"""The condition scale of the aggregate backward's parity bar.

The gradients are fp32 results of fp32 arithmetic on exactly widened inputs,
so they are compared at the fp32 bar, 1e-5, relative to a scale built from
magnitudes (fp64, from the inputs alone):
  |g|_i   = sum_d |dh_d V_id|          (magnitude behind g_i = dh . V_i)
  S_i     = sum_d |q~_d V_id| / r_i    (magnitude behind the score s_i)
  DS_i    = |ds_i| + a_i (|g|_i + sum_j a_j |g|_j)
            + 2 a_i (|g_i| + 2 sum_j a_j |g_j|) max_j S_j
            (rounding of g, and of the scores through the softmax)
  dV_i[d] : a_i |dh_d| + DS_i (|q~_d| / r_i + |s_i| |V_id| / (D r_i^2))
  dq~[d]  : sum_rows sum_i DS_i |V_id| / r_i;  dw: * |gamma|, dgamma: * |w|
A rounding error of u per operation, summed over the at most ~100 sequential
steps of any of these sums, stays well below 1e-5 of the scale.
tests/test_backward_tolerance.py checks both directions on the CPU: an fp32
evaluation passes, planted mistakes fail.
"""
import numpy as np


def bwd_scales(V, q, dh, eps):
    """Condition scales of dV [n,R,D], dq~ [D] for fp64 V [n,R,D], q [D], dh [R,D]."""
    D = V.shape[-1]
    r = np.sqrt((V * V).mean(-1) + eps)                     # [n,R]
    s = (V @ q) / r
    a = np.exp(s - s.max(0)); a /= a.sum(0)
    g = (V * dh[None]).sum(-1)
    ds = a * (g - (a * g).sum(0))
    gmag = (np.abs(V) * np.abs(dh)[None]).sum(-1)
    smag = (np.abs(V) @ np.abs(q)) / r
    DS = (np.abs(ds) + a * (gmag + (a * gmag).sum(0))
          + 2 * a * (np.abs(g) + 2 * (a * np.abs(g)).sum(0)) * smag.max(0))
    sc_dV = (a[..., None] * np.abs(dh)[None]
             + DS[..., None] * (np.abs(q)[None, None] / r[..., None]
                                + np.abs(s)[..., None] * np.abs(V) / (D * r[..., None] ** 2)))
    sc_dq = (DS[..., None] * np.abs(V) / r[..., None]).sum((0, 1))
    return sc_dV, sc_dq
