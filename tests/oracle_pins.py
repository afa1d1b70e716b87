"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes a loaded oracle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with a closed form, an invariant, a
special case, a value printed on the pages or a brute-force check. The same
pins run against deliberately mutated oracle builds in
``test_oracle_pins.py``: every planted mistake must trip at least one of them.

Pages cited: K3 course notes, section "Attention Residual 深度残差" (K3 §9.x);
"Attention Residuals" survey page on wineandchord.com (WC, by section name).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# small helpers (no method arithmetic beyond what each pin states)
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_via_torch(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, rounded by torch (nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_normal(rng, shape, sigma=1.0) -> np.ndarray:
    return f64_to_bf16_via_torch((rng.standard_normal(shape) * sigma).astype(np.float32))


def widen(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def os2_merge(a, b):
    """Merge two group summaries given as (lse, o): log-sum-exp lse of the
    group's scores and its normalised output o (K3 §9.4 eq. OS2, here with each
    group's denominator folded into lse). The merged lse is the log-add-exp of
    the two; each group's share of the merged softmax mass is e^(lse_g - lse)."""
    lse = np.logaddexp(a[0], b[0])
    wa, wb = np.exp(a[0] - lse), np.exp(b[0] - lse)
    return lse, wa[..., None] * a[1] + wb[..., None] * b[1]


def summary_of(out):
    """(lse, o) of an oracle aggregate."""
    return out["lse"], out["h"]


# ----------------------------------------------------------------------------
# rounding
# ----------------------------------------------------------------------------

def pin_round_bf16_bruteforce(orc):
    """bf16 rounding is nearest with ties to even: checked against the two
    neighbouring bf16 values of every result, on exact midpoints, and against
    torch's fp32 -> bf16 conversion."""
    rng = np.random.default_rng(11)
    mant = rng.uniform(1.0, 2.0, 4000)
    expo = rng.integers(-140, 120, 4000)
    x = np.ldexp(mant, expo)
    # exact midpoints between consecutive bf16 values (ties)
    base = rng.integers(0x0080, 0x7F00, 2000).astype(np.uint16)
    mid = (bf16_to_f64(base) + bf16_to_f64(base + 1)) / 2.0
    x = np.concatenate([x, mid])
    bits = orc.round_to(x, "bf16").astype(np.int64)
    r = bf16_to_f64(bits.astype(np.uint16))
    up = bf16_to_f64((bits + 1).astype(np.uint16))
    dn = bf16_to_f64(np.maximum(bits - 1, 0).astype(np.uint16))
    err = np.abs(x - r)
    assert np.all(err <= np.abs(x - up)), "bf16 rounding is not nearest (upper neighbour)"
    ok_dn = (bits == 0) | (err <= np.abs(x - dn))
    assert np.all(ok_dn), "bf16 rounding is not nearest (lower neighbour)"
    tie = (err == np.abs(x - up)) | ((bits > 0) & (err == np.abs(x - dn)))
    assert np.all(bits[tie] % 2 == 0), "bf16 ties are not rounded to even"
    assert tie[-2000:].all(), "midpoints should be ties"
    neg = orc.round_to(-x, "bf16").astype(np.int64)
    assert np.array_equal(neg, bits | 0x8000), "bf16 rounding is not sign-symmetric"
    x32 = rng.standard_normal(5000).astype(np.float32) * np.float32(37.0)
    assert np.array_equal(orc.round_to(x32.astype(np.float64), "bf16"), f64_to_bf16_via_torch(x32))


def pin_round_f32(orc):
    """fp32 rounding equals numpy's nearest-even double -> float cast."""
    rng = np.random.default_rng(12)
    x = np.ldexp(rng.uniform(-2, 2, 5000), rng.integers(-100, 100, 5000))
    assert np.array_equal(orc.round_to(x, "f32"), x.astype(np.float32))


# ----------------------------------------------------------------------------
# AGG (eqs. A1-A3)
# ----------------------------------------------------------------------------

def _cfg1_sources(rng, rows=16, D=256):
    sig = (1.0, 3.0, 0.3, 10.0)  # per-source standard deviations of the single-aggregate workload
    return [(rng.standard_normal((rows, D)) * s).astype(np.float32) for s in sig]


def pin_zero_query_is_mean(orc):
    """A zero query gives equal logits, so the output is the plain mean of the
    sources (K3 §9.2 (3); WC reference check with torch.zeros)."""
    rng = np.random.default_rng(1)
    src = _cfg1_sources(rng)
    gamma = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    out = orc.aggregate(src, np.zeros(256, np.float32), gamma, want_alpha=True)
    mean = np.mean([s.astype(np.float64) for s in src], axis=0)
    big = np.max(np.abs([s.astype(np.float64) for s in src]))
    assert np.max(np.abs(out["h"] - mean)) <= 8 * np.finfo(np.float64).eps * big
    assert np.all(out["m"] == 0.0) and np.allclose(out["lse"], math.log(4), rtol=0, atol=1e-15)
    assert np.allclose(out["alpha"], 0.25, rtol=0, atol=1e-16)
    # bf16 sources too
    srcb = [bf16_normal(rng, (8, 64), s) for s in (1.0, 2.0, 0.5)]
    outb = orc.aggregate(srcb, np.zeros(64, np.float32))
    meanb = np.mean([bf16_to_f64(s) for s in srcb], axis=0)
    assert np.max(np.abs(outb["h"] - meanb)) <= 1e-14


def pin_single_source_identity(orc):
    """One source: the softmax weight is exactly 1, so h equals the source bit
    for bit and m = lse = its score (K3 §9.4 single-source triple)."""
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((8, 32)) * 3).astype(np.float32)
    w = (rng.standard_normal(32) * 0.5).astype(np.float32)
    out = orc.aggregate([v], w)
    assert np.array_equal(out["h"], v.astype(np.float64))
    assert np.array_equal(out["m"], out["lse"])
    assert np.array_equal(out["scale"], np.abs(v.astype(np.float64)))


def pin_closed_form_scores(orc):
    """Sources that are scaled one-hot vectors c_i * e_{d_i} have
    mean_d(V^2) = c_i^2 / D, so their RMS-normalised copy is
    sign(c_i) * e_{d_i} / sqrt(c_i^2/D + eps) * |c_i| and the score is
    q[d_i] * c_i / sqrt(c_i^2/D + eps). The softmax over two sources is the
    logistic function of the score difference (A1, A2; WC reference: eps
    inside the root, mean over the hidden axis)."""
    D = 16
    q = np.linspace(-0.9, 1.3, D).astype(np.float32)
    for eps in (0.0, 0.25, 3.0):
        for (c0, d0, c1, d1) in [(2.0, 3, -0.5, 7), (4.0, 0, 4.0, 15), (0.125, 5, 8.0, 5)]:
            V0 = np.zeros((1, D), np.float32); V0[0, d0] = c0
            V1 = np.zeros((1, D), np.float32); V1[0, d1] = c1
            s0 = float(q[d0]) * c0 / math.sqrt(c0 * c0 / D + eps)
            s1 = float(q[d1]) * c1 / math.sqrt(c1 * c1 / D + eps)
            a0 = 1.0 / (1.0 + math.exp(s1 - s0))
            a1 = 1.0 / (1.0 + math.exp(s0 - s1))
            out = orc.aggregate([V0, V1], q, eps=eps, want_alpha=True)
            exp_h = a0 * V0[0].astype(np.float64) + a1 * V1[0].astype(np.float64)
            assert np.allclose(out["h"][0], exp_h, rtol=1e-13, atol=1e-15), (eps, c0, c1)
            assert np.allclose(out["alpha"][0], [a0, a1], rtol=1e-13, atol=0)
            lse = max(s0, s1) + math.log(math.exp(s0 - max(s0, s1)) + math.exp(s1 - max(s0, s1)))
            assert abs(out["lse"][0] - lse) <= 1e-13 * (1 + abs(lse))
            assert abs(out["m"][0] - max(s0, s1)) <= 1e-14 * (1 + abs(lse))
    # the gain folds into the query: gamma scales each hidden coordinate's weight (K3 §9.2 (1))
    V0 = np.zeros((1, D), np.float32); V0[0, 2] = 1.0
    V1 = np.zeros((1, D), np.float32); V1[0, 9] = 1.0
    gamma = np.ones(D, np.float32); gamma[2] = 3.0
    out = orc.aggregate([V0, V1], q, gamma, eps=0.0, want_alpha=True)
    s0, s1 = 3.0 * float(q[2]) * 4.0, float(q[9]) * 4.0
    assert np.allclose(out["alpha"][0], [1 / (1 + math.exp(s1 - s0)), 1 / (1 + math.exp(s0 - s1))],
                       rtol=1e-13)


def pin_scale_invariance(orc):
    """Rescaling a source by c > 0 leaves every score, weight, m and lse
    unchanged: the score reads the direction only (K3 §9.2 (2); WC 'Full
    AttnRes'). Exact at eps = 0; within 1e-6 at eps = 1e-8 for these scales."""
    rng = np.random.default_rng(3)
    src = _cfg1_sources(rng, rows=8, D=64)
    w = (rng.standard_normal(64) * 0.3).astype(np.float32)
    # powers of two rescale exactly (exact invariance at eps = 0); other factors
    # round in fp32, which the looser eps = 1e-8 tolerance absorbs
    for eps, tol, cases in ((0.0, 1e-13, ((0, 2.0), (2, 0.25), (3, 16.0))),
                            (1e-8, 1e-6, ((0, 2.0), (2, 0.37), (3, 11.0)))):
        base = orc.aggregate(src, w, eps=eps, want_alpha=True)
        for j, c in cases:
            mod = list(src)
            mod[j] = (src[j] * np.float32(c)).astype(np.float32)
            out = orc.aggregate(mod, w, eps=eps, want_alpha=True)
            assert np.allclose(out["alpha"], base["alpha"], rtol=tol, atol=tol)
            assert np.allclose(out["lse"], base["lse"], rtol=tol, atol=tol)
            # the output moves only along the rescaled source: h' - h = a_j (c - 1) V_j
            diff = out["h"] - base["h"]
            pred = base["alpha"][:, j:j + 1] * (mod[j].astype(np.float64) - src[j].astype(np.float64))
            vmax = max(np.abs(a).max() for a in mod)
            assert np.allclose(diff, pred, rtol=1e-6, atol=10 * tol * vmax)


def pin_convex_combination(orc):
    """Softmax weights make h a convex combination of the raw sources
    (WC 'Full AttnRes'): min_i V_i <= h <= max_i V_i, weights sum to 1."""
    rng = np.random.default_rng(4)
    src = [bf16_normal(rng, (12, 48), s) for s in (1.0, 5.0, 0.1, 2.0, 0.7)]
    w = (rng.standard_normal(48) * 0.4).astype(np.float32)
    out = orc.aggregate(src, w, want_alpha=True)
    V = np.stack([bf16_to_f64(s) for s in src])
    lo, hi = V.min(0), V.max(0)
    slack = 1e-12 * np.abs(V).max()
    assert np.all(out["h"] >= lo - slack) and np.all(out["h"] <= hi + slack)
    assert np.allclose(out["alpha"].sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(out["alpha"] > 0)
    assert np.all(np.abs(out["h"]) <= out["scale"] + slack)


def pin_permutation(orc):
    """The source order does not matter for h, m or lse (WC validation list:
    source permutation)."""
    rng = np.random.default_rng(5)
    src = [bf16_normal(rng, (6, 40), s) for s in (1.0, 4.0, 0.2, 9.0, 1.5, 0.8)]
    w = (rng.standard_normal(40) * 0.3).astype(np.float32)
    base = orc.aggregate(src, w)
    for perm in ([5, 4, 3, 2, 1, 0], [2, 0, 5, 1, 3, 4]):
        out = orc.aggregate([src[i] for i in perm], w)
        assert np.allclose(out["h"], base["h"], rtol=1e-13, atol=1e-13)
        assert np.allclose(out["lse"], base["lse"], rtol=1e-14, atol=1e-14)
        assert np.array_equal(out["m"], base["m"])


def pin_identical_sources(orc):
    """n identical sources: uniform weights, h = V and lse = s + log n."""
    rng = np.random.default_rng(6)
    v = bf16_normal(rng, (5, 24), 2.0)
    w = (rng.standard_normal(24) * 0.5).astype(np.float32)
    one = orc.aggregate([v], w)
    for n in (2, 3, 7):
        out = orc.aggregate([v] * n, w)
        assert np.allclose(out["h"], bf16_to_f64(v), rtol=1e-15, atol=0)
        assert np.allclose(out["lse"], one["lse"] + math.log(n), rtol=1e-14, atol=1e-14)


def pin_os2_bipartition(orc):
    """Online-softmax summaries of any two disjoint source groups merge into
    the summary of the whole (K3 §9.4 OS1/OS2; WC reference check on 7 sources
    of shape (2, 3, 5) split 3/4, with eps 1e-6). The running max of the whole
    is the larger of the two groups' maxima."""
    rng = np.random.default_rng(0)
    src = [rng.standard_normal((6, 5)).astype(np.float32) for _ in range(7)]
    q = rng.standard_normal(5).astype(np.float32)
    whole = orc.aggregate(src, q, eps=1e-6)
    for k in range(1, 7):
        a = orc.aggregate(src[:k], q, eps=1e-6)
        b = orc.aggregate(src[k:], q, eps=1e-6)
        lse, h = os2_merge(summary_of(a), summary_of(b))
        assert np.allclose(h, whole["h"], rtol=1e-12, atol=1e-12), k
        assert np.allclose(lse, whole["lse"], rtol=1e-13, atol=1e-13), k
        assert np.array_equal(np.maximum(a["m"], b["m"]), whole["m"]), k


# ----------------------------------------------------------------------------
# the condition scale sum_i a_i |V_i[d]| (every parity tolerance divides by it)
# ----------------------------------------------------------------------------

def pin_scale_aggregate_closed_forms(orc):
    """The per-element condition scale of an aggregate is sum_i a_i |V_i[d]|,
    the convex combination (A3) applied to the magnitudes. Three closed forms
    fix it independently of the oracle's own weights:
    - a zero query gives equal weights 1/n, so the scale is mean_i |V_i[d]|
      (K3 §9.2 zero init);
    - two dense sources c_0 * 1 and c_1 * (+1, -1, +1, ...) have mean square
      c_i^2, so their scores are sign(c_i) * (sum_d q[d] sign_i[d]) /
      sqrt(1 + eps / c_i^2) and their weights the logistic function of the
      difference (A1, A2); the scale is a_0 |c_0| + a_1 |c_1| in every element;
    - scaled one-hot sources on distinct coordinates give a_i |c_i| at
      coordinate d_i and zero elsewhere."""
    rng = np.random.default_rng(61)
    src = _cfg1_sources(rng, rows=8, D=64)
    out = orc.aggregate(src, np.zeros(64, np.float32))
    want = np.mean([np.abs(a.astype(np.float64)) for a in src], axis=0)
    big = max(np.abs(a).max() for a in src)
    assert np.max(np.abs(out["scale"] - want)) <= 8 * np.finfo(np.float64).eps * big
    D = 32
    q = np.linspace(-0.4, 0.9, D).astype(np.float32)
    alt = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    for eps in (0.0, 1e-8, 0.5):
        for c0, c1 in ((1.0, 3.0), (-2.0, 0.25), (5.0, -4.0)):
            V0 = np.full((1, D), c0, np.float32)
            V1 = (c1 * alt).astype(np.float32)[None, :]
            s0 = math.copysign(1.0, c0) * float(q.astype(np.float64).sum()) / math.sqrt(1 + eps / c0 ** 2)
            s1 = math.copysign(1.0, c1) * float((q.astype(np.float64) * alt).sum()) / math.sqrt(1 + eps / c1 ** 2)
            a0 = 1.0 / (1.0 + math.exp(s1 - s0))
            a1 = 1.0 / (1.0 + math.exp(s0 - s1))
            got = orc.aggregate([V0, V1], q, eps=eps)["scale"][0]
            np.testing.assert_allclose(got, a0 * abs(c0) + a1 * abs(c1), rtol=1e-12, atol=0)
    V0 = np.zeros((1, D), np.float32); V0[0, 4] = 3.0
    V1 = np.zeros((1, D), np.float32); V1[0, 11] = -0.5
    s0 = float(q[4]) * 3.0 / math.sqrt(9.0 / D)
    s1 = float(q[11]) * -0.5 / math.sqrt(0.25 / D)
    a0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = np.zeros(D); want[4] = a0 * 3.0; want[11] = (1.0 - a0) * 0.5
    np.testing.assert_allclose(orc.aggregate([V0, V1], q, eps=0.0)["scale"][0], want, rtol=1e-12, atol=0)


def pin_scale_phase2_closed_forms(orc):
    """The Phase-2 scale is the merged softmax's weights on |o| and |p|. With
    a zero query the partial scores exactly 0, so a Phase-1 lse of l gives the
    group weight 1/(1 + e^-l) and the partial 1/(1 + e^l) (K3 §9.4 OS2 and the
    single-source triple); lse -200 and +200 leave |p| and |o| alone."""
    rng = np.random.default_rng(62)
    rows, D = 4, 32
    o = (rng.standard_normal((rows, D)) * 2).astype(np.float32)
    v = (rng.standard_normal((rows, D)) * 0.7).astype(np.float32)
    ao, av = np.abs(o.astype(np.float64)), np.abs(v.astype(np.float64))
    zero = np.zeros(D, np.float32)
    for l in (0.0, math.log(3.0), -1.25, 7.0):
        lse = np.full(rows, l, np.float32)
        lf = float(lse[0])
        wo = 1.0 / (1.0 + math.exp(-lf))
        got = orc.phase2(o, lse, zero, None, v)["scale"]
        np.testing.assert_allclose(got, wo * ao + (1.0 - wo) * av, rtol=1e-13, atol=0)
    w = (rng.standard_normal(D) * 0.3).astype(np.float32)
    sp = orc.aggregate([v], w)["m"]
    for shift, want in ((-200.0, av), (200.0, ao)):
        got = orc.phase2(o, (sp + shift).astype(np.float32), w, None, v)["scale"]
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def pin_scale_merge_closed_form(orc):
    """The merge scale is (e^lse |o| + sum_i e^s_i |v_i|) / (e^lse + sum_i e^s_i).
    With a zero query every new source scores 0, so for a group lse of l it is
    (e^l |o| + sum_i |v_i|) / (e^l + n) (K3 §9.4 OS2, each new source its own
    term)."""
    rng = np.random.default_rng(63)
    A, B, _, g = _merge_inputs(rng, nB=3)
    o = A[1]
    zero = np.zeros(o.shape[1], np.float32)
    sumv = sum(np.abs(b.astype(np.float64)) for b in B)
    for l in (0.0, 1.5, -2.0):
        lse = np.full(o.shape[0], l, np.float32)
        e = math.exp(float(lse[0]))
        got = orc.merge(o, lse, B, zero, g)["scale"]
        want = (e * np.abs(o.astype(np.float64)) + sumv) / (e + len(B))
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def pin_scale_stack_zero_queries(orc):
    """With zero queries every aggregate of the stack weighs its sources
    equally, so the scale of h_l is the mean of |source| over the sources the
    plan gives sublayer l, and y's over the completed blocks (K3 §9.3 listing,
    §9.2 zero init). Checked on two blocks with a short last one."""
    rng = np.random.default_rng(64)
    L, S, rows, D = 5, 3, 3, 16
    x, v, _ = _stack_inputs(rng, L, rows, D, "f32")
    W = np.zeros((L + 1, D), np.float32)
    st = orc.block_stack(x, v, W, S=S)
    X = np.abs(x.astype(np.float64))
    V = [a.astype(np.float64) for a in v]
    p1 = [V[0], V[0] + V[1]]          # partials inside block 1 (fp32 sums, rounded)
    b1 = orc.round_to(orc.round_to(V[0] + V[1], "f32").astype(np.float64) + V[2], "f32").astype(np.float64)
    p1[1] = orc.round_to(p1[1], "f32").astype(np.float64)
    want = [X, (X + np.abs(p1[0])) / 2, (X + np.abs(p1[1])) / 2,
            (X + np.abs(b1)) / 2, (X + np.abs(b1) + np.abs(V[3])) / 3]
    for l in range(L):
        np.testing.assert_allclose(st["h_scale"][l], want[l], rtol=1e-14, atol=0, err_msg=f"h_{l + 1}")
    b2 = orc.round_to(V[3] + V[4], "f32").astype(np.float64)
    np.testing.assert_allclose(st["y_scale"], (X + np.abs(b1) + np.abs(b2)) / 3, rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------
# Phase 1 / Phase 2 definitions
# ----------------------------------------------------------------------------

def pin_phase1_is_per_query_aggregate(orc):
    """Phase 1 is S aggregates of the same fixed sources, one per stacked query
    (K3 §9.4 step 1)."""
    rng = np.random.default_rng(7)
    src = [bf16_normal(rng, (4, 32), s) for s in (1.0, 2.0, 0.5)]
    W = (rng.standard_normal((5, 32)) * 0.2).astype(np.float32)
    G = rng.uniform(0.5, 1.5, (5, 32)).astype(np.float32)
    ph = orc.phase1(src, W, G)
    for s in range(5):
        a = orc.aggregate(src, W[s], G[s])
        assert np.array_equal(ph["o"][s], a["h"]) and np.array_equal(ph["lse"][s], a["lse"])
        assert np.array_equal(ph["m"][s], a["m"])


def pin_phase2_merge_limits(orc):
    """Merging the Phase-1 group (lse, o) with the partial's single-source
    triple (s_p, p, 1) by OS2: lse far below s_p gives h = p, far above gives
    h = o, equal gives the midpoint (K3 §9.4 OS2 and single-source triple)."""
    rng = np.random.default_rng(8)
    rows, D = 3, 32
    o = (rng.standard_normal((rows, D))).astype(np.float32)
    v = (rng.standard_normal((rows, D)) * 2).astype(np.float32)
    w = (rng.standard_normal(D) * 0.3).astype(np.float32)
    sp = orc.aggregate([v], w)["m"]  # score of the single source p = v
    for shift, expect in ((-200.0, v.astype(np.float64)), (200.0, o.astype(np.float64))):
        lse = (sp + shift).astype(np.float32)
        out = orc.phase2(o, lse, w, None, v)
        assert np.allclose(out["h"], expect, rtol=1e-12, atol=1e-12), shift
        assert np.array_equal(out["p"], v)
    # a zero query scores p at exactly 0; with lse = 0 the two groups tie
    out = orc.phase2(o, np.zeros(rows, np.float32), np.zeros(D, np.float32), None, v)
    assert np.array_equal(out["h"], 0.5 * o.astype(np.float64) + 0.5 * v.astype(np.float64))


def pin_phase2_partial_update(orc):
    """p <- p + v is kept in the model dtype: fp32 add then one rounding to
    bf16 (torch's bf16 arithmetic), bit for bit (K3 §9.3/§9.4 listings)."""
    rng = np.random.default_rng(9)
    rows, D = 4, 64
    # magnitudes spread over many binades so exponent gaps exceed 16 sometimes
    p = f64_to_bf16_via_torch((rng.standard_normal((rows, D)) * np.exp2(rng.integers(-20, 20, (rows, D)))).astype(np.float32))
    v = f64_to_bf16_via_torch((rng.standard_normal((rows, D)) * np.exp2(rng.integers(-20, 20, (rows, D)))).astype(np.float32))
    o = bf16_normal(rng, (rows, D))
    w = (rng.standard_normal(D) * 0.1).astype(np.float32)
    out = orc.phase2(o, np.zeros(rows, np.float32), w, p, v)
    tp = torch.from_numpy(p.view(np.int16)).view(torch.bfloat16)
    tv = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
    ref = (tp + tv).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["p"], ref)
    # and the merge uses the rounded partial: compare with an aggregate over it
    single = orc.aggregate([ref], w)
    assert np.allclose(orc.phase2(o, np.full(rows, -1e4, np.float32), w, p, v)["h"],
                       single["h"], rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------
# stack bookkeeping
# ----------------------------------------------------------------------------

def _stack_inputs(rng, L, rows, D, dtype, scale_hi=5.0):
    if dtype == "bf16":
        x = bf16_normal(rng, (rows, D))
        v = [bf16_normal(rng, (rows, D), rng.uniform(0.1, scale_hi)) for _ in range(L)]
    else:
        x = rng.standard_normal((rows, D)).astype(np.float32)
        v = [(rng.standard_normal((rows, D)) * rng.uniform(0.1, scale_hi)).astype(np.float32)
             for _ in range(L)]
    W = (rng.standard_normal((L + 1, D)) * 0.3).astype(np.float32)
    return x, v, W


def pin_plan_golden(orc):
    """Block plan and unit conversion against the integers the pages print."""
    with open(os.path.join(GOLDEN, "plan_examples.json")) as f:
        g = json.load(f)
    for c in g["atomic_block_size"]:
        assert orc.atomic_block_size(c["num_hidden_layers"], c["layers_per_block"]) == c["expect"], c["cite"]
    for c in g["block_plan"]:
        nb, starts, ns = orc.block_plan(c["L"], c["S"])
        assert nb == c["expect_nb"], c["cite"]
        if "expect_final_sources" in c:
            assert ns[-1] == c["expect_final_sources"], c["cite"]
        if "expect_max_sources_at_most" in c:
            assert ns.max() <= c["expect_max_sources_at_most"], c["cite"]
        # structural: blocks tile 1..L in order, each at most S long, only the last may be short
        sizes = np.diff(starts)
        assert starts[0] == 1 and starts[-1] == c["L"] + 1
        assert np.all(sizes[:-1] == c["S"]) and 1 <= sizes[-1] <= c["S"]
    for c in g["new_parameters"]:
        N = 2 * c["num_hidden_layers"]
        assert N == c["N"], c["cite"]
        _, _, ns = orc.block_plan(N, orc.atomic_block_size(c["num_hidden_layers"]))
        # one query and one gain per aggregation: N sublayers plus the final aggregate
        assert 2 * len(ns) * c["D"] == c["expect"], c["cite"]


def pin_plan_source_counts(orc):
    """Sublayer l of block k sees the k+1 completed sources plus the partial
    once it exists (K3 §9.3 listing; WC 'Block AttnRes'); Full (S = 1) sees l."""
    for L in range(1, 30):
        for S in range(1, L + 2):
            nb, starts, ns = orc.block_plan(L, S)
            assert nb == -(-L // S)
            for l in range(1, L + 1):
                k = (l - 1) // S
                j = (l - 1) % S
                assert ns[l - 1] == k + 1 + (1 if j >= 1 else 0), (L, S, l)
            assert ns[L] == nb + 1
            if S == 1:
                assert list(ns[:L]) == list(range(1, L + 1))


def pin_full_equals_block_s1(orc):
    """Block with S = 1 is Full AttnRes: sublayer l aggregates
    [x, v_1, ..., v_{l-1}] and the final query all L+1 sources (WC 'Block
    AttnRes', N = L limit; K3 §9.3)."""
    rng = np.random.default_rng(13)
    L, rows, D = 5, 3, 16
    x, v, W = _stack_inputs(rng, L, rows, D, "bf16")
    st = orc.block_stack(x, v, W, S=1)
    for l in range(1, L + 1):
        a = orc.aggregate([x] + v[: l - 1], W[l - 1])
        assert np.array_equal(st["h"][l - 1], a["h"]) and np.array_equal(st["h_lse"][l - 1], a["lse"])
    a = orc.aggregate([x] + v, W[L])
    assert np.array_equal(st["y"], a["h"])
    for k in range(L):
        assert np.array_equal(st["block_sums"][k], v[k])


def pin_one_block_is_standard_residual(orc):
    """One block (S >= L): the block sum is the plain left-fold sum of the
    sublayer outputs, the sources are {x, partial}, and with zero queries the
    final output is (x + sum v)/2, i.e. half the standard residual stream
    x_N = x_0 + sum f_l (WC 'Block AttnRes', N = 1 limit; K3 §9.1)."""
    rng = np.random.default_rng(14)
    L, rows, D = 6, 4, 32
    x, v, _ = _stack_inputs(rng, L, rows, D, "bf16")
    W = np.zeros((L + 1, D), np.float32)
    for S in (L, L + 3):
        st = orc.block_stack(x, v, W, S=S)
        t = torch.from_numpy(v[0].view(np.int16)).view(torch.bfloat16)
        folds = [t]
        for a in v[1:]:
            t = t + torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
            folds.append(t)
        b1 = folds[-1].view(torch.int16).numpy().view(np.uint16)
        assert st["nb"] == 1 and np.array_equal(st["block_sums"][0], b1)
        X = bf16_to_f64(x)
        assert np.array_equal(st["h"][0], X)
        for l in range(2, L + 1):
            p = bf16_to_f64(folds[l - 2].view(torch.int16).numpy().view(np.uint16))
            assert np.allclose(st["h"][l - 1], 0.5 * (X + p), rtol=1e-15, atol=1e-15)
        assert np.allclose(2 * st["y"], X + bf16_to_f64(b1), rtol=1e-15, atol=1e-15)


def pin_two_phase_bruteforce(orc):
    """Two-phase equals naive (K3 §9.4 equivalence box; WC online softmax):
    for every L <= 7 and S <= L+1, Phase 1 over the completed sources merged
    by OS2 with the partial's single-source triple reproduces the naive
    stack's h_l, in fp64, on tiny rows."""
    rng = np.random.default_rng(15)
    for dtype in ("bf16", "f32"):
        for D in (8, 16):
            for L in range(1, 8):
                x, v, W = _stack_inputs(rng, L, 3, D, dtype)
                for S in range(1, L + 2):
                    st = orc.block_stack(x, v, W, S=S)
                    blocks = [x]
                    for k, start in enumerate(range(1, L + 1, S)):
                        end = min(start + S - 1, L)
                        ph = orc.phase1(blocks, W[start - 1:end])
                        partial = None
                        for j, l in enumerate(range(start, end + 1)):
                            summ = (ph["lse"][j], ph["o"][j])
                            if partial is not None:
                                # one source: its lse is its score and its output is itself
                                single = orc.aggregate([partial], W[l - 1])
                                summ = os2_merge(summ, (single["m"], widen(partial)))
                            h = summ[1]
                            assert np.allclose(h, st["h"][l - 1], rtol=1e-12, atol=1e-12), (dtype, D, L, S, l)
                            if partial is None:
                                partial = v[l - 1]
                            else:
                                partial = orc.round_to(widen(partial) + widen(v[l - 1]), dtype)
                        assert np.array_equal(st["block_sums"][k], partial), (dtype, L, S, k)
                        blocks.append(partial)
                    y = orc.aggregate(blocks, W[L])
                    assert np.allclose(y["h"], st["y"], rtol=1e-13, atol=1e-13)


def pin_phase2_composes_to_naive(orc):
    """The isolated Phase-2 step, fed the Phase-1 output rounded to fp32 and
    its lse, reproduces the naive stack's h_l to fp32 accuracy."""
    rng = np.random.default_rng(16)
    L, S, rows, D = 6, 4, 3, 32
    x, v, W = _stack_inputs(rng, L, rows, D, "f32")
    st = orc.block_stack(x, v, W, S=S)
    ph = orc.phase1([x], W[0:4])
    p = None
    for j in range(1, 4):
        out = orc.phase2(ph["o"][j].astype(np.float32), ph["lse"][j].astype(np.float32), W[j],
                         p, v[j - 1])
        assert np.allclose(out["h"], st["h"][j], rtol=0, atol=2e-6 * out["scale"].max())
        p = out["p"]


def pin_causality(orc):
    """Depth weights are per token and never mix positions: perturbing one
    row's inputs changes only that row's outputs (K3 §9.1 importantbox;
    attnres_is_still_causal in the K3 §9.7 table)."""
    rng = np.random.default_rng(17)
    L, S, rows, D = 5, 2, 4, 16
    x, v, W = _stack_inputs(rng, L, rows, D, "f32")
    base = orc.block_stack(x, v, W, S=S)
    v2 = [a.copy() for a in v]
    v2[1][2] += np.float32(1.5)
    pert = orc.block_stack(x, v2, W, S=S)
    other = [0, 1, 3]
    assert np.array_equal(base["h"][:, other], pert["h"][:, other])
    assert np.array_equal(base["y"][other], pert["y"][other])
    assert not np.array_equal(base["y"][2], pert["y"][2])


def pin_rmsnorm_library(orc):
    """The sublayer input norm equals torch's rms_norm evaluated in float64
    (same definition: eps inside the root, mean over the hidden axis, times
    the gain), with and without a gain."""
    import torch
    rng = np.random.default_rng(31)
    for D, eps in ((64, 1e-6), (256, 1e-8), (40, 0.25)):
        x = (rng.standard_normal((7, D)) * rng.uniform(0.1, 5.0, (7, 1))).astype(np.float32)
        g = rng.uniform(0.5, 1.5, D).astype(np.float32)
        for gain in (g, None):
            got = orc.rmsnorm(x, gain, eps=eps)["out"]
            ref = torch.nn.functional.rms_norm(
                torch.from_numpy(x.astype(np.float64)), (D,),
                None if gain is None else torch.from_numpy(gain.astype(np.float64)), eps=eps).numpy()
            np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def pin_rmsnorm_closed_forms(orc):
    """A constant row c gives gamma * c / sqrt(c^2 + eps) in every element; with
    eps = 0 and unit gain every row has mean square exactly 1 (up to fp64
    rounding) and rescaling a row by a power of two leaves it unchanged."""
    for c, eps in ((3.0, 1e-6), (-0.5, 0.25), (2.0 ** -10, 1e-8)):
        x = np.full((2, 32), c, dtype=np.float32)
        g = np.linspace(0.5, 1.5, 32).astype(np.float32)
        out = orc.rmsnorm(x, g, eps=eps)
        want = g.astype(np.float64) * c / np.sqrt(c * c + eps)
        np.testing.assert_allclose(out["out"], np.broadcast_to(want, (2, 32)), rtol=1e-14)
        np.testing.assert_allclose(out["rms"], np.sqrt(c * c + eps), rtol=1e-14)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 48)).astype(np.float32)
    out = orc.rmsnorm(x, None, eps=0.0)["out"]
    np.testing.assert_allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-13)
    out4 = orc.rmsnorm((x * np.float32(4.0)).astype(np.float32), None, eps=0.0)["out"]
    assert np.array_equal(out, out4)


def _merge_inputs(rng, rows=6, D=32, nA=3, nB=2):
    A = [(rng.standard_normal((rows, D)) * s).astype(np.float32) for s in (1.0, 3.0, 0.4)[:nA]]
    B = [(rng.standard_normal((rows, D)) * s).astype(np.float32) for s in (2.0, 0.7, 5.0)[:nB]]
    w = (0.3 * rng.standard_normal(D)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return A, B, w, g


def pin_merge_is_aggregate_of_union(orc):
    """Merging the summary (lse, o) of sources A with sources B equals one
    aggregate over A and B together: the exactness of the online-softmax merge
    across phases (K3 §9.4 (OS1)/(OS2) and its equivalence box), on which the
    Full two-phase schedule rests. o and lse are rounded to fp32 on the way,
    as a kernel stores them."""
    rng = np.random.default_rng(41)
    A, B, w, g = _merge_inputs(rng)
    a = orc.aggregate(A, w, g)
    o = orc.round_to(a["h"], "f32")
    lse = a["lse"].astype(np.float32)
    got = orc.merge(o, lse, B, w, g)
    want = orc.aggregate(A + B, w, g)
    assert np.all(np.abs(got["h"] - want["h"]) <= 1e-6 * want["scale"])
    # lse is invariant; m is only the merge's reference point (max(lse_A, s_B))
    np.testing.assert_allclose(got["lse"], want["lse"], rtol=0, atol=1e-6 * (1 + np.abs(want["lse"])).max())


def pin_merge_one_source_is_phase2(orc):
    """With a single new source the merge is the Phase-2 step on a first
    partial p = v (K3 §9.4 single-source triple)."""
    rng = np.random.default_rng(43)
    A, B, w, g = _merge_inputs(rng, nB=1)
    a = orc.aggregate(A, w, g)
    o = orc.round_to(a["h"], "f32")
    lse = a["lse"].astype(np.float32)
    got = orc.merge(o, lse, B, w, g)["h"]
    ref = orc.phase2(o, lse, w, None, B[0], g)["h"]
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def pin_merge_limits(orc):
    """A group with lse far below the new sources' scores contributes nothing
    (the merge is the aggregate of the new sources); far above, the merge
    returns the group's output."""
    rng = np.random.default_rng(47)
    A, B, w, g = _merge_inputs(rng)
    o = A[0]
    low = orc.merge(o, np.full(o.shape[0], -1e4, np.float32), B, w, g)["h"]
    np.testing.assert_allclose(low, orc.aggregate(B, w, g)["h"], rtol=1e-12, atol=1e-12)
    high = orc.merge(o, np.full(o.shape[0], 1e4, np.float32), B, w, g)["h"]
    np.testing.assert_allclose(high, o.astype(np.float64), rtol=1e-12, atol=1e-12)


def _grid_values(rng, shape, scale_bits, lo, hi):
    """fp32 values k * 2^-scale_bits, integer k in [lo, hi): exact in fp32, and
    stay exact after adding or subtracting 2^-10 when scale_bits >= 10."""
    return (rng.integers(lo, hi, size=shape).astype(np.float64) * 2.0 ** -scale_bits).astype(np.float32)


def pin_backward_finite_differences(orc):
    """The aggregate backward against central finite differences of
    L = sum(dh * h) computed by the forward oracle, for every source element,
    every w and every gain (K3 §9.1 (A1)-(A3) differentiated). Inputs are
    fp32 grid values, so each +-2^-10 perturbation is exact, w * gamma is exact
    in fp32, and the fp64 forward makes the difference quotients accurate to
    about 1e-9 of the gradient scale."""
    rng = np.random.default_rng(53)
    rows, D, n = 2, 16, 3
    V = [_grid_values(rng, (rows, D), 12, -8192, 8192) for _ in range(n)]
    w = _grid_values(rng, D, 12, -1024, 1024)
    g = _grid_values(rng, D, 4, 8, 24)  # gains 0.5 .. 1.5
    dh = _grid_values(rng, (rows, D), 12, -4096, 4096)
    eps = 1e-3
    got = orc.aggregate_backward(V, w, dh, g, eps=eps)
    delta = np.float32(2.0 ** -10)

    def loss(VV, ww, gg):
        return float((orc.aggregate(VV, ww, gg, eps=eps)["h"] * dh.astype(np.float64)).sum())

    scale = max(np.abs(got["dV"]).max(), np.abs(got["dw"]).max(), np.abs(got["dgamma"]).max())
    for i in range(n):
        for r in range(rows):
            for d in range(D):
                Vp = [a.copy() for a in V]; Vm = [a.copy() for a in V]
                Vp[i][r, d] += delta; Vm[i][r, d] -= delta
                fd = (loss(Vp, w, g) - loss(Vm, w, g)) / (2 * float(delta))
                assert abs(fd - got["dV"][i, r, d]) <= 1e-6 * scale, (i, r, d, fd, got["dV"][i, r, d])
    for d in range(D):
        wp, wm = w.copy(), w.copy()
        wp[d] += delta; wm[d] -= delta
        fd = (loss(V, wp, g) - loss(V, wm, g)) / (2 * float(delta))
        assert abs(fd - got["dw"][d]) <= 1e-6 * scale, ("w", d, fd, got["dw"][d])
        gp, gm = g.copy(), g.copy()
        gp[d] += delta; gm[d] -= delta
        fd = (loss(V, w, gp) - loss(V, w, gm)) / (2 * float(delta))
        assert abs(fd - got["dgamma"][d]) <= 1e-6 * scale, ("gamma", d, fd, got["dgamma"][d])


def pin_stack_backward_finite_differences(orc):
    """The stack backward (the aggregate backward composed over the naive
    Block forward) against central differences of
    L = sum_l <dh_l, h_l> + <dy, y> computed by the oracle's naive stack
    forward (K3 9.3), for every element of x, of every sublayer output, of
    every query and of every gain. Five sublayers in blocks of two exercise
    the partials, the block sums and a one-sublayer last block. Inputs are
    fp32 grid values, so partials, block sums and the +-2^-10 steps are exact
    and the loss is smooth in every input."""
    rng = np.random.default_rng(67)
    L, S, rows, D, eps = 5, 2, 2, 8, 1e-3
    x = _grid_values(rng, (rows, D), 12, -4096, 4096)
    v = [_grid_values(rng, (rows, D), 12, -4096, 4096) for _ in range(L)]
    W = _grid_values(rng, (L + 1, D), 12, -2048, 2048)
    G = _grid_values(rng, (L + 1, D), 4, 8, 24)
    dh = [_grid_values(rng, (rows, D), 12, -4096, 4096) for _ in range(L)]
    dy = _grid_values(rng, (rows, D), 12, -4096, 4096)
    got = orc.block_stack_backward(x, v, W, S, dh, dy, Gamma=G, eps=eps)
    delta = np.float32(2.0 ** -10)

    def loss(xx, vv, WW, GG):
        st = orc.block_stack(xx, vv, WW, S, Gamma=GG, eps=eps)
        return float(sum((st["h"][l] * dh[l].astype(np.float64)).sum() for l in range(L))
                     + (st["y"] * dy.astype(np.float64)).sum())

    scale = max(np.abs(got["dx"]).max(), np.abs(got["dv"]).max(), np.abs(got["dW"]).max(),
                np.abs(got["dGamma"]).max())

    def check(fd, val, what):
        assert abs(fd - val) <= 1e-6 * scale, (what, fd, val)

    for r in range(rows):
        for d in range(D):
            xp, xm = x.copy(), x.copy()
            xp[r, d] += delta; xm[r, d] -= delta
            check((loss(xp, v, W, G) - loss(xm, v, W, G)) / (2 * float(delta)), got["dx"][r, d], ("x", r, d))
            for l in range(L):
                vp = [a.copy() for a in v]; vm = [a.copy() for a in v]
                vp[l][r, d] += delta; vm[l][r, d] -= delta
                check((loss(x, vp, W, G) - loss(x, vm, W, G)) / (2 * float(delta)), got["dv"][l, r, d],
                      ("v", l, r, d))
    for l in range(L + 1):
        for d in range(D):
            Wp, Wm = W.copy(), W.copy()
            Wp[l, d] += delta; Wm[l, d] -= delta
            check((loss(x, v, Wp, G) - loss(x, v, Wm, G)) / (2 * float(delta)), got["dW"][l, d], ("W", l, d))
            Gp, Gm = G.copy(), G.copy()
            Gp[l, d] += delta; Gm[l, d] -= delta
            check((loss(x, v, W, Gp) - loss(x, v, W, Gm)) / (2 * float(delta)), got["dGamma"][l, d],
                  ("Gamma", l, d))


def pin_backward_special_cases(orc):
    """One source: h is the source, so dV = dh exactly and the query gets no
    gradient; a zero upstream gradient gives zero gradients; with eps = 0 the
    score part of dV_i is orthogonal to V_i (scores ignore a source's scale,
    K3 §9.2)."""
    rng = np.random.default_rng(59)
    V = [rng.standard_normal((3, 32)).astype(np.float32) for _ in range(4)]
    w = (0.2 * rng.standard_normal(32)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 32).astype(np.float32)
    dh = rng.standard_normal((3, 32)).astype(np.float32)
    one = orc.aggregate_backward(V[:1], w, dh, g)
    assert np.array_equal(one["dV"][0], dh.astype(np.float64))
    assert not np.any(one["dw"]) and not np.any(one["dgamma"])
    zero = orc.aggregate_backward(V, w, np.zeros_like(dh), g)
    assert not np.any(zero["dV"]) and not np.any(zero["dw"])
    full = orc.aggregate_backward(V, w, dh, g, eps=0.0)
    alpha = orc.aggregate(V, w, g, eps=0.0, want_alpha=True)["alpha"]
    for i in range(4):
        score_part = full["dV"][i] - alpha[:, i:i + 1] * dh.astype(np.float64)
        dot = (score_part * V[i].astype(np.float64)).sum(axis=1)
        ref = np.abs(score_part).sum(axis=1) * np.abs(V[i]).max()
        assert np.all(np.abs(dot) <= 1e-12 * ref)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
