"""The CPU oracle against its pins, and the pins against planted mistakes.

``test_pin`` runs every pin of ``oracle_pins`` on the real oracle. The
mutation tests compile copies of ``oracle/oracle.c`` with one plausible
mistake each (a dropped term, a wrong sign or index, a transposed operand, a
misplaced eps, a wrong rounding rule) and require that at least one pin fails
on every mutant: the pins are strong enough to catch them.
"""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("bwd_drops_rms_term", "ds * (c->q[d] / rr[i] - s[i] * V[i][d] / ((double)D * rr[i] * rr[i]))",
     "ds * (c->q[d] / rr[i])"),
    ("bwd_softmax_no_centering", "const double ds = a[i] * (gi - gh);", "const double ds = a[i] * gi;"),
    ("bwd_dgamma_uses_gain", "if (dgamma) dgamma[d] = t * (double)w[d];",
     "if (dgamma) dgamma[d] = t * g;"),
    ("bwd_dq_raw_sources", "dq[d] += ds * V[i][d] / rr[i];", "dq[d] += ds * V[i][d];"),
    ("merge_drops_group", "const double wo = exp(la - mm);", "const double wo = 0.0 * exp(la - mm);"),
    ("merge_lse_drops_max", "if (c->lse_out) c->lse_out[r] = mm + log(z);",
     "if (c->lse_out) c->lse_out[r] = log(z);"),
    ("merge_wrong_source_weight", "const double a = exp(s[i] - mm);",
     "const double a = exp(s[c->n - 1 - i] - mm);"),
    ("norm_sum_not_mean", "const double rms = sqrt(ss / (double)D + c->eps);",
     "const double rms = sqrt(ss + c->eps);"),
    ("norm_eps_outside_root", "const double rms = sqrt(ss / (double)D + c->eps);",
     "const double rms = sqrt(ss / (double)D) + c->eps;"),
    ("norm_gain_dropped", "const double g = c->gamma ? (double)c->gamma[d] : 1.0;", "const double g = 1.0;"),
    ("norm_multiplies_by_rms", "c->out[r * D + d] = g * widen(c->x, c->dtype, r * D + d) / rms;",
     "c->out[r * D + d] = g * widen(c->x, c->dtype, r * D + d) * rms;"),
    ("rms_sum_not_mean", "sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    ("eps_outside_root", "sqrt(ss / (double)D + eps)", "(sqrt(ss / (double)D) + eps)"),
    ("softmax_sign", "a[i] = exp(s[i] - m);", "a[i] = exp(m - s[i]);"),
    ("weighted_sum_wrong_index", "acc += a[i] * V[i][d];", "acc += a[i] * V[n - 1 - i][d];"),
    ("scores_on_raw_sources", "dot += q[d] * (V[i][d] * inv_rms);", "dot += q[d] * V[i][d];"),
    ("weights_on_normalised_values", "acc += a[i] * V[i][d];", "acc += a[i] * V[i][d] / sqrt(1e-300 + V[i][d] * V[i][d]);"),
    ("lse_drops_max", "*lse_out = m + log(z);", "*lse_out = log(z);"),
    ("gain_dropped", "q[d] = (double)(float)((double)w[d] * (double)g);", "q[d] = (double)w[d];"),
    ("merge_weights_swapped", "double num = wa * ov + wb * p[d];", "double num = wb * ov + wa * p[d];"),
    ("partial_not_accumulated", "p[d] = c->p_prev ? oracle_round(widen(c->p_prev, c->dtype, r * D + d) + v, c->dtype) : v;",
     "p[d] = v;"),
    ("stack_partial_not_rounded", "partial[d] = have_partial ? oracle_round(partial[d] + vd, c->dtype) : vd;",
     "partial[d] = have_partial ? partial[d] + vd : vd;"),
    ("short_last_block_dropped", "if (l % c->S == 0 || l == c->L) {", "if (l % c->S == 0) {"),
    ("plan_partial_not_counted", "n_sources[l - 1] = nblocks_done + (have_partial ? 1 : 0);",
     "n_sources[l - 1] = nblocks_done;"),
    ("round_ties_away", "double r = ldexp(nearbyint(ldexp(x, -qexp)), qexp);",
     "double r = ldexp(round(ldexp(x, -qexp)), qexp);"),
    ("round_keeps_7_bits", "int qexp = e - 8;", "int qexp = e - 7;"),
    ("final_query_wrong_row", "agg_row(n, src, c->q + (int64_t)c->L * D,", "agg_row(n, src, c->q + (int64_t)(c->L - 1) * D,"),
    ("auto_block_size_floor", "((num_hidden_layers + 7) / 8 > 1 ? (num_hidden_layers + 7) / 8 : 1)",
     "(num_hidden_layers / 8 > 1 ? num_hidden_layers / 8 : 1)"),
    ("agg_scale_drops_weights", "sc += a[i] * fabs(V[i][d]);", "sc += fabs(V[i][d]);"),
    ("agg_scale_signed", "sc += a[i] * fabs(V[i][d]);", "sc += a[i] * V[i][d];"),
    ("agg_scale_wrong_source", "sc += a[i] * fabs(V[i][d]);", "sc += a[n - 1 - i] * fabs(V[i][d]);"),
    ("ph2_scale_drops_weights", "c->scale[r * D + d] = (wa * fabs(ov) + wb * fabs(p[d])) / den;",
     "c->scale[r * D + d] = fabs(ov) + fabs(p[d]);"),
    ("ph2_scale_weights_swapped", "c->scale[r * D + d] = (wa * fabs(ov) + wb * fabs(p[d])) / den;",
     "c->scale[r * D + d] = (wb * fabs(ov) + wa * fabs(p[d])) / den;"),
    ("merge_scale_drops_weights", "sc += a * fabs(V[i][d]);", "sc += fabs(V[i][d]);"),
    ("merge_scale_drops_group", "double num = wo * ov, sc = wo * fabs(ov);", "double num = wo * ov, sc = 0.0;"),
    ("stack_scale_is_h", "if (c->h_scale) memcpy(c->h_scale + ho * D, srow,", "if (c->h_scale) memcpy(c->h_scale + ho * D, hrow,"),
    ("phase1_same_query", "fold_query(W + (int64_t)s * D, Gamma ? Gamma + (int64_t)s * D : NULL, D, q + (int64_t)s * D);",
     "fold_query(W, Gamma, D, q + (int64_t)s * D);"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in oracle.c"
    mutated = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    c = d / "oracle.c"
    c.write_text(mutated)
    return oracle.compile_oracle(str(c), str(d / "liboracle.so"))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    mutant = oracle.Oracle(_build_mutant(tmp_path, name, old, new))
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
