/*
 * oracle.c -- the plain, slow, fp64 CPU oracle for AttnRes depth aggregation.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load the library built from this file. It shares no code,
 * header, helper or constant with the GPU library, and neither side includes
 * or links the other.
 *
 * Every function below is the plain definition written out, in fp64, one
 * token row at a time, with no blocking, fusion or reordering beyond what the
 * definition states. Inputs arrive in the I/O dtype (fp32 or bf16 bit
 * patterns) and are widened exactly to double.
 *
 * Sources (page title, then the passage):
 *  [K3]  K3 course notes, section "Attention Residual 深度残差":
 *        9.1 eqs. (A1)-(A4); 9.2 DepthResidual (gain folding, scoring on the
 *        normalised copy, weighted sum of the raw sources, zero-init query);
 *        9.3 Full vs Block and BlockAttnResStack.forward_naive; 9.4 online
 *        softmax triples (OS1), the two-group merge (OS2) and the
 *        single-source triple; 9.6 atomic_block_size.
 *  [WC]  "Attention Residuals: when network depth can also address"
 *        (wineandchord.com): "Depth attention & online merge reference"
 *        (RMS normalisation with eps inside the root, mean over the hidden
 *        axis), "Block AttnRes" (the embedding stays its own source).
 *  [RH]  Reading notes on "Attention Residuals" (ranhao.site), 4.2 Inference:
 *        Phase 1 returns the outputs plus the max and log-sum-exp statistics.
 *  [ZZ]  "Attention Residuals" notes (zhangzhe.space): the block listing, where
 *        every sublayer applies its own RMSNorm to the aggregate it receives.
 *
 * Readings where the pages leave a step open (each is listed in the design doc):
 *  - RMS(v) = v / sqrt(mean_d(v^2) + eps)            [WC reference code]
 *  - folded query q~ = fp32(w * gamma), then widened  [K3 9.2 (1)]
 *  - the intra-block partial is kept in the I/O dtype: each add is exact in
 *    fp64 and rounded once to the dtype, nearest-even  [K3 9.3 listing]
 *  - Phase-1 statistics are exported as (m, lse) with normalised outputs.
 *
 * Parity pins live in tests/test_oracle_pins.py (closed forms, invariants,
 * special cases and brute force); no function here is unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_MAX_SOURCES 1024

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* ------------------------------------------------------------------------ */
/* dtype handling                                                           */
/* ------------------------------------------------------------------------ */

static double widen(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round an exact real held in a double to bf16, nearest with ties to even.
   bf16 keeps 8 significant bits (1 implicit + 7 stored) over fp32's exponent
   range, so the rounding quantum is 2^(e-8) for x = f * 2^e, 0.5 <= |f| < 1,
   and 2^-133 below the smallest normal 2^-126. */
static double round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  (void)frexp(x, &e);
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  double r = ldexp(nearbyint(ldexp(x, -qexp)), qexp);
  if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, x);
  return r;
}

double oracle_round(double x, int dtype) {
  if (dtype == ORACLE_F32) return (double)(float)x; /* C rounds to nearest even */
  return round_bf16(x);
}

static void store_dtype(void* base, int dtype, int64_t i, double rounded) {
  float f = (float)rounded; /* exact: rounded is representable in the dtype */
  if (dtype == ORACLE_F32) {
    ((float*)base)[i] = f;
  } else {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    ((uint16_t*)base)[i] = (uint16_t)(u >> 16);
  }
}

/* Round an array of doubles to the dtype and store the bit patterns. */
void oracle_store_rounded(const double* x, int64_t count, int dtype, void* out) {
  for (int64_t i = 0; i < count; ++i) store_dtype(out, dtype, i, oracle_round(x[i], dtype));
}

/* ------------------------------------------------------------------------ */
/* AGG: eqs. (A1)-(A3) for one token row                                    */
/* ------------------------------------------------------------------------ */

/* Depth attention over n sources for one row [K3 9.1 (A1)-(A3), 9.2]:
     s_i   = q~ . ( V_i / sqrt(mean_d V_i^2 + eps) )    score on the gain-free RMS copy
     a_i   = exp(s_i) / sum_j exp(s_j)                   softmax over the source axis
     h     = sum_i a_i V_i                               weighted sum of the RAW sources
   plus the online-softmax statistics of the group [K3 9.4 (OS1); RH 4.2]:
     m = max_i s_i,  lse = m + log(sum_i exp(s_i - m)),
   and the per-element condition scale sum_i a_i |V_i[d]| used by the tests'
   tolerance rule. */
static void agg_row(int n, const double* const* V, const double* q, int64_t D, double eps,
                    double* h, double* scale, double* m_out, double* lse_out, double* alpha_out) {
  double s[ORACLE_MAX_SOURCES];
  double a[ORACLE_MAX_SOURCES];
  for (int i = 0; i < n; ++i) {
    double ss = 0.0;
    for (int64_t d = 0; d < D; ++d) ss += V[i][d] * V[i][d];
    double inv_rms = 1.0 / sqrt(ss / (double)D + eps);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * (V[i][d] * inv_rms);
    s[i] = dot;
  }
  double m = s[0];
  for (int i = 1; i < n; ++i)
    if (s[i] > m) m = s[i];
  double z = 0.0;
  for (int i = 0; i < n; ++i) {
    a[i] = exp(s[i] - m);
    z += a[i];
  }
  for (int i = 0; i < n; ++i) a[i] /= z;
  for (int64_t d = 0; d < D; ++d) {
    double acc = 0.0, sc = 0.0;
    for (int i = 0; i < n; ++i) {
      acc += a[i] * V[i][d];
      sc += a[i] * fabs(V[i][d]);
    }
    if (h) h[d] = acc;
    if (scale) scale[d] = sc;
  }
  if (m_out) *m_out = m;
  if (lse_out) *lse_out = m + log(z);
  if (alpha_out)
    for (int i = 0; i < n; ++i) alpha_out[i] = a[i];
}

/* Folded pseudo-query q~ = w * gamma, formed in fp32 and widened [K3 9.2 (1)].
   gamma == NULL means the RMSNorm gain's neutral value, ones. */
static void fold_query(const float* w, const float* gamma, int64_t D, double* q) {
  for (int64_t d = 0; d < D; ++d) {
    float g = gamma ? gamma[d] : 1.0f;
    q[d] = (double)(float)((double)w[d] * (double)g);
  }
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver: rows are independent [K3 9.1, "weights are per token"] */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t r, double* scratch);

typedef struct {
  row_fn fn;
  void* ctx;
  int64_t r0, r1;
  size_t scratch_doubles;
  int failed;
} worker_arg;

static void* worker_main(void* p) {
  worker_arg* w = (worker_arg*)p;
  double* scratch = (double*)malloc((w->scratch_doubles ? w->scratch_doubles : 1) * sizeof(double));
  if (!scratch) {
    w->failed = 1;
    return NULL;
  }
  for (int64_t r = w->r0; r < w->r1; ++r) w->fn(w->ctx, r, scratch);
  free(scratch);
  return NULL;
}

static int run_rows(int64_t rows, int nthreads, row_fn fn, void* ctx, size_t scratch_doubles) {
  if (rows <= 0) return ORACLE_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  worker_arg args[256];
  int64_t per = rows / nthreads, extra = rows % nthreads, r = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t cnt = per + (t < extra ? 1 : 0);
    args[t] = (worker_arg){fn, ctx, r, r + cnt, scratch_doubles, 0};
    r += cnt;
  }
  int started = 0, failed = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker_main, &args[t]) != 0) {
      failed = 1;
      break;
    }
    started = t;
  }
  if (!failed) worker_main(&args[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = 0; t < nthreads; ++t) failed |= args[t].failed;
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Aggregate and Phase 1                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t D;
  int dtype, n;
  const void* const* src;
  const double* q; /* [nq][D] folded queries */
  int nq;
  int64_t rows;
  double eps;
  double *h, *scale, *m, *lse, *alpha; /* h/scale [nq][rows][D], m/lse [nq][rows], alpha [nq][rows][n] */
} agg_ctx;

static void agg_rowfn(void* p, int64_t r, double* scratch) {
  agg_ctx* c = (agg_ctx*)p;
  const int64_t D = c->D;
  const double* V[ORACLE_MAX_SOURCES];
  for (int i = 0; i < c->n; ++i) {
    double* dst = scratch + (int64_t)i * D;
    for (int64_t d = 0; d < D; ++d) dst[d] = widen(c->src[i], c->dtype, r * D + d);
    V[i] = dst;
  }
  for (int s = 0; s < c->nq; ++s) {
    int64_t o = ((int64_t)s * c->rows + r);
    agg_row(c->n, V, c->q + (int64_t)s * D, D, c->eps, c->h ? c->h + o * D : NULL,
            c->scale ? c->scale + o * D : NULL, c->m ? c->m + o : NULL, c->lse ? c->lse + o : NULL,
            c->alpha ? c->alpha + o * c->n : NULL);
  }
}

static int check_common(int64_t rows, int64_t D, int dtype) {
  if (rows < 0 || D < 1) return ORACLE_EINVAL;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/* One depth aggregation per row over n sources with one query
   [K3 9.2 DepthResidual.forward; WC depth_summary + finish]. */
int oracle_aggregate(int64_t rows, int64_t D, int dtype, int n, const void* const* sources,
                     const float* w, const float* gamma, double eps, double* h, double* scale,
                     double* m, double* lse, double* alpha, int nthreads) {
  if (check_common(rows, D, dtype) || n < 1 || n > ORACLE_MAX_SOURCES || !sources || !w)
    return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)D * sizeof(double));
  if (!q) return ORACLE_ENOMEM;
  fold_query(w, gamma, D, q);
  agg_ctx c = {D, dtype, n, sources, q, 1, rows, eps, h, scale, m, lse, alpha};
  int rc = run_rows(rows, nthreads, agg_rowfn, &c, (size_t)n * (size_t)D);
  free(q);
  return rc;
}

/* Phase 1 of the two-phase Block schedule: the S queries of a block each
   aggregate the same fixed list of completed sources; outputs are normalised,
   with the max and log-sum-exp of each query's scores [K3 9.4 step 1;
   RH 4.2 Phase 1]. Written as its definition: S independent aggregates. */
int oracle_phase1(int64_t rows, int64_t D, int dtype, int n, const void* const* blocks, int S,
                  const float* W, const float* Gamma, double eps, double* o, double* scale,
                  double* m, double* lse, int nthreads) {
  if (check_common(rows, D, dtype) || n < 1 || n > ORACLE_MAX_SOURCES || !blocks || !W || S < 1)
    return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)S * (size_t)D * sizeof(double));
  if (!q) return ORACLE_ENOMEM;
  for (int s = 0; s < S; ++s)
    fold_query(W + (int64_t)s * D, Gamma ? Gamma + (int64_t)s * D : NULL, D, q + (int64_t)s * D);
  agg_ctx c = {D, dtype, n, blocks, q, S, rows, eps, o, scale, m, lse, NULL};
  int rc = run_rows(rows, nthreads, agg_rowfn, &c, (size_t)n * (size_t)D);
  free(q);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Phase 2: one online-softmax merge step                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t D;
  int dtype;
  const void *o, *p_prev, *v_prev;
  const float* lse;
  const double* q;
  double eps;
  void* p_out;
  double *h, *scale;
} ph2_ctx;

static void ph2_rowfn(void* pc, int64_t r, double* p) {
  ph2_ctx* c = (ph2_ctx*)pc;
  const int64_t D = c->D;
  /* Partial update p <- p + v in the model dtype [K3 9.3 listing, 9.4 listing]. */
  for (int64_t d = 0; d < D; ++d) {
    double v = widen(c->v_prev, c->dtype, r * D + d);
    p[d] = c->p_prev ? oracle_round(widen(c->p_prev, c->dtype, r * D + d) + v, c->dtype) : v;
    if (c->p_out) store_dtype(c->p_out, c->dtype, r * D + d, p[d]);
  }
  /* Single-source triple (s_p, p, 1) [K3 9.4 single_source_stats]. */
  double sp, dummy_lse;
  const double* src[1] = {p};
  agg_row(1, src, c->q, D, c->eps, NULL, NULL, &sp, &dummy_lse, NULL);
  /* Phase-1 group as a triple: normalised output o with denominator 1 at the
     reference point lse, i.e. (lse, o, 1); merge with (s_p, p, 1) by (OS2). */
  double la = (double)c->lse[r];
  double mm = la > sp ? la : sp;
  double wa = exp(la - mm), wb = exp(sp - mm);
  double den = wa + wb;
  for (int64_t d = 0; d < D; ++d) {
    double ov = widen(c->o, c->dtype, r * D + d);
    double num = wa * ov + wb * p[d];
    if (c->h) c->h[r * D + d] = num / den;
    if (c->scale) c->scale[r * D + d] = (wa * fabs(ov) + wb * fabs(p[d])) / den;
  }
}

/* Phase 2 of the two-phase schedule for one sublayer [K3 9.4 step 2 and the
   _run_block_two_phase listing; RH 4.2 Phase 2]:
     p = p_prev ? round(p_prev + v_prev) : v_prev
     h = normalized( merge( (lse, o, 1), (s_p, p, 1) ) ). */
int oracle_phase2(int64_t rows, int64_t D, int dtype, const void* o, const float* lse,
                  const float* w, const float* gamma, double eps, const void* p_prev,
                  const void* v_prev, void* p_out, double* h, double* scale, int nthreads) {
  if (check_common(rows, D, dtype) || !o || !lse || !w || !v_prev) return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)D * sizeof(double));
  if (!q) return ORACLE_ENOMEM;
  fold_query(w, gamma, D, q);
  ph2_ctx c = {D, dtype, o, p_prev, v_prev, lse, q, eps, p_out, h, scale};
  int rc = run_rows(rows, nthreads, ph2_rowfn, &c, (size_t)D);
  free(q);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Block plan and the naive Block stack                                     */
/* ------------------------------------------------------------------------ */

/* Integer bookkeeping of forward_naive [K3 9.3 listing; WC "Block AttnRes"]:
   sublayer l (1-based) sees the completed block list plus the running partial
   when one exists; a block closes after l when l % S == 0 or l == L (the last
   block may be short). block_start[k] is the first sublayer of block k, with
   block_start[nb] = L + 1. n_sources[l-1] counts sublayer l's sources and
   n_sources[L] the final aggregate's. Returns nb, or a negative code. */
int oracle_block_plan(int L, int S, int* block_start, int* n_sources) {
  if (L < 1 || S < 1) return ORACLE_EINVAL;
  int nblocks_done = 1; /* blocks = [x] */
  int have_partial = 0;
  int nb = 0;
  if (block_start) block_start[0] = 1;
  for (int l = 1; l <= L; ++l) {
    if (n_sources) n_sources[l - 1] = nblocks_done + (have_partial ? 1 : 0);
    have_partial = 1;
    if (l % S == 0 || l == L) {
      nblocks_done += 1;
      have_partial = 0;
      nb += 1;
      if (block_start) block_start[nb] = l + 1;
    }
  }
  if (n_sources) n_sources[L] = nblocks_done;
  return nb;
}

/* DecoderBlock count -> atomic sublayers per block [K3 9.6 atomic_block_size]:
   layers_per_block <= 0 stands for None, which targets about eight blocks. */
int oracle_atomic_block_size(int num_hidden_layers, int layers_per_block) {
  int per = layers_per_block > 0 ? layers_per_block
                                 : ((num_hidden_layers + 7) / 8 > 1 ? (num_hidden_layers + 7) / 8 : 1);
  return per * 2;
}

typedef struct {
  int64_t D, rows;
  int dtype, L, S, nb;
  const void* x;
  const void* const* v;
  const double* q; /* [L+1][D] */
  double eps;
  double *h, *h_scale, *h_m, *h_lse; /* [L][rows][D], [L][rows] */
  double *y, *y_scale, *y_m, *y_lse; /* [rows][D], [rows] */
  void* block_sums;                  /* [nb][rows][D] dtype */
} stack_ctx;

/* forward_naive for one row [K3 9.3 listing], with the final aggregate
   [K3 9.1, is_final_aggregate]. Scratch: (nb + 1) block rows, the partial,
   and two row temporaries. */
static void stack_rowfn(void* pc, int64_t r, double* scratch) {
  stack_ctx* c = (stack_ctx*)pc;
  const int64_t D = c->D;
  double* blocks = scratch;                        /* [(nb+1)][D] */
  double* partial = blocks + (int64_t)(c->nb + 1) * D;
  double* hrow = partial + D;
  double* srow = hrow + D;
  const double* src[ORACLE_MAX_SOURCES];
  int nblocks = 1, have_partial = 0, closed = 0;
  for (int64_t d = 0; d < D; ++d) blocks[d] = widen(c->x, c->dtype, r * D + d);
  for (int l = 1; l <= c->L; ++l) {
    int n = 0;
    for (int i = 0; i < nblocks; ++i) src[n++] = blocks + (int64_t)i * D;
    if (have_partial) src[n++] = partial;
    double m, lse;
    agg_row(n, src, c->q + (int64_t)(l - 1) * D, D, c->eps, hrow, srow, &m, &lse, NULL);
    int64_t ho = ((int64_t)(l - 1) * c->rows + r);
    if (c->h) memcpy(c->h + ho * D, hrow, (size_t)D * sizeof(double));
    if (c->h_scale) memcpy(c->h_scale + ho * D, srow, (size_t)D * sizeof(double));
    if (c->h_m) c->h_m[ho] = m;
    if (c->h_lse) c->h_lse[ho] = lse;
    /* out = layer(h): the sublayer outputs are given inputs here. */
    const void* v = c->v[l - 1];
    for (int64_t d = 0; d < D; ++d) {
      double vd = widen(v, c->dtype, r * D + d);
      partial[d] = have_partial ? oracle_round(partial[d] + vd, c->dtype) : vd;
    }
    have_partial = 1;
    if (l % c->S == 0 || l == c->L) {
      memcpy(blocks + (int64_t)nblocks * D, partial, (size_t)D * sizeof(double));
      if (c->block_sums)
        for (int64_t d = 0; d < D; ++d)
          store_dtype(c->block_sums, c->dtype, ((int64_t)closed * c->rows + r) * D + d, partial[d]);
      nblocks += 1;
      closed += 1;
      have_partial = 0;
    }
  }
  int n = 0;
  for (int i = 0; i < nblocks; ++i) src[n++] = blocks + (int64_t)i * D;
  agg_row(n, src, c->q + (int64_t)c->L * D, D, c->eps, c->y ? c->y + r * D : NULL,
          c->y_scale ? c->y_scale + r * D : NULL, c->y_m ? c->y_m + r : NULL,
          c->y_lse ? c->y_lse + r : NULL, NULL);
}

/* The naive Block AttnRes stack forward (Full when S == 1) over a set of token
   rows, with the sublayer outputs v_1..v_L given as inputs (eq. (A4) with f_l
   replaced by a table) [K3 9.3 forward_naive; WC "Full AttnRes", "Block
   AttnRes"]. W/Gamma hold L+1 rows: row l-1 is sublayer l's query and row L
   the final aggregate's. Any output pointer may be NULL. */
int oracle_block_stack(int64_t rows, int64_t D, int dtype, int L, int S, const void* x,
                       const void* const* v, const float* W, const float* Gamma, double eps,
                       double* h, double* h_scale, double* h_m, double* h_lse, double* y,
                       double* y_scale, double* y_m, double* y_lse, void* block_sums,
                       int nthreads) {
  if (check_common(rows, D, dtype) || L < 1 || S < 1 || !x || !v || !W) return ORACLE_EINVAL;
  int nb = oracle_block_plan(L, S, NULL, NULL);
  if (nb + 1 > ORACLE_MAX_SOURCES) return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)(L + 1) * (size_t)D * sizeof(double));
  if (!q) return ORACLE_ENOMEM;
  for (int l = 0; l <= L; ++l)
    fold_query(W + (int64_t)l * D, Gamma ? Gamma + (int64_t)l * D : NULL, D, q + (int64_t)l * D);
  stack_ctx c = {D, rows, dtype, L, S, nb, x, v, q, eps, h, h_scale, h_m, h_lse,
                 y, y_scale, y_m, y_lse, block_sums};
  int rc = run_rows(rows, nthreads, stack_rowfn, &c, (size_t)(nb + 4) * (size_t)D);
  free(q);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward of one aggregate (A1)-(A3), with the scores recomputed          */
/* ------------------------------------------------------------------------ */

/* Given the upstream gradient dh of h = sum_i a_i V_i, with
     r_i = sqrt(mean_d V_i^2 + eps),  s_i = q~ . V_i / r_i,  a = softmax(s),
   the chain rule through (A1)-(A3) gives, per row:
     g_i    = dh . V_i                           (dL/da_i)
     ds_i   = a_i (g_i - dh . h)                 (softmax Jacobian)
     dV_i   = a_i dh + ds_i (q~ / r_i - s_i V_i / (D r_i^2))
                                                 (weighted sum, then the score
                                                  through V_i and through r_i)
     dq~    = sum_i ds_i V_i / r_i,
   and, through the fold q~ = w * gamma (its fp32 rounding taken as exact),
     dw = dq~ * gamma,  dgamma = dq~ * w,  summed over rows. */
typedef struct {
  int64_t D;
  int dtype, n;
  const void* const* src;
  const void* dh;
  const double* q;
  double eps;
  double* dV;  /* [n][rows][D] */
  double* dq;  /* [rows][D], per-row dq~ (summed over rows afterwards) */
  int64_t rows;
} bwd_ctx;

static void bwd_rowfn(void* pc, int64_t r, double* scratch) {
  bwd_ctx* c = (bwd_ctx*)pc;
  const int64_t D = c->D;
  const int n = c->n;
  const double* V[ORACLE_MAX_SOURCES];
  double* g = scratch + (int64_t)n * D; /* [D]: dh, then the recomputed h */
  double* h = g + D;
  for (int i = 0; i < n; ++i) {
    double* dst = scratch + (int64_t)i * D;
    for (int64_t d = 0; d < D; ++d) dst[d] = widen(c->src[i], c->dtype, r * D + d);
    V[i] = dst;
  }
  for (int64_t d = 0; d < D; ++d) g[d] = widen(c->dh, c->dtype, r * D + d);
  double a[ORACLE_MAX_SOURCES], s[ORACLE_MAX_SOURCES], rr[ORACLE_MAX_SOURCES];
  agg_row(n, V, c->q, D, c->eps, h, NULL, NULL, NULL, a);
  for (int i = 0; i < n; ++i) {
    double ss = 0.0, dot = 0.0;
    for (int64_t d = 0; d < D; ++d) ss += V[i][d] * V[i][d];
    rr[i] = sqrt(ss / (double)D + c->eps);
    for (int64_t d = 0; d < D; ++d) dot += c->q[d] * V[i][d];
    s[i] = dot / rr[i];
  }
  double gh = 0.0;
  for (int64_t d = 0; d < D; ++d) gh += g[d] * h[d];
  double* dq = c->dq + r * D;
  for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
  for (int i = 0; i < n; ++i) {
    double gi = 0.0;
    for (int64_t d = 0; d < D; ++d) gi += g[d] * V[i][d];
    const double ds = a[i] * (gi - gh);
    double* dv = c->dV + ((int64_t)i * c->rows + r) * D;
    for (int64_t d = 0; d < D; ++d) {
      dv[d] = a[i] * g[d] + ds * (c->q[d] / rr[i] - s[i] * V[i][d] / ((double)D * rr[i] * rr[i]));
      dq[d] += ds * V[i][d] / rr[i];
    }
  }
}

int oracle_aggregate_backward(int64_t rows, int64_t D, int dtype, int n, const void* const* sources,
                              const float* w, const float* gamma, double eps, const void* dh,
                              double* dV, double* dw, double* dgamma, int nthreads) {
  int rc = check_common(rows, D, dtype);
  if (rc) return rc;
  if (n < 1 || n > ORACLE_MAX_SOURCES || !sources || !w || !dh || !dV || !dw) return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)D * sizeof(double));
  double* dq = (double*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)D * sizeof(double));
  if (!q || !dq) {
    free(q);
    free(dq);
    return ORACLE_ENOMEM;
  }
  fold_query(w, gamma, D, q);
  bwd_ctx c = {D, dtype, n, sources, dh, q, eps, dV, dq, rows};
  rc = run_rows(rows, nthreads, bwd_rowfn, &c, (size_t)(n + 2) * (size_t)D);
  if (rc == ORACLE_OK) {
    for (int64_t d = 0; d < D; ++d) {
      double t = 0.0;
      for (int64_t r = 0; r < rows; ++r) t += dq[r * D + d];
      const double g = gamma ? (double)gamma[d] : 1.0;
      dw[d] = t * g;
      if (dgamma) dgamma[d] = t * (double)w[d];
    }
  }
  free(q);
  free(dq);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Merge of a group summary with more sources (the Full two-phase step)     */
/* ------------------------------------------------------------------------ */

/* An earlier group enters as its triple (lse, 1, o) -- normalised output o
   with denominator 1 at the reference point lse [K3 9.4 (OS1)] -- and each new
   source v_i as (s_i, 1, v_i) with s_i its score [K3 (A1)-(A2)]; (OS2) gives
     M = max(lse, s_1..s_n),  Z = e^(lse-M) + sum_i e^(s_i-M),
     h = (e^(lse-M) o + sum_i e^(s_i-M) v_i) / Z,
   the merged statistics m = M, lse' = M + log Z, and the condition scale
   (e^(lse-M) |o| + sum_i e^(s_i-M) |v_i|) / Z. */
typedef struct {
  int64_t D;
  int dtype, n;
  const void* o;
  const float* lse;
  const void* const* src;
  const double* q;
  double eps;
  double *h, *scale, *m, *lse_out;
} merge_ctx;

static void merge_rowfn(void* pc, int64_t r, double* scratch) {
  merge_ctx* c = (merge_ctx*)pc;
  const int64_t D = c->D;
  const double* V[ORACLE_MAX_SOURCES];
  double s[ORACLE_MAX_SOURCES];
  for (int i = 0; i < c->n; ++i) {
    double* dst = scratch + (int64_t)i * D;
    for (int64_t d = 0; d < D; ++d) dst[d] = widen(c->src[i], c->dtype, r * D + d);
    V[i] = dst;
    double one_lse;
    const double* one[1] = {dst};
    agg_row(1, one, c->q, D, c->eps, NULL, NULL, &s[i], &one_lse, NULL); /* m of one source = its score */
  }
  const double la = (double)c->lse[r];
  double mm = la;
  for (int i = 0; i < c->n; ++i) mm = s[i] > mm ? s[i] : mm;
  const double wo = exp(la - mm);
  double z = wo;
  for (int i = 0; i < c->n; ++i) z += exp(s[i] - mm);
  for (int64_t d = 0; d < D; ++d) {
    const double ov = widen(c->o, c->dtype, r * D + d);
    double num = wo * ov, sc = wo * fabs(ov);
    for (int i = 0; i < c->n; ++i) {
      const double a = exp(s[i] - mm);
      num += a * V[i][d];
      sc += a * fabs(V[i][d]);
    }
    if (c->h) c->h[r * D + d] = num / z;
    if (c->scale) c->scale[r * D + d] = sc / z;
  }
  if (c->m) c->m[r] = mm;
  if (c->lse_out) c->lse_out[r] = mm + log(z);
}

int oracle_merge(int64_t rows, int64_t D, int dtype, const void* o, const float* lse, int n,
                 const void* const* sources, const float* w, const float* gamma, double eps,
                 double* h, double* scale, double* m, double* lse_out, int nthreads) {
  int rc = check_common(rows, D, dtype);
  if (rc) return rc;
  if (n < 1 || n > ORACLE_MAX_SOURCES || !o || !lse || !sources || !w) return ORACLE_EINVAL;
  double* q = (double*)malloc((size_t)D * sizeof(double));
  if (!q) return ORACLE_ENOMEM;
  fold_query(w, gamma, D, q);
  merge_ctx c = {D, dtype, n, o, lse, sources, q, eps, h, scale, m, lse_out};
  rc = run_rows(rows, nthreads, merge_rowfn, &c, (size_t)n * (size_t)D);
  free(q);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm: the input norm of the sublayer that consumes an aggregate       */
/* ------------------------------------------------------------------------ */

/* out[r][d] = gamma[d] * x[r][d] / sqrt(mean_d x[r][:]^2 + eps), in fp64 on
   the exactly widened input; rms[r] = sqrt(mean_d x[r][:]^2 + eps). The RMS
   form is the keys' one [WC reference code: eps inside the root, mean over
   the hidden axis]; each sublayer applies it to its input with its own gain
   [ZZ block listing: attn(attn_norm(h)), mlp(mlp_norm(h))]. gamma NULL means
   ones. */
typedef struct {
  int64_t D;
  int dtype;
  const void* x;
  const float* gamma;
  double eps;
  double *out, *rms;
} norm_ctx;

static void norm_rowfn(void* pc, int64_t r, double* scratch) {
  norm_ctx* c = (norm_ctx*)pc;
  const int64_t D = c->D;
  (void)scratch;
  double ss = 0.0;
  for (int64_t d = 0; d < D; ++d) {
    const double v = widen(c->x, c->dtype, r * D + d);
    ss += v * v;
  }
  const double rms = sqrt(ss / (double)D + c->eps);
  for (int64_t d = 0; d < D; ++d) {
    const double g = c->gamma ? (double)c->gamma[d] : 1.0;
    c->out[r * D + d] = g * widen(c->x, c->dtype, r * D + d) / rms;
  }
  if (c->rms) c->rms[r] = rms;
}

int oracle_rmsnorm(int64_t rows, int64_t D, int dtype, const void* x, const float* gamma,
                   double eps, double* out, double* rms, int nthreads) {
  int rc = check_common(rows, D, dtype);
  if (rc) return rc;
  if (!x || !out || !(eps >= 0.0)) return ORACLE_EINVAL;
  norm_ctx c = {D, dtype, x, gamma, eps, out, rms};
  return run_rows(rows, nthreads, norm_rowfn, &c, 1);
}

int oracle_max_sources(void) { return ORACLE_MAX_SOURCES; }
