// api.hip -- the C ABI of libattnres (declared in include/attnres.h).
//
// Host side only: argument validation (everything is checked before anything
// is enqueued), the integer block plan, workspace carving, the two-phase
// Block stack orchestration with its sublayer callback, and optional launch
// timing. All device work is in kernels.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "attnres.h"
#include "launch.hpp"

#define ATTNRES_API extern "C" __attribute__((visibility("default")))

using attnres::AggArgs;
using attnres::BwdArgs;
using attnres::MergeBwdArgs;
using attnres::BwdPlan;
using attnres::Launch;
using attnres::Phase1Args;
using attnres::Phase2Args;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTNRES_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize_of(int dtype) { return dtype == ATTNRES_BF16 ? 2 : dtype == ATTNRES_F32 ? 4 : 0; }

// Common [R,D] shape checks.
int check_shape(const char* fn, int64_t R, int64_t D, int dtype, float eps) {
  const int es = esize_of(dtype);
  if (!es) return fail(ATTNRES_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (R < 0) return fail(ATTNRES_EINVAL, "%s: R = %lld < 0", fn, (long long)R);
  if (D < 1 || (D * es) % 16 != 0)
    return fail(ATTNRES_EINVAL, "%s: D = %lld must be >= 1 with D*%d a multiple of 16 bytes", fn,
                (long long)D, es);
  if (D * es > ATTNRES_MAX_ROW_BYTES)
    return fail(ATTNRES_EUNSUPPORTED, "%s: row of %lld bytes exceeds %d", fn, (long long)(D * es),
                ATTNRES_MAX_ROW_BYTES);
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(ATTNRES_EINVAL, "%s: eps must be finite and >= 0", fn);
  return ATTNRES_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, bool required) {
  if (!p) return required ? fail(ATTNRES_EINVAL, "%s: %s is NULL", fn, name) : ATTNRES_OK;
  if (!aligned16(p)) return fail(ATTNRES_EINVAL, "%s: %s is not 16-byte aligned", fn, name);
  return ATTNRES_OK;
}

#define TRY(expr)                      \
  do {                                 \
    int rc_ = (expr);                  \
    if (rc_ != ATTNRES_OK) return rc_; \
  } while (0)

// ---------------------------------------------------------------------------
// launch timing (instrumentation)
// ---------------------------------------------------------------------------
enum Kind {
  K_PHASE1 = 0,
  K_PHASE2 = 1,
  K_AGG = 2,
  K_CLOSE = 3,
  K_FOLD = 4,
  K_NORM = 5,
  K_BWD = 6,
  K_BWD_REDUCE = 7,
  K_PHASE1_STATS = 8,
  K_COUNT = 9
};

// the kernel a kind's launches run, unless the launch names another
const char* kind_kernel(int kind) {
  switch (kind) {
    case K_PHASE2: return "phase2_kernel";
    case K_AGG: return "aggregate_kernel";
    case K_CLOSE: return "close_kernel";
    case K_FOLD: return "fold_kernel";
    case K_NORM: return "rmsnorm_kernel";
    case K_BWD: return "aggregate_bwd_kernel";
    case K_BWD_REDUCE: return "bwd_colsum_kernel";
    default: return "phase1_kernel";
  }
}

struct Timing {
  int capacity = 0;
  std::vector<hipEvent_t> ev;  // 2 per slot: the kernel's start and end
  std::vector<int> kind;
  std::vector<double> bytes;
  std::vector<const char*> name;  // kernel(s) of the slot's launch
  std::vector<hipStream_t> stream;
  std::string names[K_COUNT];     // distinct kernel names per kind, comma-separated
  // the last collected launches in record order: kind, stream and start / end
  // relative to the first one's start (ms)
  struct Span {
    int kind;
    uintptr_t stream;
    double start, end;
  };
  std::vector<Span> trace;
  int used = 0;
  bool paused = false;
  int64_t launches[K_COUNT] = {0};
  double ms[K_COUNT] = {0};
  double total_bytes[K_COUNT] = {0};
};
thread_local Timing g_timing;

// The Launch of one kernel: when timing is on and a slot is free, it carries
// an event pair that the dispatch itself stamps (no extra queue packets).
Launch timed_launch(int kind, double bytes, hipStream_t st, const char* kernel = nullptr) {
  Launch L{st, nullptr, nullptr};
  Timing& t = g_timing;
  if (t.capacity > 0 && !t.paused && t.used < t.capacity) {
    const int slot = t.used++;
    t.kind[slot] = kind;
    t.bytes[slot] = bytes;
    t.name[slot] = kernel ? kernel : kind_kernel(kind);
    t.stream[slot] = st;
    L.start = t.ev[2 * slot];
    L.stop = t.ev[2 * slot + 1];
  }
  return L;
}

int hip_fail(const char* fn, hipError_t e) {
  return fail(ATTNRES_EHIP, "%s: %s", fn, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// the kernel families with their algorithmic byte accounting: inputs read
// once plus outputs written once; a fused block close counts its reference
// traffic (p and v read, b written) in the launch that performs it
// ---------------------------------------------------------------------------
double close_bytes(double rb, const void* close_p, const void* close_v) {
  // the reference close reads p and v and writes b; the launch's own read of
  // b as a source is counted with its sources (the fusion saves that read)
  return close_v ? rb * (close_p ? 3 : 2) : 0.0;
}

int do_aggregate(const char* fn, int dtype, const AggArgs& a, hipStream_t st) {
  if (a.R == 0) return ATTNRES_OK;
  const double rb = (double)a.R * a.D * esize_of(dtype);
  const double bytes = rb * (a.n + 1) + (double)a.R * ((a.m_out ? 4 : 0) + (a.lse_out ? 4 : 0)) +
                       close_bytes(rb, a.close_p, a.close_v) +
                       (a.o_init ? rb + (double)a.R * 4 : 0.0);
  hipError_t e = attnres::launch_aggregate(dtype, a, timed_launch(K_AGG, bytes, st));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
}

int do_close(const char* fn, const void* p, const void* v, void* b, int64_t R, int64_t D,
             int dtype, hipStream_t st) {
  if (R == 0) return ATTNRES_OK;
  const double rb = (double)R * D * esize_of(dtype);
  hipError_t e = attnres::launch_close(dtype, p, v, b, R, D, timed_launch(K_CLOSE, rb * (p ? 3 : 2), st));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
}

int do_rmsnorm(const char* fn, int dtype, const void* x, int64_t R, int64_t D, const float* g,
               float eps, void* out, hipStream_t st);

// whether do_phase1 takes the scores/outputs passes for this launch
bool takes_gemm(int dtype, const Phase1Args& a) {
  return a.gemm_ws && attnres::phase1_gemm_eligible(dtype, a.n, a.S, a.D, a.R);
}

int do_phase1(const char* fn, int dtype, const Phase1Args& a, hipStream_t st) {
  if (a.R == 0) return ATTNRES_OK;
  const int64_t row_bytes = a.D * esize_of(dtype);
  // output 0's input norm, where the kernel that runs does not write it
  auto norm_after = [&]() -> int {
    if (!a.nf_out) return ATTNRES_OK;
    return do_rmsnorm(fn, dtype, a.out ? a.out : a.src[0], a.R, a.D, a.nf_g, a.nf_eps, a.nf_out, st);
  };
  if (takes_gemm(dtype, a)) {
    // the scores pass reads materialised sources: close first
    if (a.close_v) TRY(do_close(fn, a.close_p, a.close_v, a.close_b, a.R, a.D, dtype, st));
    Phase1Args g = a;
    g.close_p = nullptr;
    g.close_v = nullptr;
    g.close_b = nullptr;
    const double rb = (double)a.R * row_bytes;
    const double bytes = rb * (a.n + (a.out ? a.S : 0)) + (double)a.R * a.S * ((a.m_out ? 4 : 0) + 4);
    hipError_t e = attnres::launch_phase1_gemm(
        g, a.gemm_ws, timed_launch(a.out ? K_PHASE1 : K_PHASE1_STATS, bytes, st,
                                   attnres::phase1_kernel_name(dtype, g, true)));
    if (e != hipSuccess) return hip_fail(fn, e);
    return norm_after();
  }
  if (attnres::phase1_supported(dtype, a.n, a.S, a.D)) {
    const bool fused = a.nf_out && attnres::phase1_norm_fused(dtype, a, false);
    Phase1Args b = a;
    if (!fused) b.nf_out = nullptr;
    const double rb = (double)a.R * row_bytes;
    const double bytes = rb * (a.n + (a.out ? a.S : 0) + (fused && !a.out ? 1 : 0)) +
                         (double)a.R * a.S * ((a.m_out ? 4 : 0) + 4) + close_bytes(rb, a.close_p, a.close_v);
    hipError_t e = attnres::launch_phase1(
        dtype, b, timed_launch(a.out ? K_PHASE1 : K_PHASE1_STATS, bytes, st,
                               attnres::phase1_kernel_name(dtype, a, false)));
    if (e != hipSuccess) return hip_fail(fn, e);
    return fused ? ATTNRES_OK : norm_after();
  }
  // More sources than the register-resident pass holds: close separately,
  // then one aggregate per query.
  if (a.close_v) TRY(do_close(fn, a.close_p, a.close_v, a.close_b, a.R, a.D, dtype, st));
  for (int s = 0; s < a.S; ++s) {
    AggArgs g{a.src, a.n, a.R, a.D, a.W + (int64_t)s * a.D, a.G ? a.G + (int64_t)s * a.D : nullptr,
              a.eps, static_cast<char*>(a.out) + (int64_t)s * a.R * row_bytes,
              a.m_out ? a.m_out + (int64_t)s * a.R : nullptr, a.lse_out + (int64_t)s * a.R,
              nullptr, nullptr, nullptr};
    if (s == 0) {  // the aggregate kernel writes output 0's input norm itself
      g.nf_g = a.nf_g;
      g.nf_eps = a.nf_eps;
      g.nf_out = a.nf_out;
    }
    TRY(do_aggregate(fn, dtype, g, st));
  }
  return ATTNRES_OK;
}

int do_phase2(const char* fn, int dtype, const Phase2Args& a, hipStream_t st) {
  if (a.R == 0) return ATTNRES_OK;
  const double rb = (double)a.R * a.D * esize_of(dtype);
  const int writes = (a.h_out ? 1 : 0) + (a.hn_out ? 1 : 0);
  const double bytes = rb * ((a.p_prev ? 4 : 2) + (a.xs ? 1 : 0) + writes) + (double)a.R * 4;
  hipError_t e = attnres::launch_phase2(dtype, a, timed_launch(K_PHASE2, bytes, st));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
}

int do_rmsnorm(const char* fn, int dtype, const void* x, int64_t R, int64_t D, const float* g,
               float eps, void* out, hipStream_t st) {
  if (R == 0) return ATTNRES_OK;
  const double bytes = 2.0 * (double)R * D * esize_of(dtype);
  hipError_t e = attnres::launch_rmsnorm(dtype, x, R, D, g, eps, out, timed_launch(K_NORM, bytes, st));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
}

// The folded queries q~ = w * gamma of all L+1 aggregations [K3 9.2 (1)],
// formed once per forward into `ws_q`; without gains q~ is w itself, read in
// place (no launch).
int fold_queries(const char* fn, const float* W, const float* Gamma, int L, int64_t D, float* ws_q,
                 hipStream_t st, const float** Q) {
  if (!Gamma) {
    *Q = W;
    return ATTNRES_OK;
  }
  hipError_t e = attnres::launch_fold(W, Gamma, ws_q, (int64_t)(L + 1) * D,
                                      timed_launch(K_FOLD, (double)(L + 1) * D * 12, st));
  if (e != hipSuccess) return hip_fail(fn, e);
  *Q = ws_q;
  return ATTNRES_OK;
}

// ---------------------------------------------------------------------------
// block plan [K3 9.3 forward_naive]
// ---------------------------------------------------------------------------
int plan(int L, int S, int* block_start, int* n_sources) {
  int completed = 1, partial = 0, nb = 0;
  if (block_start) block_start[0] = 1;
  for (int l = 1; l <= L; ++l) {
    if (n_sources) n_sources[l - 1] = completed + partial;
    partial = 1;
    if (l % S == 0 || l == L) {
      ++completed;
      partial = 0;
      ++nb;
      if (block_start) block_start[nb] = l + 1;
    }
  }
  if (n_sources) n_sources[L] = completed;
  return nb;
}

// workspace layout of the stack forward, each region 256-byte aligned
struct StackLayout {
  size_t q, o, m, lse, p, h, g, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

StackLayout stack_layout(int L, int S, int64_t R, int64_t D, int es) {
  StackLayout s;
  const int Sk = S < L ? S : L;  // widest block
  const size_t row = (size_t)R * (size_t)D * es;
  size_t off = 0;
  s.q = off; off = align256(off + (size_t)(L + 1) * D * sizeof(float));
  s.o = off; off = align256(off + (Sk > 1 ? (size_t)Sk * row : 0));
  s.m = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.lse = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.p = off; off = align256(off + (Sk > 2 ? row : 0));
  s.h = off; off = align256(off + row);
  // the scores/outputs Phase 1 (query parts and softmax weights) where some
  // block's Phase 1 takes it (block k scores over k sources, up to nb)
  s.g = off;
  const int ng = attnres::phase1_gemm_needed(es == 2 ? 1 : 0, Sk, D, R, plan(L, S, nullptr, nullptr));
  if (ng) off = align256(off + attnres::phase1_gemm_workspace(Sk, R, D, ng));
  s.total = off;
  return s;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

ATTNRES_API const char* attnres_status_string(int code) {
  switch (code) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_EINVAL: return "invalid argument";
    case ATTNRES_EUNSUPPORTED: return "unsupported by this build";
    case ATTNRES_EWORKSPACE: return "workspace too small";
    case ATTNRES_EHIP: return "HIP runtime error";
    case ATTNRES_ECALLBACK: return "sublayer callback failed";
    default: return "unknown status";
  }
}

ATTNRES_API const char* attnres_last_error(void) { return g_last_error.c_str(); }

ATTNRES_API int attnres_aggregate(const void* const* sources, int n, int64_t R, int64_t D,
                                  int dtype, const float* w, const float* gamma, float eps,
                                  void* out, float* m_out, float* lse_out, void* stream) {
  const char* fn = "attnres_aggregate";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (!sources) return fail(ATTNRES_EINVAL, "%s: sources is NULL", fn);
  if (n < 1 || n > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: n = %d outside 1..%d", fn, n, ATTNRES_MAX_SOURCES);
  if (R == 0) return ok();  // nothing is accessed
  for (int i = 0; i < n; ++i) {
    TRY(check_ptr(fn, "sources[i]", sources[i], true));
    if (sources[i] == out) return fail(ATTNRES_EINVAL, "%s: out aliases sources[%d]", fn, i);
  }
  TRY(check_ptr(fn, "w", w, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "out", out, true));
  TRY(check_ptr(fn, "m_out", m_out, false));
  TRY(check_ptr(fn, "lse_out", lse_out, false));
  AggArgs a{sources, n, R, D, w, gamma, eps, out, m_out, lse_out, nullptr, nullptr, nullptr};
  TRY(do_aggregate(fn, dtype, a, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_phase1_batched(const void* const* blocks, int n, int64_t R, int64_t D,
                                       int dtype, const float* W, const float* Gamma, int S,
                                       float eps, void* out, float* m_out, float* lse_out,
                                       void* stream) {
  const char* fn = "attnres_phase1_batched";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (!blocks) return fail(ATTNRES_EINVAL, "%s: blocks is NULL", fn);
  if (n < 1 || n > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: n = %d outside 1..%d", fn, n, ATTNRES_MAX_SOURCES);
  if (S < 1 || S > 1024) return fail(ATTNRES_EINVAL, "%s: S = %d outside 1..1024", fn, S);
  if (R == 0) return ok();
  for (int i = 0; i < n; ++i) TRY(check_ptr(fn, "blocks[i]", blocks[i], true));
  TRY(check_ptr(fn, "W", W, true));
  TRY(check_ptr(fn, "Gamma", Gamma, false));
  TRY(check_ptr(fn, "out", out, true));
  TRY(check_ptr(fn, "m_out", m_out, false));
  TRY(check_ptr(fn, "lse_out", lse_out, true));
  Phase1Args a{blocks, n, R, D, W, Gamma, S, eps, out, m_out, lse_out, nullptr, nullptr, nullptr};
  TRY(do_phase1(fn, dtype, a, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_phase2_merge(const void* o, const float* lse, const float* w,
                                     const float* gamma, float eps, const void* p_prev,
                                     const void* v_prev, void* p_out, void* h_out, int64_t R,
                                     int64_t D, int dtype, void* stream) {
  const char* fn = "attnres_phase2_merge";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (R == 0) return ok();
  TRY(check_ptr(fn, "o", o, true));
  TRY(check_ptr(fn, "lse", lse, true));
  TRY(check_ptr(fn, "w", w, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "p_prev", p_prev, false));
  TRY(check_ptr(fn, "v_prev", v_prev, true));
  TRY(check_ptr(fn, "p_out", p_out, p_prev != nullptr));
  TRY(check_ptr(fn, "h_out", h_out, true));
  if (!p_prev && p_out) return fail(ATTNRES_EINVAL, "%s: p_out must be NULL when p_prev is NULL", fn);
  if (h_out == o || h_out == p_prev || h_out == v_prev || h_out == p_out)
    return fail(ATTNRES_EINVAL, "%s: h_out aliases an input or p_out", fn);
  if (p_out && (p_out == o || p_out == v_prev))
    return fail(ATTNRES_EINVAL, "%s: p_out aliases o or v_prev", fn);
  Phase2Args a{o, lse, w, gamma, eps, p_prev, v_prev, p_out, h_out, nullptr, 0.f, nullptr, R, D};
  TRY(do_phase2(fn, dtype, a, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_phase2_merge_norm(const void* o, const float* lse, const float* w,
                                          const float* gamma, float eps, const void* p_prev,
                                          const void* v_prev, void* p_out, void* h_out,
                                          const float* gamma_f, float eps_f, void* hn_out,
                                          int64_t R, int64_t D, int dtype, void* stream) {
  const char* fn = "attnres_phase2_merge_norm";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (!std::isfinite(eps_f) || eps_f < 0.f)
    return fail(ATTNRES_EINVAL, "%s: eps_f must be finite and >= 0", fn);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "o", o, true));
  TRY(check_ptr(fn, "lse", lse, true));
  TRY(check_ptr(fn, "w", w, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "p_prev", p_prev, false));
  TRY(check_ptr(fn, "v_prev", v_prev, true));
  TRY(check_ptr(fn, "p_out", p_out, p_prev != nullptr));
  TRY(check_ptr(fn, "h_out", h_out, false));
  TRY(check_ptr(fn, "gamma_f", gamma_f, false));
  TRY(check_ptr(fn, "hn_out", hn_out, true));
  if (!p_prev && p_out) return fail(ATTNRES_EINVAL, "%s: p_out must be NULL when p_prev is NULL", fn);
  for (const void* out : {h_out, hn_out}) {
    if (!out) continue;
    if (out == o || out == p_prev || out == v_prev || out == p_out)
      return fail(ATTNRES_EINVAL, "%s: h_out or hn_out aliases an input or p_out", fn);
  }
  if (h_out && h_out == hn_out) return fail(ATTNRES_EINVAL, "%s: h_out and hn_out alias", fn);
  if (p_out && (p_out == o || p_out == v_prev))
    return fail(ATTNRES_EINVAL, "%s: p_out aliases o or v_prev", fn);
  Phase2Args a{o, lse, w, gamma, eps, p_prev, v_prev, p_out, h_out, gamma_f, eps_f, hn_out, R, D};
  TRY(do_phase2(fn, dtype, a, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_rmsnorm(const void* x, int64_t R, int64_t D, int dtype, const float* gamma,
                                float eps, void* out, void* stream) {
  const char* fn = "attnres_rmsnorm";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "out", out, true));
  TRY(do_rmsnorm(fn, dtype, x, R, D, gamma, eps, out, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_table_sublayer(void* ctx, int l, const void* h_l, const void** v_out,
                                       void* stream) {
  (void)h_l;
  (void)stream;
  if (!ctx || !v_out || l < 1) return 1;
  *v_out = static_cast<const void* const*>(ctx)[l - 1];
  return 0;
}

ATTNRES_API int attnres_block_layout(int L, int S, int* block_start, int* n_sources) {
  if (L < 1 || S < 1) return fail(ATTNRES_EINVAL, "attnres_block_layout: L and S must be >= 1");
  return plan(L, S, block_start, n_sources);
}

ATTNRES_API int attnres_atomic_block_size(int num_decoder_layers, int layers_per_block) {
  if (num_decoder_layers < 1)
    return fail(ATTNRES_EINVAL, "attnres_atomic_block_size: num_decoder_layers must be >= 1");
  int per = layers_per_block > 0 ? layers_per_block : (num_decoder_layers + 7) / 8;
  if (per < 1) per = 1;
  return 2 * per;
}

ATTNRES_API size_t attnres_stack_workspace_bytes(int L, int S, int64_t R, int64_t D, int dtype) {
  const int es = esize_of(dtype);
  if (!es || L < 1 || S < 1 || R < 0 || D < 1) return 0;
  return stack_layout(L, S, R, D, es).total;
}

namespace {

// The output norm handed to the sublayers, when the stack runs with one: the
// callback for sublayer l receives RMSNorm(h_l) * Gamma_f[l-1] instead of h_l.
struct OutNorm {
  bool on;
  const float* Gamma_f;  // [L, D] or null (ones)
  float eps_f;
};

int stack_forward(const char* fn, const void* x, int L, int S, int64_t R, int64_t D, int dtype,
                  const float* W, const float* Gamma, float eps, attnres_sublayer_fn f, void* f_ctx,
                  void* const* block_sums, void* y, void* workspace, size_t workspace_bytes,
                  const OutNorm& nm, void* stream);

}  // namespace

ATTNRES_API int attnres_block_stack_forward(const void* x, int L, int S, int64_t R, int64_t D,
                                            int dtype, const float* W, const float* Gamma,
                                            float eps, attnres_sublayer_fn f, void* f_ctx,
                                            void* const* block_sums, void* y, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return stack_forward("attnres_block_stack_forward", x, L, S, R, D, dtype, W, Gamma, eps, f, f_ctx,
                       block_sums, y, workspace, workspace_bytes, OutNorm{false, nullptr, 0.f}, stream);
}

ATTNRES_API int attnres_block_stack_forward_norm(const void* x, int L, int S, int64_t R, int64_t D,
                                                 int dtype, const float* W, const float* Gamma,
                                                 float eps, const float* Gamma_f, float eps_f,
                                                 attnres_sublayer_fn f, void* f_ctx,
                                                 void* const* block_sums, void* y, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  const char* fn = "attnres_block_stack_forward_norm";
  if (!std::isfinite(eps_f) || eps_f < 0.f)
    return fail(ATTNRES_EINVAL, "%s: eps_f must be finite and >= 0", fn);
  if (R > 0) TRY(check_ptr(fn, "Gamma_f", Gamma_f, false));
  return stack_forward(fn, x, L, S, R, D, dtype, W, Gamma, eps, f, f_ctx, block_sums, y, workspace,
                       workspace_bytes, OutNorm{true, Gamma_f, eps_f}, stream);
}

namespace {

int stack_forward_overlap(const char* fn, const void* x, int L, int S, int64_t R, int64_t D,
                          int dtype, const float* W, const float* Gamma, float eps,
                          attnres_sublayer_fn f, void* f_ctx, void* const* block_sums, void* y,
                          void* workspace, size_t workspace_bytes, const OutNorm& nm, void* stream,
                          void* side_stream);
struct OverlapLayout;
size_t overlap_total(int L, int S, int64_t R, int64_t D, int es);

}  // namespace

ATTNRES_API size_t attnres_stack_overlap_workspace_bytes(int L, int S, int64_t R, int64_t D,
                                                         int dtype) {
  const int es = esize_of(dtype);
  if (!es || L < 1 || S < 1 || R < 0 || D < 1) return 0;
  return overlap_total(L, S, R, D, es);
}

ATTNRES_API int attnres_block_stack_forward_overlap(const void* x, int L, int S, int64_t R,
                                                    int64_t D, int dtype, const float* W,
                                                    const float* Gamma, float eps, int out_norm,
                                                    const float* Gamma_f, float eps_f,
                                                    attnres_sublayer_fn f, void* f_ctx,
                                                    void* const* block_sums, void* y,
                                                    void* workspace, size_t workspace_bytes,
                                                    void* stream, void* side_stream) {
  const char* fn = "attnres_block_stack_forward_overlap";
  if (out_norm) {
    if (!std::isfinite(eps_f) || eps_f < 0.f)
      return fail(ATTNRES_EINVAL, "%s: eps_f must be finite and >= 0", fn);
    if (R > 0) TRY(check_ptr(fn, "Gamma_f", Gamma_f, false));
  }
  return stack_forward_overlap(fn, x, L, S, R, D, dtype, W, Gamma, eps, f, f_ctx, block_sums, y,
                               workspace, workspace_bytes,
                               OutNorm{out_norm != 0, out_norm ? Gamma_f : nullptr, eps_f}, stream,
                               side_stream);
}

namespace {

int stack_forward(const char* fn, const void* x, int L, int S, int64_t R, int64_t D, int dtype,
                  const float* W, const float* Gamma, float eps, attnres_sublayer_fn f, void* f_ctx,
                  void* const* block_sums, void* y, void* workspace, size_t workspace_bytes,
                  const OutNorm& nm, void* stream) {
  TRY(check_shape(fn, R, D, dtype, eps));
  if (L < 1 || S < 1) return fail(ATTNRES_EINVAL, "%s: L = %d and S = %d must be >= 1", fn, L, S);
  const int nb = plan(L, S, nullptr, nullptr);
  if (nb + 1 > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: %d blocks plus the embedding exceed %d sources", fn, nb,
                ATTNRES_MAX_SOURCES);
  if (R == 0) return ok();  // nothing is accessed and no sublayer is called
  TRY(check_ptr(fn, "x", x, true));
  TRY(check_ptr(fn, "W", W, true));
  TRY(check_ptr(fn, "Gamma", Gamma, false));
  TRY(check_ptr(fn, "y", y, true));
  if (!f) return fail(ATTNRES_EINVAL, "%s: sublayer callback is NULL", fn);
  if (!block_sums && S != 1)
    return fail(ATTNRES_EINVAL, "%s: block_sums may be NULL only when S == 1", fn);
  if (block_sums)
    for (int k = 0; k < nb; ++k) TRY(check_ptr(fn, "block_sums[k]", block_sums[k], true));
  const int es = esize_of(dtype);
  const StackLayout lay = stack_layout(L, S, R, D, es);
  if (!workspace) return fail(ATTNRES_EINVAL, "%s: workspace is NULL", fn);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTNRES_EINVAL, "%s: workspace is not 256-byte aligned", fn);
  if (workspace_bytes < lay.total)
    return fail(ATTNRES_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                lay.total);

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  char* O = ws + lay.o;
  float* M = reinterpret_cast<float*>(ws + lay.m);
  float* LSE = reinterpret_cast<float*>(ws + lay.lse);
  void* P = ws + lay.p;
  void* H = ws + lay.h;
  const int64_t tensor_bytes = R * D * es;

  const float* Q = nullptr;
  TRY(fold_queries(fn, W, Gamma, L, D, reinterpret_cast<float*>(ws + lay.q), st, &Q));

  auto call = [&](int l, const void* h, const void** v) -> int {
    const void* out = nullptr;
    const int rc = f(f_ctx, l, h, &out, stream);
    if (rc != 0)
      return fail(ATTNRES_ECALLBACK, "%s: sublayer callback returned %d at l = %d", fn, rc, l);
    if (!out || !aligned16(out))
      return fail(ATTNRES_ECALLBACK, "%s: callback gave a NULL or misaligned v at l = %d", fn, l);
    *v = out;
    return ATTNRES_OK;
  };

  // src[0..k] are the completed sources seen by block k. The close of block
  // k-1 (b_k = p + v_last) is fused into block k's first launch, which forms
  // b_k from (p, v_last) as its last source and stores it to block_sums[k-1].
  std::vector<const void*> src;
  src.reserve(nb + 1);
  src.push_back(x);
  const void* close_p = nullptr;
  const void* close_v = nullptr;
  void* close_b = nullptr;

  for (int k = 0; k < nb; ++k) {
    const int start = k * S + 1;
    const int end = (k + 1) * S < L ? (k + 1) * S : L;
    const int Sk = end - start + 1;
    const int n = k + 1;
    const float* Qk = Q + (int64_t)(start - 1) * D;
    if (Sk == 1) {
      // a one-sublayer block: a single aggregate over the completed sources
      AggArgs a{src.data(), n, R, D, Qk, nullptr, eps, H, nullptr, nullptr,
                close_p, close_v, close_b};
      if (nm.on) {  // the aggregate writes its sublayer's input norm to H itself
        a.nf_g = nm.Gamma_f ? nm.Gamma_f + (int64_t)(start - 1) * D : nullptr;
        a.nf_eps = nm.eps_f;
        a.nf_out = H;
      }
      TRY(do_aggregate(fn, dtype, a, st));
      const void* v = nullptr;
      TRY(call(start, H, &v));
      if (block_sums) {  // b_{k+1} = v, copied by the next launch
        close_p = nullptr;
        close_v = v;
        close_b = block_sums[k];
        src.push_back(block_sums[k]);
      } else {  // S == 1 without block_sums: the outputs themselves are the sources
        close_v = nullptr;
        src.push_back(v);
      }
      continue;
    }
    // Phase 1: the block's Sk queries over [b_0 .. b_k] in one pass. With the
    // embedding as the only source every weight is exactly 1, so each output
    // o_s is b_0 itself: only the statistics are computed and b_0 stands in
    // for the outputs.
    const bool one_source = n == 1 && !close_v && attnres::phase1_stats_supported(dtype, 1, Sk, D);
    auto o_slice = [&](int j) -> const void* {
      return one_source ? src[0] : static_cast<const void*>(O + (int64_t)j * tensor_bytes);
    };
    Phase1Args a1{src.data(), n, R, D, Qk, nullptr, Sk, eps, one_source ? nullptr : O, M, LSE,
                  close_p, close_v, close_b, lay.g < lay.total ? ws + lay.g : nullptr};
    if (nm.on) {  // output 0's input norm to H, fused where the Phase-1 kernel allows
      a1.nf_g = nm.Gamma_f ? nm.Gamma_f + (int64_t)(start - 1) * D : nullptr;
      a1.nf_eps = nm.eps_f;
      a1.nf_out = H;
    }
    // Outputs 0 and 1 straight into H and P where the kernel allows: those
    // two are rewritten for every sublayer and stay in the last-level cache,
    // slices of O do not. P's last reader is this launch's close, which
    // reads each row before the row's outputs are written; output 1 is read
    // once, by the first merge, which writes no partial.
    // (P has room only where some block has more than two sublayers.)
    const bool o01 = !one_source && attnres::phase1_out01_supported(dtype, a1, takes_gemm(dtype, a1));
    const bool o0_in_h = o01 && !nm.on;
    const bool o1_in_p = o01 && (S < L ? S : L) > 2;
    if (o0_in_h) a1.out0 = H;
    if (o1_in_p) a1.out1 = P;
    auto o_at = [&](int j) -> const void* { return j == 1 && o1_in_p ? P : o_slice(j); };
    TRY(do_phase1(fn, dtype, a1, st));
    const void* v_first = nullptr;
    // h_start = o_0: no partial yet
    TRY(call(start, nm.on || o0_in_h ? H : o_slice(0), &v_first));
    const void* p_cur = v_first;    // p_1 = v_start (aliased, no copy)
    const void* v_prev = v_first;
    for (int j = 1; j < Sk; ++j) {
      const int l = start + j;
      Phase2Args a2{o_at(j), LSE + (int64_t)j * R, Q + (int64_t)(l - 1) * D,
                    nullptr, eps, j == 1 ? nullptr : p_cur, v_prev, j == 1 ? nullptr : P,
                    nm.on ? nullptr : H,
                    nm.on && nm.Gamma_f ? nm.Gamma_f + (int64_t)(l - 1) * D : nullptr, nm.eps_f,
                    nm.on ? H : nullptr, R, D};
      TRY(do_phase2(fn, dtype, a2, st));
      if (j > 1) p_cur = P;
      const void* v = nullptr;
      TRY(call(l, H, &v));
      v_prev = v;
    }
    // b_{k+1} = p + v_end, formed by the next launch
    close_p = p_cur;
    close_v = v_prev;
    close_b = block_sums[k];
    src.push_back(block_sums[k]);
  }
  // final aggregate over [b_0 .. b_nb] [K3 9.1 is_final_aggregate]
  AggArgs af{src.data(), nb + 1, R, D, Q + (int64_t)L * D, nullptr, eps, y, nullptr, nullptr,
             close_p, close_v, close_b};
  TRY(do_aggregate(fn, dtype, af, st));
  return ok();
}

// ---------------------------------------------------------------------------
// The decode schedule: block k+1's Phase 1 runs on a side stream while block
// k's sublayers run on the main stream [WC "Kimi Linear and K3 integration",
// decode: the batched inter-block pass on a side stream]. The merge of
// source groups is exact [K3 9.4 (OS2)], so that Phase 1 needs only the
// sources that exist when block k starts, [b_0 .. b_k]; the block sum
// b_{k+1} that block k closes with is merged in afterwards as one more
// single-source term: block k+1's first sublayer gets OS2((lse_0, o_0),
// b_{k+1}) from one launch that also performs the close, and each further
// sublayer's Phase-2 step merges three terms, (lse_j, o_j), b_{k+1} and the
// partial. Two Phase-1 slots alternate between the streams.
// ---------------------------------------------------------------------------
#ifndef ATTNRES_OVERLAP_SIDE_GROUPS
#define ATTNRES_OVERLAP_SIDE_GROUPS 128  // workgroup budget of a side-stream Phase 1: half the CUs
#endif

struct OverlapLayout {
  size_t q, o[2], m[2], lse[2], p, h, g, total;
};

OverlapLayout overlap_layout(int L, int S, int64_t R, int64_t D, int es) {
  OverlapLayout s;
  const int Sk = S < L ? S : L;  // widest block
  const size_t row = (size_t)R * (size_t)D * es;
  size_t off = 0;
  s.q = off; off = align256(off + (size_t)(L + 1) * D * sizeof(float));
  for (int b = 0; b < 2; ++b) {
    s.o[b] = off; off = align256(off + (size_t)Sk * row);
    s.m[b] = off; off = align256(off + (size_t)Sk * R * sizeof(float));
    s.lse[b] = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  }
  s.p = off; off = align256(off + (Sk > 2 ? row : 0));
  s.h = off; off = align256(off + row);
  s.g = off;
  const int ng = attnres::phase1_gemm_needed(es == 2 ? 1 : 0, Sk, D, R, plan(L, S, nullptr, nullptr));
  if (ng) off = align256(off + attnres::phase1_gemm_workspace(Sk, R, D, ng));
  s.total = off;
  return s;
}

size_t overlap_total(int L, int S, int64_t R, int64_t D, int es) {
  return overlap_layout(L, S, R, D, es).total;
}

// The two ordering events of the decode schedule, per thread and device,
// created at first use and reused by every later call (timing disabled).
struct OverlapEvents {
  hipEvent_t main_ready = nullptr;  // main stream: the sources and the next slot are ready
  hipEvent_t side_done = nullptr;   // side stream: a block's Phase 1 is written
};
thread_local OverlapEvents g_overlap_events[64];

int overlap_events(const char* fn, int dev, OverlapEvents** out) {
  if (dev < 0 || dev >= 64)
    return fail(ATTNRES_EUNSUPPORTED, "%s: device %d beyond the 64 this build tracks", fn, dev);
  OverlapEvents& e = g_overlap_events[dev];
  for (hipEvent_t* ev : {&e.main_ready, &e.side_done}) {
    if (*ev) continue;
    hipError_t rc = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (rc != hipSuccess) {
      *ev = nullptr;
      return hip_fail(fn, rc);
    }
  }
  *out = &e;
  return ATTNRES_OK;
}

int stream_device(const char* fn, hipStream_t st, int* dev) {
  hipError_t e;
  if (st) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(st, &d);
    *dev = (int)d;
  } else {
    e = hipGetDevice(dev);
  }
  return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
}

int stack_forward_overlap(const char* fn, const void* x, int L, int S, int64_t R, int64_t D,
                          int dtype, const float* W, const float* Gamma, float eps,
                          attnres_sublayer_fn f, void* f_ctx, void* const* block_sums, void* y,
                          void* workspace, size_t workspace_bytes, const OutNorm& nm, void* stream,
                          void* side_stream) {
  TRY(check_shape(fn, R, D, dtype, eps));
  if (L < 1 || S < 1) return fail(ATTNRES_EINVAL, "%s: L = %d and S = %d must be >= 1", fn, L, S);
  const int nb = plan(L, S, nullptr, nullptr);
  if (nb + 1 > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: %d blocks plus the embedding exceed %d sources", fn, nb,
                ATTNRES_MAX_SOURCES);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, true));
  TRY(check_ptr(fn, "W", W, true));
  TRY(check_ptr(fn, "Gamma", Gamma, false));
  TRY(check_ptr(fn, "y", y, true));
  if (!f) return fail(ATTNRES_EINVAL, "%s: sublayer callback is NULL", fn);
  if (!block_sums) return fail(ATTNRES_EINVAL, "%s: block_sums is NULL", fn);
  for (int k = 0; k < nb; ++k) TRY(check_ptr(fn, "block_sums[k]", block_sums[k], true));
  if (!side_stream || side_stream == stream)
    return fail(ATTNRES_EINVAL, "%s: side_stream must be a stream other than stream", fn);
  const int es = esize_of(dtype);
  const OverlapLayout lay = overlap_layout(L, S, R, D, es);
  if (!workspace) return fail(ATTNRES_EINVAL, "%s: workspace is NULL", fn);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTNRES_EINVAL, "%s: workspace is not 256-byte aligned", fn);
  if (workspace_bytes < lay.total)
    return fail(ATTNRES_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                lay.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStream_t side = static_cast<hipStream_t>(side_stream);
  int dev_main = -1, dev_side = -1;
  TRY(stream_device(fn, st, &dev_main));
  TRY(stream_device(fn, side, &dev_side));
  if (dev_main != dev_side)
    return fail(ATTNRES_EINVAL, "%s: stream is on device %d, side_stream on device %d", fn,
                dev_main, dev_side);
  OverlapEvents* ev = nullptr;
  TRY(overlap_events(fn, dev_main, &ev));

  char* ws = static_cast<char*>(workspace);
  void* P = ws + lay.p;
  void* H = ws + lay.h;
  void* gemm_ws = lay.g < lay.total ? ws + lay.g : nullptr;
  const int64_t tensor_bytes = R * D * es;
  auto hip_ok = [&](hipError_t e) { return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e); };

  const float* Q = nullptr;
  TRY(fold_queries(fn, W, Gamma, L, D, reinterpret_cast<float*>(ws + lay.q), st, &Q));
  // with the norm, a block's first launch writes its first sublayer's input
  // norm RMSNorm(h) * Gamma_f[l-1] to H itself
  auto with_norm = [&](int l, auto& args) {
    if (!nm.on) return;
    args.nf_g = nm.Gamma_f ? nm.Gamma_f + (int64_t)(l - 1) * D : nullptr;
    args.nf_eps = nm.eps_f;
    args.nf_out = H;
  };
  auto call = [&](int l, const void* h, const void** v) -> int {
    const void* out = nullptr;
    const int rc = f(f_ctx, l, h, &out, stream);
    if (rc != 0)
      return fail(ATTNRES_ECALLBACK, "%s: sublayer callback returned %d at l = %d", fn, rc, l);
    if (!out || !aligned16(out))
      return fail(ATTNRES_ECALLBACK, "%s: callback gave a NULL or misaligned v at l = %d", fn, l);
    *v = out;
    return ATTNRES_OK;
  };
  auto block_range = [&](int k, int* start, int* Sk) {
    *start = k * S + 1;
    const int end = (k + 1) * S < L ? (k + 1) * S : L;
    *Sk = end - *start + 1;
  };

  std::vector<const void*> src;
  src.reserve(nb + 1);
  src.push_back(x);
  // Phase 1 of block k over the first n = k completed sources into slot k & 1
  // (for k == 0, over [b_0] on the main stream). Returns, through one_source,
  // whether the outputs were elided (one source: each output is b_0 itself).
  bool one_src[2] = {false, false};
  auto phase1_into_slot = [&](int k, int n, hipStream_t on, bool norm0 = false) -> int {
    int start, Sk;
    block_range(k, &start, &Sk);
    const int b = k & 1;
    char* O = ws + lay.o[b];
    float* M = reinterpret_cast<float*>(ws + lay.m[b]);
    float* LSE = reinterpret_cast<float*>(ws + lay.lse[b]);
    const float* Qk = Q + (int64_t)(start - 1) * D;
    if (Sk == 1) {
      one_src[b] = false;
      AggArgs a{src.data(), n, R, D, Qk, nullptr, eps, O, nullptr, LSE, nullptr, nullptr, nullptr};
      return do_aggregate(fn, dtype, a, on);
    }
    one_src[b] = n == 1 && attnres::phase1_stats_supported(dtype, 1, Sk, D);
    Phase1Args a1{src.data(), n, R, D, Qk, nullptr, Sk, eps, one_src[b] ? nullptr : O, M, LSE,
                  nullptr, nullptr, nullptr, gemm_ws};
    // off the critical path, Phase 1 leaves most of the chip to the main stream
    if (on != st) a1.max_groups = ATTNRES_OVERLAP_SIDE_GROUPS;
    if (norm0) with_norm(start, a1);
    return do_phase1(fn, dtype, a1, on);
  };
  auto o_slice = [&](int k, int j) -> const void* {
    const int b = k & 1;
    return one_src[b] ? src[0] : static_cast<const void*>(ws + lay.o[b] + (int64_t)j * tensor_bytes);
  };
  auto lse_slice = [&](int k, int j) -> const float* {
    return reinterpret_cast<const float*>(ws + lay.lse[k & 1]) + (int64_t)j * R;
  };

  const void* close_p = nullptr;
  const void* close_v = nullptr;
  for (int k = 0; k < nb; ++k) {
    int start, Sk;
    block_range(k, &start, &Sk);
    const void* xs = nullptr;  // the newest completed source, merged as its own term
    if (k == 0) {
      // block 0: its Phase 1 over [b_0] on the main stream, then (when a next
      // block exists) the side stream starts block 1's Phase 1 over [b_0]
      if (Sk == 1) {
        AggArgs a{src.data(), 1, R, D, Q, nullptr, eps, H, nullptr, nullptr, nullptr, nullptr, nullptr};
        with_norm(start, a);
        TRY(do_aggregate(fn, dtype, a, st));
      } else {
        TRY(phase1_into_slot(0, 1, st, true));
      }
      if (nb > 1) {
        TRY(hip_ok(hipEventRecord(ev->main_ready, st)));
        TRY(hip_ok(hipStreamWaitEvent(side, ev->main_ready, 0)));
        TRY(phase1_into_slot(1, 1, side));
        TRY(hip_ok(hipEventRecord(ev->side_done, side)));
      }
    } else {
      // block k: its Phase 1 over [b_0 .. b_{k-1}] ran on the side stream;
      // close b_k = p + v_last and merge it into query 0's summary
      TRY(hip_ok(hipStreamWaitEvent(st, ev->side_done, 0)));
      src.push_back(block_sums[k - 1]);
      xs = block_sums[k - 1];
      AggArgs am{src.data() + k, 1, R, D, Q + (int64_t)(start - 1) * D, nullptr, eps, H, nullptr,
                 nullptr, close_p, close_v, block_sums[k - 1], o_slice(k, 0), lse_slice(k, 0)};
      with_norm(start, am);
      TRY(do_aggregate(fn, dtype, am, st));
      if (k + 1 < nb) {
        // b_k is stored and slot (k+1) & 1 was last read by block k-1:
        // block k+1's Phase 1 over [b_0 .. b_k] can start
        TRY(hip_ok(hipEventRecord(ev->main_ready, st)));
        TRY(hip_ok(hipStreamWaitEvent(side, ev->main_ready, 0)));
        TRY(phase1_into_slot(k + 1, k + 1, side));
        TRY(hip_ok(hipEventRecord(ev->side_done, side)));
      }
    }
    const void* h0 = (k == 0 && Sk > 1 && !nm.on) ? o_slice(0, 0) : H;
    const void* v_first = nullptr;
    TRY(call(start, h0, &v_first));
    const void* p_cur = v_first;
    const void* v_prev = v_first;
    for (int j = 1; j < Sk; ++j) {
      const int l = start + j;
      Phase2Args a2{o_slice(k, j), lse_slice(k, j), Q + (int64_t)(l - 1) * D,
                    nullptr, eps, j == 1 ? nullptr : p_cur, v_prev, j == 1 ? nullptr : P,
                    nm.on ? nullptr : H,
                    nm.on && nm.Gamma_f ? nm.Gamma_f + (int64_t)(l - 1) * D : nullptr, nm.eps_f,
                    nm.on ? H : nullptr, R, D, xs};
      TRY(do_phase2(fn, dtype, a2, st));
      if (j > 1) p_cur = P;
      const void* v = nullptr;
      TRY(call(l, H, &v));
      v_prev = v;
    }
    // b_{k+1} = p + v_end (or v alone for a one-sublayer block), formed by
    // the next block's first launch or the final aggregate
    close_p = Sk > 1 ? p_cur : nullptr;
    close_v = v_prev;
  }
  src.push_back(block_sums[nb - 1]);
  AggArgs af{src.data(), nb + 1, R, D, Q + (int64_t)L * D, nullptr, eps, y, nullptr, nullptr,
             close_p, close_v, block_sums[nb - 1]};
  TRY(do_aggregate(fn, dtype, af, st));
  return ok();
}

// Full AttnRes with a two-phase schedule [K3 9.4: with schedule_block_size
// the Full mixer runs the two-phase algorithm and matches the naive one]:
// sublayers are taken in chunks of C; Phase 1 scores a chunk's queries over
// every source that exists before the chunk in one pass, and sublayer j of
// the chunk merges that summary with the j outputs produced inside the
// chunk so far, each its own softmax term (OS2 over individual sources).
struct FullLayout {
  size_t q, o, m, lse, h, g, total;
};

FullLayout full_layout(int L, int C, int64_t R, int64_t D, int es) {
  FullLayout f;
  const int Ck = C < L ? C : L;
  const size_t row = (size_t)R * (size_t)D * es;
  size_t off = 0;
  f.q = off; off = align256(off + (size_t)(L + 1) * D * sizeof(float));
  f.o = off; off = align256(off + (Ck > 1 ? (size_t)Ck * row : 0));
  f.m = off; off = align256(off + (size_t)Ck * R * sizeof(float));
  f.lse = off; off = align256(off + (size_t)Ck * R * sizeof(float));
  f.h = off; off = align256(off + row);
  // the scores/outputs Phase 1 where some chunk takes it: the chunk from
  // sublayer s0 scores over s0 sources
  f.g = off;
  int nmax = 0;
  for (int s0 = 1; s0 <= L; s0 += C)
    if (L - s0 + 1 >= 2 && C >= 2) nmax = s0;
  const int ng = nmax > 0 ? attnres::phase1_gemm_needed(es == 2 ? 1 : 0, Ck, D, R, nmax) : 0;
  if (ng) off = align256(off + attnres::phase1_gemm_workspace(Ck, R, D, ng));
  f.total = off;
  return f;
}

}  // namespace

ATTNRES_API size_t attnres_full_workspace_bytes(int L, int C, int64_t R, int64_t D, int dtype) {
  const int es = esize_of(dtype);
  if (!es || L < 1 || C < 1 || R < 0 || D < 1) return 0;
  return full_layout(L, C, R, D, es).total;
}

ATTNRES_API int attnres_merge_sources(const void* o, const float* lse, const void* const* sources,
                                      int n, int64_t R, int64_t D, int dtype, const float* w,
                                      const float* gamma, float eps, void* out, float* m_out,
                                      float* lse_out, void* stream) {
  const char* fn = "attnres_merge_sources";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (n < 1 || n > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: n = %d outside [1, %d]", fn, n, ATTNRES_MAX_SOURCES);
  if (!sources) return fail(ATTNRES_EINVAL, "%s: sources is NULL", fn);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "o", o, true));
  TRY(check_ptr(fn, "lse", lse, true));
  for (int i = 0; i < n; ++i) TRY(check_ptr(fn, "sources[i]", sources[i], true));
  TRY(check_ptr(fn, "w", w, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "out", out, true));
  TRY(check_ptr(fn, "m_out", m_out, false));
  TRY(check_ptr(fn, "lse_out", lse_out, false));
  if (out == o) return fail(ATTNRES_EINVAL, "%s: out aliases o", fn);
  for (int i = 0; i < n; ++i)
    if (out == sources[i]) return fail(ATTNRES_EINVAL, "%s: out aliases a source", fn);
  AggArgs a{sources, n, R, D, w, gamma, eps, out, m_out, lse_out, nullptr, nullptr, nullptr, o, lse};
  TRY(do_aggregate(fn, dtype, a, static_cast<hipStream_t>(stream)));
  return ok();
}

ATTNRES_API int attnres_full_stack_forward(const void* x, int L, int C, int64_t R, int64_t D,
                                           int dtype, const float* W, const float* Gamma, float eps,
                                           attnres_sublayer_fn f, void* f_ctx, void* y,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "attnres_full_stack_forward";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (L < 1 || C < 1) return fail(ATTNRES_EINVAL, "%s: L = %d and C = %d must be >= 1", fn, L, C);
  if (L + 1 > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: L + 1 = %d sources exceed %d", fn, L + 1, ATTNRES_MAX_SOURCES);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, true));
  TRY(check_ptr(fn, "W", W, true));
  TRY(check_ptr(fn, "Gamma", Gamma, false));
  TRY(check_ptr(fn, "y", y, true));
  if (!f) return fail(ATTNRES_EINVAL, "%s: sublayer callback is NULL", fn);
  const int es = esize_of(dtype);
  const FullLayout lay = full_layout(L, C, R, D, es);
  if (!workspace) return fail(ATTNRES_EINVAL, "%s: workspace is NULL", fn);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTNRES_EINVAL, "%s: workspace is not 256-byte aligned", fn);
  if (workspace_bytes < lay.total)
    return fail(ATTNRES_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                lay.total);

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  char* O = ws + lay.o;
  float* M = reinterpret_cast<float*>(ws + lay.m);
  float* LSE = reinterpret_cast<float*>(ws + lay.lse);
  void* H = ws + lay.h;
  void* gemm_ws = lay.g < lay.total ? ws + lay.g : nullptr;
  const int64_t tensor_bytes = R * D * es;
  const float* Q = nullptr;
  TRY(fold_queries(fn, W, Gamma, L, D, reinterpret_cast<float*>(ws + lay.q), st, &Q));
  auto call = [&](int l, const void* h, const void** v) -> int {
    const void* out = nullptr;
    const int rc = f(f_ctx, l, h, &out, stream);
    if (rc != 0)
      return fail(ATTNRES_ECALLBACK, "%s: sublayer callback returned %d at l = %d", fn, rc, l);
    if (!out || !aligned16(out))
      return fail(ATTNRES_ECALLBACK, "%s: callback gave a NULL or misaligned v at l = %d", fn, l);
    *v = out;
    return ATTNRES_OK;
  };

  // src = [x, v_1, ..., v_{l-1}]: every sublayer output is a source of its own
  std::vector<const void*> src;
  src.reserve(L + 1);
  src.push_back(x);
  for (int s0 = 1; s0 <= L; s0 += C) {
    const int e0 = s0 + C - 1 < L ? s0 + C - 1 : L;
    const int Ck = e0 - s0 + 1;
    const int n = (int)src.size();  // = s0
    const float* Qk = Q + (int64_t)(s0 - 1) * D;
    if (Ck == 1) {
      AggArgs a{src.data(), n, R, D, Qk, nullptr, eps, H, nullptr, nullptr, nullptr, nullptr, nullptr};
      TRY(do_aggregate(fn, dtype, a, st));
      const void* v = nullptr;
      TRY(call(s0, H, &v));
      src.push_back(v);
      continue;
    }
    // the first chunk sees only the embedding: its outputs are x itself
    const bool one_source = n == 1 && attnres::phase1_stats_supported(dtype, 1, Ck, D);
    auto o_slice = [&](int j) -> const void* {
      return one_source ? src[0] : static_cast<const void*>(O + (int64_t)j * tensor_bytes);
    };
    Phase1Args a1{src.data(), n, R, D, Qk, nullptr, Ck, eps, one_source ? nullptr : O, M, LSE,
                  nullptr, nullptr, nullptr, gemm_ws};
    TRY(do_phase1(fn, dtype, a1, st));
    const void* v = nullptr;
    TRY(call(s0, o_slice(0), &v));  // the first sublayer of the chunk: h = o_0
    src.push_back(v);
    for (int j = 1; j < Ck; ++j) {
      const int l = s0 + j;
      // merge (lse_j, o_j) with the chunk's outputs v_{s0} .. v_{l-1}
      AggArgs am{src.data() + n, j, R, D, Q + (int64_t)(l - 1) * D, nullptr, eps, H, nullptr, nullptr,
                 nullptr, nullptr, nullptr, o_slice(j), LSE + (int64_t)j * R};
      TRY(do_aggregate(fn, dtype, am, st));
      TRY(call(l, H, &v));
      src.push_back(v);
    }
  }
  AggArgs af{src.data(), L + 1, R, D, Q + (int64_t)L * D, nullptr, eps, y, nullptr, nullptr,
             nullptr, nullptr, nullptr};
  TRY(do_aggregate(fn, dtype, af, st));
  return ok();
}

ATTNRES_API size_t attnres_aggregate_backward_workspace_bytes(int64_t R, int64_t D, int dtype) {
  if (!esize_of(dtype) || R < 0 || D < 1) return 0;
  return attnres::plan_aggregate_bwd(dtype, R, D).bytes;
}

namespace {

// Every argument of the aggregate backward except its workspace, checked
// before anything is enqueued; fills the launch plan.
int validate_backward(const char* fn, const void* const* sources, int n, int64_t R, int64_t D,
                      int dtype, const float* w, const float* gamma, float eps, const void* dh,
                      float* const* dV, float* dw, float* dgamma, BwdPlan* plan) {
  TRY(check_shape(fn, R, D, dtype, eps));
  if (n < 1 || n > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: n = %d outside 1..%d", fn, n, ATTNRES_MAX_SOURCES);
  // dw / dgamma are produced even for R == 0
  TRY(check_ptr(fn, "w", w, true));
  TRY(check_ptr(fn, "gamma", gamma, false));
  TRY(check_ptr(fn, "dw", dw, true));
  TRY(check_ptr(fn, "dgamma", dgamma, false));
  if (dgamma && dgamma == dw) return fail(ATTNRES_EINVAL, "%s: dgamma aliases dw", fn);
  *plan = attnres::plan_aggregate_bwd(dtype, R, D);
  if (!plan->supported) return fail(ATTNRES_EUNSUPPORTED, "%s: D = %lld", fn, (long long)D);
  if (R > 0) {
    if (!sources) return fail(ATTNRES_EINVAL, "%s: sources is NULL", fn);
    if (!dV) return fail(ATTNRES_EINVAL, "%s: dV is NULL", fn);
    TRY(check_ptr(fn, "dh", dh, true));
    for (int i = 0; i < n; ++i) {
      TRY(check_ptr(fn, "sources[i]", sources[i], true));
      TRY(check_ptr(fn, "dV[i]", dV[i], true));
      const void* d = dV[i];
      if (d == dh || d == w || d == gamma || d == dw || d == dgamma)
        return fail(ATTNRES_EINVAL, "%s: dV[%d] aliases another argument", fn, i);
      for (int j = 0; j < n; ++j)
        if (d == sources[j] || (j < i && d == dV[j]))
          return fail(ATTNRES_EINVAL, "%s: dV[%d] aliases a source or another dV", fn, i);
    }
  }
  return ATTNRES_OK;
}

// The backward's three launches: the main kernel (dV and the per-workgroup
// dq~ partials in the workspace), then the two fixed-order reduction stages.
int launch_backward(const char* fn, int dtype, const BwdArgs& a, const BwdPlan& pl,
                    hipStream_t st) {
  const double rb = (double)a.R * a.D * esize_of(dtype);
  const double gb = (double)a.R * a.D * 4 * a.n * (a.accumulate ? 2 : 1);
  hipError_t e = attnres::launch_aggregate_bwd(dtype, a, pl, timed_launch(K_BWD, rb * (a.n + 1) + gb, st));
  if (e != hipSuccess) return hip_fail(fn, e);
  const double pbytes = (double)pl.P * a.D * 4;
  if (pl.P2) {
    e = attnres::launch_bwd_reduce(a, pl, 0, timed_launch(K_BWD_REDUCE, pbytes + pl.P2 * a.D * 4.0, st));
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  const double fin = (double)(pl.P2 ? pl.P2 : pl.P) * a.D * 4 +
                     a.D * 4.0 * ((a.dgamma ? 2 : 1) * (a.accumulate ? 2 : 1));
  e = attnres::launch_bwd_reduce(a, pl, 1, timed_launch(K_BWD_REDUCE, fin, st));
  if (e != hipSuccess) return hip_fail(fn, e);
  return ATTNRES_OK;
}

}  // namespace

ATTNRES_API int attnres_aggregate_backward(const void* const* sources, int n, int64_t R, int64_t D,
                                           int dtype, const float* w, const float* gamma, float eps,
                                           const void* dh, float* const* dV, int accumulate,
                                           float* dw, float* dgamma, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  const char* fn = "attnres_aggregate_backward";
  BwdPlan pl;
  TRY(validate_backward(fn, sources, n, R, D, dtype, w, gamma, eps, dh, dV, dw, dgamma, &pl));
  if (pl.bytes > 0) {
    TRY(check_ptr(fn, "workspace", workspace, true));
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(ATTNRES_EINVAL, "%s: workspace is not 256-byte aligned", fn);
    if (workspace_bytes < pl.bytes)
      return fail(ATTNRES_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                  workspace_bytes, pl.bytes);
  }
  BwdArgs a{sources, n, R, D, w, gamma, eps, dh, dV, accumulate, dw, dgamma, workspace};
  TRY(launch_backward(fn, dtype, a, pl, static_cast<hipStream_t>(stream)));
  return ok();
}

// ---------------------------------------------------------------------------
// The aggregate backward without a workspace argument, for callers that
// cannot allocate. Its dq~ partials live in `scratch`, a device array of a
// fixed size that the HIP runtime places on each GPU when it loads this
// library's code there and keeps until the process ends. On the host the
// name `scratch` is only a stand-in for the array: its device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ATTNRES_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until looked up

// The device address of `scratch` on the device that `stream` runs on, which
// must be the calling thread's current device.
int scratch_address(const char* fn, hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (sd != cur)
      return fail(ATTNRES_EINVAL, "%s: the stream belongs to device %d, but device %d is current", fn,
                  (int)sd, cur);
  }
  if (cur < 0 || cur >= kMaxDevices)
    return fail(ATTNRES_EUNSUPPORTED, "%s: device %d beyond the %d this build tracks", fn, cur,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!p) return fail(ATTNRES_EHIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return ATTNRES_OK;
}

}  // namespace

ATTNRES_API size_t attnres_noalloc_scratch_bytes(void) { return ATTNRES_NOALLOC_SCRATCH_BYTES; }

ATTNRES_API int attnres_aggregate_backward_noalloc(const void* const* sources, int n, int64_t R,
                                                   int64_t D, int dtype, const float* w,
                                                   const float* gamma, float eps, const void* dh,
                                                   float* const* dV, int accumulate, float* dw,
                                                   float* dgamma, void* stream) {
  const char* fn = "attnres_aggregate_backward_noalloc";
  BwdPlan pl;
  TRY(validate_backward(fn, sources, n, R, D, dtype, w, gamma, eps, dh, dV, dw, dgamma, &pl));
  if (pl.bytes > (size_t)ATTNRES_NOALLOC_SCRATCH_BYTES)
    return fail(ATTNRES_EUNSUPPORTED,
                "%s: D = %lld needs %zu bytes of scratch, above the fixed %zu; use "
                "attnres_aggregate_backward with a workspace",
                fn, (long long)D, pl.bytes, (size_t)ATTNRES_NOALLOC_SCRATCH_BYTES);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  TRY(scratch_address(fn, st, &ws));
  BwdArgs a{sources, n, R, D, w, gamma, eps, dh, dV, accumulate, dw, dgamma, ws};
  TRY(launch_backward(fn, dtype, a, pl, st));
  return ok();
}

// ---------------------------------------------------------------------------
// Backward of the Block stack through the two-phase schedule, with
// recomputation [K3 9.1 (A1)-(A3), 9.4 (OS1)-(OS2) differentiated; WC
// "Depth attention & online merge reference" and "Public implementation
// boundary": forward and backward with online softmax and recomputation].
// ---------------------------------------------------------------------------
namespace {

struct BwdStackLayout {
  size_t o, m, lse, p, a, dl, g, gbytes, bw, total;
};

BwdStackLayout bwd_stack_layout(int L, int S, int64_t R, int64_t D, int dtype) {
  BwdStackLayout s;
  const int es = esize_of(dtype);
  const int Sk = S < L ? S : L;
  const size_t row = (size_t)R * (size_t)D * es;
  size_t off = 0;
  s.o = off; off = align256(off + (size_t)Sk * row);
  s.m = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.lse = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.p = off; off = align256(off + (Sk > 2 ? (size_t)(Sk - 2) * row : 0));
  s.a = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.dl = off; off = align256(off + (size_t)Sk * R * sizeof(float));
  s.g = off;
  s.gbytes = 0;
  const int ng = attnres::phase1_gemm_needed(dtype, Sk, D, R, plan(L, S, nullptr, nullptr));
  if (ng) s.gbytes = attnres::phase1_gemm_workspace(Sk, R, D, ng);
  off = align256(off + s.gbytes);
  {
    // one aggregate backward's plan, or one per merge of a block (its dq~
    // partials reduced together), or the batched Phase-1 backward's
    const size_t a = attnres::plan_aggregate_bwd(dtype, R, D).bytes;
    const size_t am = Sk > 1 ? (size_t)(Sk - 1) * a : a;
    const size_t b = attnres::phase1_bwd_workspace(R, D);
    const size_t ab = am > a ? am : a;
    s.bw = off; off = align256(off + (ab > b ? ab : b));
  }
  s.total = off;
  return s;
}

}  // namespace

ATTNRES_API int attnres_table_sublayer_bwd(void* ctx, int l, const float* dv_l, const void** dh_out,
                                           void* stream) {
  (void)dv_l;
  (void)stream;
  if (!ctx || !dh_out || l < 1) return 1;
  *dh_out = static_cast<const void* const*>(ctx)[l - 1];
  return 0;
}

ATTNRES_API size_t attnres_stack_backward_workspace_bytes(int L, int S, int64_t R, int64_t D,
                                                          int dtype) {
  if (!esize_of(dtype) || L < 1 || S < 1 || R < 0 || D < 1) return 0;
  return bwd_stack_layout(L, S, R, D, dtype).total;
}

ATTNRES_API int attnres_block_stack_backward(
    const void* x, const void* const* v, int L, int S, int64_t R, int64_t D, int dtype,
    const float* W, const float* Gamma, float eps, const void* const* block_sums, const void* dy,
    attnres_sublayer_bwd_fn fb, void* fb_ctx, float* dx, float* const* dv, float* dW, float* dGamma,
    void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "attnres_block_stack_backward";
  TRY(check_shape(fn, R, D, dtype, eps));
  if (L < 1 || S < 1) return fail(ATTNRES_EINVAL, "%s: L = %d and S = %d must be >= 1", fn, L, S);
  const int nb = plan(L, S, nullptr, nullptr);
  if (nb + 1 > ATTNRES_MAX_SOURCES)
    return fail(ATTNRES_EINVAL, "%s: %d blocks plus the embedding exceed %d sources", fn, nb,
                ATTNRES_MAX_SOURCES);
  const BwdPlan pl = attnres::plan_aggregate_bwd(dtype, R, D);
  if (!pl.supported) return fail(ATTNRES_EUNSUPPORTED, "%s: D = %lld", fn, (long long)D);
  TRY(check_ptr(fn, "W", W, true));
  TRY(check_ptr(fn, "Gamma", Gamma, false));
  TRY(check_ptr(fn, "dW", dW, true));
  TRY(check_ptr(fn, "dGamma", dGamma, false));
  if (dGamma && !Gamma) return fail(ATTNRES_EINVAL, "%s: dGamma requires Gamma", fn);
  if (R > 0) {
    TRY(check_ptr(fn, "x", x, true));
    TRY(check_ptr(fn, "dy", dy, true));
    TRY(check_ptr(fn, "dx", dx, true));
    if (!v || !dv) return fail(ATTNRES_EINVAL, "%s: v and dv are required", fn);
    for (int l = 0; l < L; ++l) {
      TRY(check_ptr(fn, "v[l]", v[l], true));
      TRY(check_ptr(fn, "dv[l]", dv[l], true));
      if ((const void*)dv[l] == (const void*)dx)
        return fail(ATTNRES_EINVAL, "%s: dv[%d] aliases dx", fn, l);
      for (int m = 0; m < l; ++m)
        if (dv[m] == dv[l]) return fail(ATTNRES_EINVAL, "%s: dv[%d] aliases dv[%d]", fn, l, m);
    }
    if (!block_sums && S != 1)
      return fail(ATTNRES_EINVAL, "%s: block_sums may be NULL only when S == 1", fn);
    if (block_sums)
      for (int k = 0; k < nb; ++k) TRY(check_ptr(fn, "block_sums[k]", block_sums[k], true));
    if (!fb) return fail(ATTNRES_EINVAL, "%s: sublayer backward callback is NULL", fn);
  }
  const BwdStackLayout lay = bwd_stack_layout(L, S, R, D, dtype);
  if (!workspace) return fail(ATTNRES_EINVAL, "%s: workspace is NULL", fn);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(ATTNRES_EINVAL, "%s: workspace is not 256-byte aligned", fn);
  if (workspace_bytes < lay.total)
    return fail(ATTNRES_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                lay.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* bw = ws + lay.bw;
  const int64_t tensor_bytes = R * D * esize_of(dtype);
  const double rb = (double)R * D * esize_of(dtype), gb = (double)R * D * 4;
  auto qrow = [&](const float* M0, int l) -> const float* { return M0 ? M0 + (int64_t)(l - 1) * D : nullptr; };
  auto frow = [&](float* M0, int l) -> float* { return M0 ? M0 + (int64_t)(l - 1) * D : nullptr; };

  // the reductions of the query gradient (dq~ partials in bw -> dw, dgamma)
  auto reduce_q = [&](const float* w, const float* g, float* dw_, float* dg_, int acc) -> int {
    BwdArgs a{nullptr, 0, R, D, w, g, eps, nullptr, nullptr, acc, dw_, dg_, bw};
    const double pbytes = (double)pl.P * D * 4;
    hipError_t e;
    if (pl.P2) {
      e = attnres::launch_bwd_reduce(a, pl, 0, timed_launch(K_BWD_REDUCE, pbytes + pl.P2 * D * 4.0, st));
      if (e != hipSuccess) return hip_fail(fn, e);
    }
    e = attnres::launch_bwd_reduce(
        a, pl, 1, timed_launch(K_BWD_REDUCE, (double)(pl.P2 ? pl.P2 : pl.P) * D * 4 + D * 4.0 * (dg_ ? 2 : 1), st));
    return e == hipSuccess ? ATTNRES_OK : hip_fail(fn, e);
  };
  // one aggregate backward over srcs[0..n) into their gradients g[0..n)
  auto agg_bwd = [&](const void* const* srcs, float* const* grads, int n, int l, const void* dh,
                     const float* scale, const float* dlse, int acc_v, int acc_q) -> int {
    BwdArgs a{srcs, n, R, D, qrow(W, l), qrow(Gamma, l), eps, dh, grads, acc_v, frow(dW, l),
              frow(dGamma, l), bw, scale, dlse, acc_q};
    hipError_t e = attnres::launch_aggregate_bwd(
        dtype, a, pl, timed_launch(K_BWD, rb * (n + 1) + gb * n * (acc_v ? 2 : 1), st));
    if (e != hipSuccess) return hip_fail(fn, e);
    return reduce_q(qrow(W, l), qrow(Gamma, l), frow(dW, l), frow(dGamma, l), acc_q);
  };
  auto callback = [&](int l, const float* dvl, const void** dh) -> int {
    const void* out = nullptr;
    const int rc = fb(fb_ctx, l, dvl, &out, stream);
    if (rc != 0)
      return fail(ATTNRES_ECALLBACK, "%s: sublayer backward callback returned %d at l = %d", fn, rc, l);
    if (!out || !aligned16(out))
      return fail(ATTNRES_ECALLBACK, "%s: callback gave a NULL or misaligned dh at l = %d", fn, l);
    *dh = out;
    return ATTNRES_OK;
  };

  if (R == 0) {
    // no rows: every query gradient is zero (the reductions over no rows)
    for (int l = 1; l <= L + 1; ++l)
      TRY(reduce_q(qrow(W, l), qrow(Gamma, l), frow(dW, l), frow(dGamma, l), 0));
    return ok();
  }

  // block k's completed sources b_0..b_k and their gradients: b_0 = x with
  // gradient dx; b_k (k >= 1) is the sum of block k-1's outputs, and its
  // gradient is exactly that of block k-1's last output, dv[end_{k-1} - 1]
  std::vector<const void*> b(nb + 1);
  std::vector<float*> db(nb + 1);
  b[0] = x;
  db[0] = dx;
  for (int k = 0; k < nb; ++k) {
    const int end = (k + 1) * S < L ? (k + 1) * S : L;
    b[k + 1] = block_sums ? block_sums[k] : v[k];  // S == 1 without sums: b_{k+1} = v_{k+1}
    db[k + 1] = dv[end - 1];
  }

  // the final aggregate y = AGG(b_0 .. b_nb; q~_{L+1}) writes every db first
  TRY(agg_bwd(b.data(), db.data(), nb + 1, L + 1, dy, nullptr, nullptr, 0, 0));

  for (int k = nb - 1; k >= 0; --k) {
    const int start = k * S + 1;
    const int end = (k + 1) * S < L ? (k + 1) * S : L;
    const int Sk = end - start + 1;
    const int n = k + 1;
    std::vector<const void*> dh(Sk, nullptr);
    // db_{k+1} = dv_end is complete: the sublayer's own backward gives dh_end
    TRY(callback(end, dv[end - 1], &dh[Sk - 1]));
    if (Sk == 1) {
      // a one-sublayer block: h = AGG(b_0 .. b_k)
      TRY(agg_bwd(b.data(), db.data(), n, start, dh[0], nullptr, nullptr, 1, 0));
      continue;
    }
    // recompute the block's Phase 1 (o_j, lse_j) and its partials p_2 .. p_{Sk-1};
    // only queries 1 .. Sk-1 are needed (the merges'; the Phase-1 backward forms
    // its own softmax), so query 0's output is not written again
    const bool one_source = n == 1 && attnres::phase1_stats_supported(dtype, 1, Sk - 1, D);
    char* O = ws + lay.o;
    float* LSE = reinterpret_cast<float*>(ws + lay.lse);
    float* A = reinterpret_cast<float*>(ws + lay.a);
    float* DL = reinterpret_cast<float*>(ws + lay.dl);
    {
      const float* Wk = W + (int64_t)start * D;
      const float* Gk = Gamma ? Gamma + (int64_t)start * D : nullptr;
      Phase1Args a1{b.data(), n, R, D, Wk, Gk, Sk - 1, eps, one_source ? nullptr : O + tensor_bytes,
                    reinterpret_cast<float*>(ws + lay.m) + R, LSE + R, nullptr, nullptr, nullptr,
                    lay.gbytes ? ws + lay.g : nullptr};
      TRY(do_phase1(fn, dtype, a1, st));
    }
    auto o_slice = [&](int j) -> const void* {
      return one_source ? b[0] : static_cast<const void*>(O + (int64_t)j * tensor_bytes);
    };
    auto p_slice = [&](int j) -> const void* {  // the partial seen by sublayer start + j (j >= 1)
      return j == 1 ? v[start - 1] : static_cast<const void*>(ws + lay.p + (int64_t)(j - 2) * tensor_bytes);
    };
    if (Sk >= 3 && Sk - 1 <= attnres::kPartialsMax) {
      // p_2 .. p_{Sk-1} in one pass over v_start .. v_{start+Sk-2}
      std::vector<const void*> in(Sk - 1);
      std::vector<void*> out(Sk - 1, nullptr);
      for (int t = 0; t < Sk - 1; ++t) in[t] = v[start - 1 + t];
      for (int t = 1; t < Sk - 1; ++t) out[t] = const_cast<void*>(p_slice(t + 1));
      hipError_t e = attnres::launch_partials(
          dtype, in.data(), out.data(), Sk - 1, R, D,
          timed_launch(K_CLOSE, (double)R * D * esize_of(dtype) * (2 * Sk - 3), st, "partials_kernel"));
      if (e != hipSuccess) return hip_fail(fn, e);
    } else {
      for (int j = 2; j < Sk; ++j)
        TRY(do_close(fn, p_slice(j - 1), v[start + j - 2], const_cast<void*>(p_slice(j)), R, D, dtype, st));
    }
    // Phase-2 merges in reverse: sublayer start + j merged (lse_j, o_j) with p_j;
    // its backward turns dh into the gradient of p_j, which (with the gradient
    // from the partial's later uses, dv[start + j - 1]) is that of v_{start+j-1}
    // (each merge's dq~ partials in a slot of their own, reduced together below)
    for (int j = Sk - 1; j >= 1; --j) {
      const int l = start + j;
      MergeBwdArgs mb{o_slice(j), LSE + (int64_t)j * R, p_slice(j), qrow(W, l), qrow(Gamma, l), eps,
                      dh[j], dv[l - 1], dv[l - 2], A + (int64_t)j * R, DL + (int64_t)j * R, R, D,
                      static_cast<char*>(bw) + (size_t)(j - 1) * pl.bytes};
      hipError_t e = attnres::launch_merge_bwd(
          dtype, mb, pl, timed_launch(K_BWD, rb * 3 + gb * 2 + R * 8.0, st, "merge_bwd_kernel"));
      if (e != hipSuccess) return hip_fail(fn, e);
      TRY(callback(l - 1, dv[l - 2], &dh[j - 1]));
    }
    // the merges' query and gain gradients (rows start + 1 .. end), written
    // before the Phase-1 backward adds to them and reuses the slots
    {
      const double qbytes = (double)(Sk - 1) * ((double)pl.P * D * 4 + (pl.P2 ? 2.0 * pl.P2 * D * 4 : 0.0) +
                                                 D * 4.0 * (dGamma ? 2 : 1));
      hipError_t e = attnres::launch_bwd_reduce_queries(
          pl, bw, pl.bytes, Sk - 1, D, qrow(W, start + 1), qrow(Gamma, start + 1), frow(dW, start + 1),
          frow(dGamma, start + 1), 0u, timed_launch(K_BWD_REDUCE, qbytes, st));
      if (e != hipSuccess) return hip_fail(fn, e);
    }
    // Phase-1 backward: query j's output received a_j dh_j (dh_0 itself: h = o_0)
    // and its log-sum-exp dlse_j; the gradients of b_0 .. b_k accumulate. Up
    // to 8 queries share one pass over the sources where the shape allows.
    if (attnres::phase1_bwd_eligible(dtype, n, D)) {
      const int QB = attnres::phase1_bwd_max_queries(n);  // queries per pass
      for (int j0 = 0; j0 < Sk; j0 += QB) {
        const int Sq = Sk - j0 < QB ? Sk - j0 : QB;
        const float* scl[8];
        const float* dls[8];
        int accq[8];
        for (int j = 0; j < Sq; ++j) {
          scl[j] = j0 + j ? A + (int64_t)(j0 + j) * R : nullptr;
          dls[j] = j0 + j ? DL + (int64_t)(j0 + j) * R : nullptr;
          accq[j] = j0 + j ? 1 : 0;
        }
        const int l0 = start + j0;
        attnres::Phase1BwdArgs pb{b.data(), n, R, D, Sq, dh.data() + j0, scl, dls, qrow(W, l0), qrow(Gamma, l0),
                                  eps, db.data(), frow(dW, l0), frow(dGamma, l0), accq};
        hipError_t e = attnres::launch_phase1_bwd(
            pb, bw, timed_launch(K_BWD, rb * (n + Sq) + gb * n * 2, st, "phase1_bwd_kernel"),
            timed_launch(K_BWD_REDUCE, (double)Sq * D * 4 * 2, st));
        if (e != hipSuccess) return hip_fail(fn, e);
      }
    } else {
      for (int j = 0; j < Sk; ++j)
        TRY(agg_bwd(b.data(), db.data(), n, start + j, dh[j], j ? A + (int64_t)j * R : nullptr,
                    j ? DL + (int64_t)j * R : nullptr, 1, j ? 1 : 0));
    }
  }
  return ok();
}

#ifndef ATTNRES_TIMING_EVENT_FLAGS
#define ATTNRES_TIMING_EVENT_FLAGS hipEventDisableSystemFence
#endif

ATTNRES_API int attnres_timing_enable(int capacity) {
  Timing& t = g_timing;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t = Timing();
  if (capacity <= 0) return ok();
  t.ev.resize(2 * (size_t)capacity, nullptr);
  // Timing-only events: no system-scope fence (cache writeback) when they
  // complete, which would otherwise add several microseconds per launch.
  for (auto& e : t.ev) {
    hipError_t rc = hipEventCreateWithFlags(&e, ATTNRES_TIMING_EVENT_FLAGS);
    if (rc != hipSuccess) {
      for (hipEvent_t x : t.ev)
        if (x) (void)hipEventDestroy(x);
      t = Timing();
      return hip_fail("attnres_timing_enable", rc);
    }
  }
  t.kind.assign(capacity, 0);
  t.bytes.assign(capacity, 0.0);
  t.name.assign(capacity, nullptr);
  t.stream.assign(capacity, nullptr);
  t.capacity = capacity;
  return ok();
}

static int collect_timing() {
  Timing& t = g_timing;
  if (t.used > 0) t.trace.clear();
  for (int s = 0; s < t.used; ++s) {
    hipError_t e = hipEventSynchronize(t.ev[2 * s + 1]);
    if (e != hipSuccess) return hip_fail("attnres_timing_read", e);
    float ms = 0.f, t0 = 0.f, t1 = 0.f;
    e = hipEventElapsedTime(&ms, t.ev[2 * s], t.ev[2 * s + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&t0, t.ev[0], t.ev[2 * s]);
    if (e == hipSuccess) e = hipEventElapsedTime(&t1, t.ev[0], t.ev[2 * s + 1]);
    if (e != hipSuccess) return hip_fail("attnres_timing_read", e);
    t.trace.push_back({t.kind[s], reinterpret_cast<uintptr_t>(t.stream[s]), t0, t1});
    t.launches[t.kind[s]] += 1;
    t.ms[t.kind[s]] += ms;
    t.total_bytes[t.kind[s]] += t.bytes[s];
    std::string& names = t.names[t.kind[s]];
    const std::string nm = t.name[s] ? t.name[s] : "";
    if (("," + names + ",").find("," + nm + ",") == std::string::npos)
      names += (names.empty() ? "" : ",") + nm;
  }
  t.used = 0;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_timing_pause(int paused) {
  g_timing.paused = paused != 0;
  return ok();
}

ATTNRES_API int attnres_timing_reset(void) {
  Timing& t = g_timing;
  t.used = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    t.launches[k] = 0;
    t.ms[k] = 0;
    t.total_bytes[k] = 0;
    t.names[k].clear();
  }
  return ok();
}

ATTNRES_API int attnres_timing_trace(int max, int* kinds, uint64_t* streams, double* start_ms,
                                     double* end_ms) {
  TRY(collect_timing());
  const Timing& t = g_timing;
  const int n = (int)t.trace.size() < max ? (int)t.trace.size() : max;
  for (int i = 0; i < n; ++i) {
    if (kinds) kinds[i] = t.trace[i].kind;
    if (streams) streams[i] = t.trace[i].stream;
    if (start_ms) start_ms[i] = t.trace[i].start;
    if (end_ms) end_ms[i] = t.trace[i].end;
  }
  return n;
}

ATTNRES_API const char* attnres_timing_kernels(int kind) {
  if (kind < 0 || kind >= K_COUNT) {
    fail(ATTNRES_EINVAL, "attnres_timing_kernels: kind %d", kind);
    return "";
  }
  if (collect_timing() != ATTNRES_OK) return "";
  return g_timing.names[kind].c_str();
}

ATTNRES_API int attnres_timing_read(int kind, int64_t* launches, double* total_ms,
                                    double* total_bytes) {
  if (kind < 0 || kind >= K_COUNT)
    return fail(ATTNRES_EINVAL, "attnres_timing_read: kind %d", kind);
  TRY(collect_timing());
  const Timing& t = g_timing;
  if (launches) *launches = t.launches[kind];
  if (total_ms) *total_ms = t.ms[kind];
  if (total_bytes) *total_bytes = t.total_bytes[kind];
  return ok();
}
