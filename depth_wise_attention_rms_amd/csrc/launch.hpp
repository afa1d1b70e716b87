// launch.hpp -- internal interface between the C ABI (api.hip) and the kernel
// launchers (kernels.hip). Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// Stream of a launch, plus an optional event pair that receives the start and
// end timestamps of the kernel's own dispatch (both null when not timed).
struct Launch {
  hipStream_t stream;
  hipEvent_t start;
  hipEvent_t stop;
};

// A "close" fused into a launch: its last source is not read from src[n-1]
// but formed as round(close_p + close_v) (or close_v when close_p is null),
// stored to close_b and used directly. close_v == null means no close.
struct Phase1Args {
  const void* const* src;  // (host) n device pointers
  int n;
  int64_t R, D;
  const float* W;  // [S][D]
  const float* G;  // [S][D] or null
  int S;
  float eps;
  void* out;       // [S][R][D], or null: statistics only (phase1_stats_supported shapes)
  float* m_out;    // [S][R] or null
  float* lse_out;  // [S][R]
  const void* close_p;
  const void* close_v;
  void* close_b;
  // workspace of phase1_gemm_workspace(S, R, D, n) bytes, or null: with it,
  // shapes phase1_gemm_eligible() accepts take the scores/outputs passes
  void* gemm_ws = nullptr;
  // the streamed kernel's workgroup budget per launch (0: its default); a
  // smaller one runs query passes one after another instead of side by side
  int max_groups = 0;
  // with nf_out: output 0 (the block's first sublayer's h, or the source
  // itself when out is null) is also written as that sublayer's input norm
  // round(nf_g * h / sqrt(mean_d h^2 + nf_eps)) to nf_out -- by the kernels
  // phase1_norm_fused() names; output 0 itself is then not written
  const float* nf_g = nullptr;
  float nf_eps = 0.f;
  void* nf_out = nullptr;
  // without nf_out: output 0 is written to out0 [R][D] instead of out's first
  // slice, and output 1 to out1 instead of its second, by the kernels
  // phase1_out01_supported() names (the others ignore both)
  void* out0 = nullptr;
  void* out1 = nullptr;
};

struct AggArgs {
  const void* const* src;  // (host) n device pointers
  int n;
  int64_t R, D;
  const float* w;  // [D]
  const float* g;  // [D] or null
  float eps;
  void* out;       // [R][D]
  float* m_out;    // [R] or null
  float* lse_out;  // [R] or null
  const void* close_p;
  const void* close_v;
  void* close_b;
  // optional starting summary of an earlier group: normalised output [R][D]
  // and its log-sum-exp [R] (both null: start empty)
  const void* o_init = nullptr;
  const float* lse_init = nullptr;
  // with nf_out: the output is written as its sublayer's input norm
  // round(nf_g * h / sqrt(mean_d h^2 + nf_eps)) to nf_out instead of to out
  const float* nf_g = nullptr;
  float nf_eps = 0.f;
  void* nf_out = nullptr;
};

struct Phase2Args {
  const void* o;
  const float* lse;
  const float* w;
  const float* g;
  float eps;
  const void* p_prev;
  const void* v_prev;
  void* p_out;
  void* h_out;      // may be null when hn_out is set
  const float* gf;  // [D] or null: gain of the fused output norm
  float eps_f;
  void* hn_out;     // RMSNorm(h) * gf, or null
  int64_t R, D;
  // a completed source [R][D] merged as one more single-source term (the
  // decode schedule's newest block sum, which its Phase-1 group left out), or null
  const void* xs = nullptr;
};

// Aggregate backward: sources, query and gain as in AggArgs, upstream gradient
// dh [R][D] in the I/O dtype, fp32 gradients dV[i] [R][D], dw [D] and dgamma
// [D] (or null), written or (accumulate != 0) added; workspace holds the
// per-workgroup dq~ partials and the first reduction stage (BwdPlan::bytes).
struct BwdArgs {
  const void* const* src;
  int n;
  int64_t R, D;
  const float* w;
  const float* g;
  float eps;
  const void* dh;
  float* const* dV;
  int accumulate;
  float* dw;
  float* dgamma;
  void* workspace;
  // [R] or null: the upstream gradient of row r is dh_scale[r] * dh[r]
  const float* dh_scale = nullptr;
  // [R] or null: gradient of the group's log-sum-exp, added to each score's
  const float* dlse = nullptr;
  // dw / dgamma written (0) or added (1); -1: as accumulate
  int accumulate_q = -1;
};

// Backward of one Phase-2 merge, h = a o + c p with (a, c) = softmax(lse,
// s_p) and s_p the score of p: from the upstream gradient dh it forms the
// gradient of p (through the weighted sum and through s_p), added to g_in
// into g_out, the group's weight a and the gradient of lse per row, and the
// per-workgroup dq~ partials in `workspace` (BwdPlan of the same shape).
struct MergeBwdArgs {
  const void* o;      // [R][D] dtype
  const float* lse;   // [R]
  const void* ps;     // [R][D] dtype: the partial p
  const float* w;     // [D]
  const float* g;     // [D] or null
  float eps;
  const void* dh;     // [R][D] dtype
  const float* g_in;  // [R][D] fp32 or null (zero)
  float* g_out;       // [R][D] fp32
  float* a_out;       // [R]
  float* dlse_out;    // [R]
  int64_t R, D;
  void* workspace;
};

struct BwdPlan {
  bool supported;
  int vpl;
  unsigned grid;         // workgroups of the main kernel (0 when R == 0)
  int64_t P;             // dq~ partial rows
  int64_t chunk;         // rows per first-stage sum
  int64_t P2;            // first-stage rows (0: the final stage reads the partials)
  size_t partial_bytes;  // 256-aligned size of the partials
  size_t bytes;          // workspace bytes
};

BwdPlan plan_aggregate_bwd(int dtype, int64_t R, int64_t D);
hipError_t launch_aggregate_bwd(int dtype, const BwdArgs& a, const BwdPlan& pl, const Launch& L);
// stage 0: partial rows -> chunk sums (no-op when P2 == 0); stage 1: final
// sum, dw and dgamma
hipError_t launch_bwd_reduce(const BwdArgs& a, const BwdPlan& pl, int stage, const Launch& L);
// The query-gradient reductions of nq aggregates (1..32) at once: query q's
// partials in the plan's layout at ws + q * slot (slot a multiple of 4
// bytes); w, g, dw, dgamma the first query's rows, the others D apart; bit q
// of acc_mask: query q adds to dw / dgamma instead of writing them.
hipError_t launch_bwd_reduce_queries(const BwdPlan& pl, void* ws, size_t slot, int nq, int64_t D,
                                     const float* w, const float* g, float* dw, float* dgamma,
                                     unsigned acc_mask, const Launch& L);
hipError_t launch_merge_bwd(int dtype, const MergeBwdArgs& a, const BwdPlan& pl, const Launch& L);

// Batched Phase-1 backward: S <= 8 queries (consecutive rows of w, g, dw,
// dgamma) over the same n <= 8 bf16 sources in one pass; query j's upstream
// gradient is dh_scale[j][r] * dh[j][r] (dh_scale[j] null: 1) and its
// log-sum-exp's gradient dlse[j] (null: 0). dV[i] fp32 are added to; dw /
// dgamma rows are written (accumulate_q[j] == 0) or added. Rows of at most
// 4096 elements (phase1_bwd_eligible). `ws` holds phase1_bwd_workspace bytes.
struct Phase1BwdArgs {
  const void* const* src;
  int n;
  int64_t R, D;
  int S;
  const void* const* dh;
  const float* const* dh_scale;
  const float* const* dlse;
  const float* w;   // [S][D]
  const float* g;   // [S][D] or null
  float eps;
  float* const* dV;
  float* dw;        // [S][D]
  float* dgamma;    // [S][D] or null
  const int* accumulate_q;  // [S]
};
bool phase1_bwd_eligible(int dtype, int n, int64_t D);
// Queries one pass takes over n sources (8, or 4 where 8 would spill).
int phase1_bwd_max_queries(int n);
size_t phase1_bwd_workspace(int64_t R, int64_t D);
hipError_t launch_phase1_bwd(const Phase1BwdArgs& a, void* ws, const Launch& L, const Launch& Lred);

hipError_t launch_fold(const float* w, const float* g, float* q, int64_t count, const Launch& L);
hipError_t launch_phase1(int dtype, const Phase1Args& a, const Launch& L);
// Phase 1 as a matrix-core scores pass and an outputs pass (bf16, n <= 16,
// S <= 32, D a multiple of 256 up to 8192, many rows; statistics only when
// out is null); needs materialised sources (no fused close) and a workspace
// of phase1_gemm_workspace(S, R, D, nmax) bytes for launches of up to nmax
// sources.
bool phase1_gemm_shape(int dtype, int S, int64_t D, int64_t R);
// the register-tile matrix-core Phase 1 (bf16, n <= 8, S <= 8, D in {1024, 2048, 3072, 4096})
bool phase1_mfma_eligible(int dtype, int n, int S, int64_t D);
bool phase1_gemm_eligible(int dtype, int n, int S, int64_t D, int64_t R);
// the most sources of a Phase 1 of S queries over 1..nmax sources that takes
// the scores/outputs passes, 0 if none does (a stack reserves their workspace
// for that many sources)
int phase1_gemm_needed(int dtype, int S, int64_t D, int64_t R, int nmax);
size_t phase1_gemm_workspace(int S, int64_t R, int64_t D, int nmax);
hipError_t launch_phase1_gemm(const Phase1Args& a, void* ws, const Launch& L);
bool phase1_supported(int dtype, int n, int S, int64_t D);
// whether the kernel a Phase-1 launch runs writes the input norm of output 0
// itself (Phase1Args::nf_out)
bool phase1_norm_fused(int dtype, const Phase1Args& a, bool gemm);
// whether the kernel a Phase-1 launch runs honours Phase1Args::out0 and out1
bool phase1_out01_supported(int dtype, const Phase1Args& a, bool gemm);
// name of the kernel(s) a Phase-1 launch runs (gemm: the scores/outputs path)
const char* phase1_kernel_name(int dtype, const Phase1Args& a, bool gemm);
// Phase 1 with out == null (statistics only) is available for these shapes
bool phase1_stats_supported(int dtype, int n, int S, int64_t D);
hipError_t launch_aggregate(int dtype, const AggArgs& a, const Launch& L);
hipError_t launch_phase2(int dtype, const Phase2Args& a, const Launch& L);
hipError_t launch_rmsnorm(int dtype, const void* x, int64_t R, int64_t D, const float* g, float eps,
                          void* out, const Launch& L);
// A block's partials in one pass: out[t] = round(p + in[t]) chained from
// p = in[0], t = 1..n-1 (2 <= n <= kPartialsMax; out[0] unused).
constexpr int kPartialsMax = 64;
hipError_t launch_partials(int dtype, const void* const* in, void* const* out, int n, int64_t R, int64_t D,
                           const Launch& L);
hipError_t launch_close(int dtype, const void* p, const void* v, void* b, int64_t R, int64_t D,
                        const Launch& L);

}  // namespace attnres
