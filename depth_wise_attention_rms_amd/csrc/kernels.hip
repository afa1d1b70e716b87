// kernels.hip -- gfx950 kernels of the AttnRes depth-aggregation hot path.
//
// Pages: K3 course notes, section "Attention Residual 深度残差" (eqs. A1-A3,
// OS1, OS2; 9.3 forward_naive; 9.4 two-phase algorithm); "Attention
// Residuals" survey page on wineandchord.com ("Depth attention & online merge
// reference"); reading notes on "Attention Residuals" (ranhao.site) 4.2
// Inference.
//
// Work decomposition. Every kernel is bandwidth-shaped: it streams [R,D] rows
// and does a short per-row contraction. A token row is owned by W waves
// (64*W lanes); lane t holds VPL 16-byte vectors of the row, vector c at index
// c*64*W + t, so each load instruction of a wave covers 1 KiB of contiguous
// memory. Rows are independent (weights are per token), so a workgroup of
// RPW*W waves walks RPW rows at a time in a grid-stride loop and no data moves
// between workgroups. Row-wide sums (sum of squares, dot products) reduce with
// DPP inside a wave and through LDS across the W waves of a row. [R,D] tensors
// are read and written with non-temporal hints; queries go through the caches.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "launch.hpp"

#include <float.h>

namespace attnres {

// Write target of lanes that own no element (past a ragged row's end, or a
// row past the last): such a lane stores here instead of skipping the store,
// so stores need no exec-mask branch, which would make the compiler wait for
// every outstanding memory operation at each one. Never read.
__device__ __attribute__((aligned(256))) unsigned char g_store_sink[256];

__device__ __forceinline__ char* store_target(bool owns, char* p) {
  return owns ? p : reinterpret_cast<char*>(g_store_sink);
}

// Row geometry of one launch, computed on the host.
struct Geom {
  int64_t R;       // token rows
  int64_t groups;  // ceil(R / RPW)
  int V;           // 16-byte vectors per row
  int W;           // waves per row
  int RPW;         // rows per workgroup iteration
  int D;           // elements per row
  float invD;      // 1 / D
};

struct Lanes {
  int lane, slot, wr, t, stride;
  __device__ __forceinline__ Lanes(int W) {
    lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    slot = wave / W;
    wr = wave - slot * W;
    t = wr * 64 + lane;
    stride = W * 64;
  }
};

// The block close b = round(p + v) (or b = v when p is null) performed by a
// kernel on the fly for its last source [K3 9.3 listing]: the closing block
// sum is computed from the partial and the last sublayer output, stored once,
// and used as a source without being read back.
struct Close {
  const void* p;  // partial before the block's last sublayer, or null
  const void* v;  // the block's last sublayer output; null = no close
  void* b;        // receives the block sum
};

// Load vector `off` of source i, applying the close when i is the closing one.
template <class T>
__device__ __forceinline__ uint4 load_source(const void* src, const Close& cl, bool closing,
                                             int64_t off) {
  if (!closing) return ld16_stream(static_cast<const char*>(src) + off);
  uint4 v = ld16_stream(static_cast<const char*>(cl.v) + off);
  if (cl.p) {
    const uint4 a = ld16_stream(static_cast<const char*>(cl.p) + off);
    float fa[T::kEPV], fv[T::kEPV];
    T::unpack(a, fa);
    T::unpack(v, fv);
    #pragma unroll
    for (int e = 0; e < T::kEPV; ++e) fa[e] += fv[e];
    v = T::pack(fa);  // rounded to the I/O dtype, as the block sum is stored
  }
  st16_stream(static_cast<char*>(cl.b) + off, v);
  return v;
}

// ---------------------------------------------------------------------------
// Query fold q~ = w * gamma in fp32 [K3 9.2 (1)], over `count` elements.
// ---------------------------------------------------------------------------
__global__ void fold_kernel(const float* __restrict__ w, const float* __restrict__ g,
                            float* __restrict__ q, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    q[i] = g ? w[i] * g[i] : w[i];
}

// Load EPV fp32 query values at element offset `off`, folding the gain.
template <int EPV>
__device__ __forceinline__ void load_query(const float* __restrict__ w, const float* __restrict__ g,
                                           int64_t off, float* q) {
  #pragma unroll
  for (int k = 0; k < EPV; k += 4) {
    float4 a = ldf4(w + off + k);
    if (g) {
      float4 b = ldf4(g + off + k);
      a.x *= b.x; a.y *= b.y; a.z *= b.z; a.w *= b.w;
    }
    q[k] = a.x; q[k + 1] = a.y; q[k + 2] = a.z; q[k + 3] = a.w;
  }
}

// EPV gains starting at element `off` (16-byte loads), or ones for a null gain.
template <int EPV>
__device__ __forceinline__ void load_gain(const float* __restrict__ g, int64_t off, float* out) {
  #pragma unroll
  for (int k = 0; k < EPV; k += 4) {
    const float4 a = g ? ldf4(g + off + k) : make_float4(1.f, 1.f, 1.f, 1.f);
    out[k] = a.x; out[k + 1] = a.y; out[k + 2] = a.z; out[k + 3] = a.w;
  }
}

// ---------------------------------------------------------------------------
// Phase 1 (batched inter-block pass) [K3 9.4 step 1; RH 4.2 Phase 1].
// The n <= NMAX sources of a row are loaded once and held in registers as
// fp32; the S queries are processed in batches of SB: per batch one row
// reduction of SB*NMAX dot products (plus the NMAX sums of squares), then the
// SB softmaxes over the source axis and SB weighted sums of the raw sources.
// ---------------------------------------------------------------------------
struct Phase1Params {
  const void* src[16];
  int n;
  int S;
  const float* Wq;  // [S][D]
  const float* G;   // [S][D] or null
  float eps;
  void* out;        // [S][R][D]
  float* m_out;     // [S][R] or null
  float* lse_out;   // [S][R]
  Close cl;         // close computing source n-1, or cl.v == null
  const float* nf_g = nullptr;  // the sublayer input norm of output 0 (see Phase1Args::nf_out)
  float nf_eps = 0.f;
  void* nf_out = nullptr;
  Geom g;
};

template <class T, int VPL, int NMAX, int SB>
__global__ __launch_bounds__(512) void phase1_kernel(Phase1Params p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  constexpr int NV = SB * NMAX + NMAX;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  const int n = p.n;
  const bool has_close = p.cl.v != nullptr;

  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;

    float x[NMAX][VPL][EPV];
    #pragma unroll
    for (int i = 0; i < NMAX; ++i) {
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int vec = c * ln.stride + ln.t;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (rv && i < n && vec < g.V)
          u = load_source<T>(p.src[i], p.cl, has_close && i == n - 1,
                             row * rowbytes + (int64_t)vec * 16);
        T::unpack(u, x[i][c]);
      }
    }

    float inv_rms[NMAX];
    for (int s0 = 0; s0 < p.S; s0 += SB) {
      float red[NV];
      #pragma unroll
      for (int k = 0; k < NV; ++k) red[k] = 0.f;
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int vec = c * ln.stride + ln.t;
        if (vec < g.V) {
          if (s0 == 0) {
            #pragma unroll
            for (int i = 0; i < NMAX; ++i)
              #pragma unroll
              for (int e = 0; e < EPV; ++e) red[SB * NMAX + i] += x[i][c][e] * x[i][c][e];
          }
          #pragma unroll
          for (int sb = 0; sb < SB; ++sb) {
            if (s0 + sb < p.S) {
              float q[EPV];
              load_query<EPV>(p.Wq, p.G, (int64_t)(s0 + sb) * g.D + (int64_t)vec * EPV, q);
              #pragma unroll
              for (int i = 0; i < NMAX; ++i)
                #pragma unroll
                for (int e = 0; e < EPV; ++e) red[sb * NMAX + i] += q[e] * x[i][c][e];
            }
          }
        }
      }
      row_reduce<NV>(red, lds, ln.slot, ln.wr, g.W);
      if (s0 == 0) {
        #pragma unroll
        for (int i = 0; i < NMAX; ++i) inv_rms[i] = rsqrtf(red[SB * NMAX + i] * g.invD + p.eps);
      }
      #pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int s = s0 + sb;
        if (s < p.S) {
          float sc[NMAX];
          float m = -FLT_MAX;
          #pragma unroll
          for (int i = 0; i < NMAX; ++i) {
            sc[i] = red[sb * NMAX + i] * inv_rms[i];
            if (i < n) m = fmaxf(m, sc[i]);
          }
          float z = 0.f;
          #pragma unroll
          for (int i = 0; i < NMAX; ++i) {
            sc[i] = i < n ? __expf(sc[i] - m) : 0.f;
            z += sc[i];
          }
          const float rz = 1.0f / z;
          #pragma unroll
          for (int i = 0; i < NMAX; ++i) sc[i] *= rz;
          if (rv) {
            if (ln.t == 0) {
              if (p.m_out) p.m_out[(int64_t)s * g.R + row] = m;
              p.lse_out[(int64_t)s * g.R + row] = m + __logf(z);
            }
            if (!p.out) continue;  // statistics only
            char* orow = static_cast<char*>(p.out) + ((int64_t)s * g.R + row) * rowbytes;
            #pragma unroll
            for (int c = 0; c < VPL; ++c) {
              const int vec = c * ln.stride + ln.t;
              if (vec < g.V) {
                float o[EPV];
                #pragma unroll
                for (int e = 0; e < EPV; ++e) o[e] = 0.f;
                #pragma unroll
                for (int i = 0; i < NMAX; ++i)
                  #pragma unroll
                  for (int e = 0; e < EPV; ++e) o[e] += sc[i] * x[i][c][e];
                st16_stream(orow + (int64_t)vec * 16, T::pack(o));
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Phase-1 statistics of a block whose only source is the embedding b_0
// [K3 9.4 step 1 with one source]: every softmax weight is exactly 1, so each
// output would be b_0 itself and is not formed; only the scores of b_0 under
// the S <= SQ queries are computed, and m = lse = score (the log of a unit
// denominator is 0). The folded queries stay in registers for every row, and
// the next row's vectors are loaded while the current row reduces.
// ---------------------------------------------------------------------------
template <class T, int VPL, int SQ, int PD>
__global__ __launch_bounds__(512) void phase1_single_kernel(Phase1Params p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  constexpr int NV = SQ + 1;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;

  float q[SQ][VPL][EPV];
  #pragma unroll
  for (int s = 0; s < SQ; ++s)
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      if (s < p.S && vec < g.V) {
        load_query<EPV>(p.Wq, p.G, (int64_t)s * g.D + (int64_t)vec * EPV, q[s][c]);
      } else {
        #pragma unroll
        for (int e = 0; e < EPV; ++e) q[s][c][e] = 0.f;
      }
    }

  // Loads are unconditional (a row past the end reads row 0, a lane past the
  // row's end reads vector 0, and both are discarded), so no branch hides
  // them from the compiler's wait counting and the prefetch stays in flight.
  auto load_row = [&](int64_t grp, uint4* dst) {
    const int64_t row = grp * g.RPW + ln.slot;
    const int64_t rr = (grp < g.groups && row < g.R) ? row : 0;
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      dst[c] = ld16_stream(static_cast<const char*>(p.src[0]) + rr * rowbytes +
                           (int64_t)(vec < g.V ? vec : 0) * 16);
    }
  };
  // the next PD rows of this workgroup are in flight while a row reduces
  uint4 ahead[PD][VPL];
  #pragma unroll
  for (int d = 0; d < PD; ++d) load_row(blockIdx.x + (int64_t)d * gridDim.x, ahead[d]);
  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    uint4 cur[VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) cur[c] = ahead[0][c];
    #pragma unroll
    for (int d = 0; d + 1 < PD; ++d)
      #pragma unroll
      for (int c = 0; c < VPL; ++c) ahead[d][c] = ahead[d + 1][c];
    load_row(grp + (int64_t)PD * gridDim.x, ahead[PD - 1]);
    float red[NV];
    #pragma unroll
    for (int k = 0; k < NV; ++k) red[k] = 0.f;
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const bool in_row = c * ln.stride + ln.t < g.V;
      float x[EPV];
      T::unpack(cur[c], x);
      #pragma unroll
      for (int e = 0; e < EPV; ++e) {
        x[e] = in_row ? x[e] : 0.f;
        red[SQ] += x[e] * x[e];
        #pragma unroll
        for (int s = 0; s < SQ; ++s) red[s] += q[s][c][e] * x[e];
      }
    }
    row_reduce<NV>(red, lds, ln.slot, ln.wr, g.W);
    if (p.nf_out && row < g.R) {
      // output 0 is the source itself: its sublayer's input norm, from the
      // same sum of squares [ZZ block listing: attn(attn_norm(h))]
      const float inv = rsqrtf(red[SQ] * g.invD + p.nf_eps);
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int vec = c * ln.stride + ln.t;
        if (vec < g.V) {
          float x[EPV], gn[EPV];
          T::unpack(cur[c], x);
          load_gain<EPV>(p.nf_g, (int64_t)vec * EPV, gn);
          #pragma unroll
          for (int e = 0; e < EPV; ++e) x[e] = gn[e] * (x[e] * inv);
          st16(static_cast<char*>(p.nf_out) + row * rowbytes + (int64_t)vec * 16, T::pack(x));
        }
      }
    }
    if (row < g.R && ln.t < SQ && ln.t < p.S) {
      // lane s writes query s's statistics
      float dot = red[0];
      #pragma unroll
      for (int s = 1; s < SQ; ++s)
        if (ln.t == s) dot = red[s];
      const float sc = dot * rsqrtf(red[SQ] * g.invD + p.eps);
      if (p.m_out) p.m_out[(int64_t)ln.t * g.R + row] = sc;
      p.lse_out[(int64_t)ln.t * g.R + row] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 1 on the matrix cores (bf16 I/O; S <= 8 queries, n <= 8 sources,
// D in {1024, 2048, 3072, 4096}). Both contractions of a token row run on the
// matrix cores with fp32 accumulation, each fp32 operand split exactly into
// three bf16 parts (h1 = bf16(x), h2 = bf16(x - h1), h3 = x - h1 - h2) so the
// bf16 x bf16 products keep fp32 accuracy:
//   scores   t[s][i] = q~_s . b_i over the hidden axis (v_mfma_f32_16x16x32_bf16;
//            A rows 4s + j hold part j of query s, row 4s + 3 is zero, so the
//            three partial products of a query land in one lane's registers;
//            B columns are the row's sources), and
//   outputs  o_s[d] = sum_i alpha[s][i] b_i[d] over the sources
//            (v_mfma_f32_32x32x16_bf16, see the output step below).
// Sums of squares (v_dot2 on the same B fragments), the softmax and the
// statistics stay on the vector ALUs in fp32.
//
// One workgroup of 8 waves per CU walks token rows. Wave w owns the hidden
// slice [w*D/8, (w+1)*D/8) and keeps the query parts of that slice in
// registers for the whole kernel. A row's sources are copied from HBM
// straight into a slot of an LDS ring (global_load_lds, 16 bytes per lane),
// up to three rows ahead of the row being scored and written. Each source row
// in a slot is padded by 32 bytes so lanes reading different sources at one
// column hit different banks. A fused block close stages its p and v rows and
// forms b = round(p + v) in place before the row is scored. At D = 4096 each
// wave copies, scores and writes only its own slice, so a row needs a single
// barrier (for the cross-wave score reduction). The copies are
// non-temporal; the outputs are written with plain stores for the first two
// and non-temporal ones after (ATTNRES_P1_OUT_NT_FROM).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kP1Waves = 8;
constexpr int kP1MaxN = 8;
constexpr int kP1MaxS = 8;
#ifndef ATTNRES_P1_FENCE
#define ATTNRES_P1_FENCE 4
#endif
constexpr int kP1Fence = ATTNRES_P1_FENCE;  // k-steps between scheduling fences (0: none)
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kP1LdsBytes = 160 * 1024;

// Shapes of one instantiation: KS k-steps of 16 per wave (D = 128 KS), NC
// sources per row; NF: output 0 is written as its sublayer's input norm.
template <int KS, int NC, bool NF = false>
struct P1Shape {
  static constexpr int D = 128 * KS;
  static constexpr int STRIDE = D + 16;    // bf16 elements per staged row
  static constexpr int NCH = KS / 4;       // 1 KiB chunks per row; wave w copies chunk w
  static constexpr int ROWS = NC + 1;      // staged rows per slot: sources, then p of a close
  static constexpr int SLOT = ROWS * STRIDE;
  static constexpr int RED = 2 * (kP1Waves * kP1MaxS * NC + kP1Waves * NC);  // floats, two rows
  // With 8 chunks per row, wave w copies, closes, scores and writes only chunk
  // w (its hidden slice) of every staged row, so rows need no barrier of their
  // own: the only exchange between waves is the score reduction.
  static constexpr bool PRIVATE = NCH == kP1Waves;
  // with NF: the gain [D] and the Gram partials [two rows][wave][NC][NC], fp32
  static constexpr int GRAM = 2 * kP1Waves * NC * NC;
  static constexpr int NFB = NF ? D + GRAM : 0;
  static constexpr int FIT = (kP1LdsBytes - 4 * RED - 4 * kP1Waves * 64 - 1024 - 4 * NFB) / (2 * SLOT);
  static constexpr int NBUF = FIT > 4 ? 4 : FIT;  // ring slots (prefetch distance NBUF - 1)
  static constexpr bool FITS = NBUF >= 2;         // a row and its successor fit in LDS
  static_assert(NF || FITS, "a row and its successor must fit in LDS");
};

struct Phase1MParams {
  const void* src[kP1MaxN];
  int n;
  int S;
  const float* Wq;  // [S][D]
  const float* G;   // [S][D] or null
  float eps;
  void* out;        // [S][R][D]
  float* m_out;     // [S][R] or null
  float* lse_out;   // [S][R]
  Close cl;
  int64_t R;
  int D;
  float invD;
  const float* nf_g;  // with nf_out: output 0 goes to nf_out as its input norm
  float nf_eps;       // round(nf_g * h / sqrt(mean_d h^2 + nf_eps)), h = output 0
  void* nf_out;       // rounded (nf_g null: a gain of 1), and not to out
  void* out0;         // [R][D] or null: without nf_out, output 0 goes here instead of to out
  void* out1;         // [R][D] or null: output 1 goes here instead of to out
};

// x rounded to the nearest bf16 (ties to even), as an fp32 value
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

// Reductions over the 8-lane groups of a wave (lanes 8g .. 8g+7): swaps within
// quads, then the mirror of each half row. Every lane gets its group's result.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  return fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
}
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  return x + dpp_mov<0x141>(x);
}
// The same over aligned groups of N = 1, 2, 4, 8 or 16 lanes (16: a
// row_mirror joins the two halves of a DPP row).
template <int N>
__device__ __forceinline__ float groupn_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_mov<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float groupn_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);
  return x;
}

// Workgroup barrier after this wave's LDS reads and writes have completed.
// It does not wait for vector memory: a fenced barrier (__syncthreads(), or
// an LDS-scope fence, which also covers loads into LDS) would make every
// wave wait for its in-flight prefetch of the next row and its stores. Loads
// into LDS are waited for explicitly before the barrier that publishes them.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A wave-uniform address as a scalar value in the global address space: the
// compiler then addresses memory as scalar base + 32-bit lane offset instead
// of keeping a 64-bit per-lane address for every stream (and the accesses
// stay global, not flat, so they count on the vector-memory counter only).
typedef __attribute__((address_space(1))) char gchar_t;
__device__ __forceinline__ gchar_t* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (gchar_t*)(((uint64_t)hi << 32) | lo);
}
typedef __attribute__((address_space(1))) u32x4_t gu32x4_t;
__device__ __forceinline__ void st16_stream(gchar_t* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<gu32x4_t*>(p));
}
// Plain (cached) 16-byte store: Phase 1's first outputs (see
// ATTNRES_P1_OUT_NT_FROM).
__device__ __forceinline__ void st16_global(gchar_t* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  *reinterpret_cast<gu32x4_t*>(p) = t;
}

// Address of a __shared__ object as an LDS byte offset.
typedef __attribute__((address_space(3))) char lchar_t;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const lchar_t*)p;
}

// Copy 16 bytes per lane from global memory (wave-uniform base + lane offset)
// into LDS at the wave-uniform offset lds + 16 * lane, non-temporal (each
// source row is read once per launch). Issued as inline
// assembly so that the compiler's own wait-counter bookkeeping, which cannot
// tell ring slots apart, adds no waits before LDS reads: the kernel waits for
// these copies itself (p1_wait), before the barrier that publishes them.
// M0 is written here; nothing else in these kernels uses it.
#ifndef ATTNRES_P1_SRC_NT
#define ATTNRES_P1_SRC_NT 1  // source copies carry the non-temporal hint
#endif
__device__ __forceinline__ void dma16(const gchar_t* base, uint32_t lane_off, uint32_t lds) {
#if ATTNRES_P1_SRC_NT
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(lane_off), "s"(base) : "memory");
#else
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(lane_off), "s"(base) : "memory");
#endif
}

// Wait until at most k (clamped to the counter's 63) vector-memory operations
// of this wave are outstanding. Global loads (including loads into LDS) and
// stores of one wave report completion in issue order, so this waits for
// everything issued before the last k operations. LDS and scalar counters
// are not waited on.
__device__ __forceinline__ void p1_wait(int k) {
  k = __builtin_amdgcn_readfirstlane(k);  // wave-uniform: a scalar branch, not a lane compare
#define ATTNRES_W(K) case K: __builtin_amdgcn_s_waitcnt(((K) & 0xF) | (((K) >> 4) << 14) | (0x7 << 4) | (0xF << 8)); break;
#define ATTNRES_W8(K) ATTNRES_W(K) ATTNRES_W(K + 1) ATTNRES_W(K + 2) ATTNRES_W(K + 3) \
                      ATTNRES_W(K + 4) ATTNRES_W(K + 5) ATTNRES_W(K + 6) ATTNRES_W(K + 7)
  switch (k < 63 ? k : 63) {
    ATTNRES_W8(0) ATTNRES_W8(8) ATTNRES_W8(16) ATTNRES_W8(24)
    ATTNRES_W8(32) ATTNRES_W8(40) ATTNRES_W8(48) ATTNRES_W8(56)
    default: break;
  }
#undef ATTNRES_W8
#undef ATTNRES_W
}

// Stage token row `row` into ring slot `slot`: the sources (for a close, v in
// place of the closing source) and, for a close with a partial, p after them.
// Returns the number of copy instructions this wave issued.
template <int KS, int NC>
__device__ __forceinline__ int p1_stage(const Phase1MParams& p, int64_t row, const __bf16* slot,
                                        int w, int l) {
  using Sh = P1Shape<KS, NC>;
  if (w >= Sh::NCH) return 0;
  const int64_t roff = row * (int64_t)Sh::D * 2;
  const uint32_t loff = (uint32_t)((w * 64 + l) * 16);
  const uint32_t lds = lds_offset(slot) + (uint32_t)(w * 1024);
  const bool has_close = p.cl.v != nullptr;
  #pragma unroll
  for (int i = 0; i < NC; ++i) {
    const void* g = (i == NC - 1 && has_close) ? p.cl.v : p.src[i];
    dma16(uniform_ptr(static_cast<const char*>(g) + roff), loff, lds + (uint32_t)(i * Sh::STRIDE * 2));
  }
  if (has_close && p.cl.p) {
    dma16(uniform_ptr(static_cast<const char*>(p.cl.p) + roff), loff,
          lds + (uint32_t)(NC * Sh::STRIDE * 2));
    return NC + 1;
  }
  return NC;
}

#ifndef ATTNRES_P1_B_NT
#define ATTNRES_P1_B_NT 1  // the fused close stores the block sum non-temporally
#endif
// Outputs of queries from this index on are stored non-temporally. The first
// two are read right after the launch (output 0 by the block's first
// sublayer, output 1 by its first Phase-2 merge) and stay cacheable; storing
// the later ones past the last-level cache measured 1-2% faster for Phase 1
// and for that merge (all eight non-temporal: 6% slower).
#ifndef ATTNRES_P1_OUT_NT_FROM
#define ATTNRES_P1_OUT_NT_FROM 2
#endif
static_assert(ATTNRES_P1_OUT_NT_FROM >= 2, "queries 0 and 1 share one store instruction");

template <int KS, int NC, bool NF>
__global__ __launch_bounds__(512, 1) void phase1_mfma_kernel(Phase1MParams p) {
  using Sh = P1Shape<KS, NC, NF>;
  constexpr int D = Sh::D, STRIDE = Sh::STRIDE, NCH = Sh::NCH, NBUF = Sh::NBUF, PF = NBUF - 1;
  __shared__ __attribute__((aligned(16))) __bf16 ring[NBUF * Sh::SLOT];
  // partial scores [row parity][wave][query][source] and sums of squares
  // [row parity][wave][source]; alternating rows use alternate halves, so a
  // wave may write row r + 1's partials while another still reads row r's
  __shared__ float cred_buf[2 * kP1Waves * kP1MaxS * NC];
  __shared__ float ssred_buf[2 * kP1Waves * NC];
  // each wave's softmax weights, lane 8 s + i = alpha[s][i]; written and read
  // back by the same wave only (its LDS accesses complete in order)
  __shared__ __attribute__((aligned(16))) float alpha_buf[kP1Waves * 64];
  // NF: the gain, and each wave's Gram partials of the row's sources over its
  // hidden slice, [row parity][wave][source k][source i]
  __shared__ __attribute__((aligned(16))) float gam_buf[NF ? D : 4];
  __shared__ float gram_buf[NF ? Sh::GRAM : 1];

  const int S = p.S;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, kg = l >> 4;  // B column (source) and k-group of this lane
  const bool has_close = p.cl.v != nullptr;
  const bool owner = w < NCH;           // this wave copies, closes and writes chunk w of each row
  const int64_t rowbytes = (int64_t)D * 2;

  // A operand: qa[2 kk + t] is tile t of k-step kk (32 wide), row m = 16 t + l % 16
  // = part j = m % 4 of query s = m / 4 (part 3 is zero), k-group l / 16.
  uint4 qa[KS];
  #pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int m = 16 * (kk & 1) + col, s = m >> 2, j = m & 3;
    float part[8];
    #pragma unroll
    for (int e = 0; e < 8; ++e) part[e] = 0.f;
    if (s < S && j < 3) {
      float q[8];
      load_query<8>(p.Wq, p.G, (int64_t)s * D + w * (D / kP1Waves) + 32 * (kk >> 1) + 8 * kg, q);
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float h1 = bf16_round(q[e]);
        const float r1 = q[e] - h1;  // exact
        const float h2 = bf16_round(r1);
        const float r2 = r1 - h2;    // exact
        part[e] = j == 0 ? h1 : j == 1 ? h2 : r2;
      }
    }
    qa[kk] = Bf16::pack(part);  // each part is a bf16 value: packing is exact
  }

  if constexpr (NF) {
    // the gain, once per workgroup; read only after the first row's barrier.
    // These loads are waited for here, before the first copy is issued.
    for (int k = tid; k < D / 4; k += 64 * kP1Waves)
      *reinterpret_cast<float4*>(gam_buf + 4 * k) = p.nf_g ? ldf4(p.nf_g + 4 * k) : make_float4(1.f, 1.f, 1.f, 1.f);
  }

  // Vector-memory operations this wave has issued (copies, block-sum and
  // output stores; the statistics stores of wave 0 are left out, which only
  // makes the waits stricter), and the count right after each in-flight
  // row's copy was issued, oldest first.
  int issued = 0;
  int mark[PF];
  const int64_t G = gridDim.x;
  #pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int64_t r = blockIdx.x + f * G;
    if (r < p.R) issued += p1_stage<KS, NC>(p, r, ring + f * Sh::SLOT, w, l);
    mark[f] = issued;
  }

  int slot = 0, parity = 0;
  for (int64_t row = blockIdx.x; row < p.R; row += G) {
    __bf16* cur = ring + slot * Sh::SLOT;
    float* cred = cred_buf + parity * (kP1Waves * kP1MaxS * NC);
    float* ssred = ssred_buf + parity * (kP1Waves * NC);
    p1_wait(issued - mark[0]);  // this wave's part of the row has landed in LDS
    #pragma unroll
    for (int f = 0; f + 1 < PF; ++f) mark[f] = mark[f + 1];
    if (has_close && owner) {
      // b = round(p + v) (or v) over the chunk this wave copied; stored as the block sum
      __bf16* bv = cur + (size_t)(NC - 1) * STRIDE + tid * 8;
      uint4 u = *reinterpret_cast<const uint4*>(bv);
      if (p.cl.p) {
        const uint4 a = *reinterpret_cast<const uint4*>(cur + (size_t)NC * STRIDE + tid * 8);
        float fa[8], fv[8];
        Bf16::unpack(a, fa);
        Bf16::unpack(u, fv);
        #pragma unroll
        for (int e = 0; e < 8; ++e) fa[e] += fv[e];
        u = Bf16::pack(fa);
        *reinterpret_cast<uint4*>(bv) = u;
      }
#if ATTNRES_P1_B_NT
      st16_stream(uniform_ptr(static_cast<char*>(p.cl.b) + row * rowbytes) + (uint32_t)(tid * 16), u);
#else
      st16_global(uniform_ptr(static_cast<char*>(p.cl.b) + row * rowbytes) + (uint32_t)(tid * 16), u);
#endif
      issued += 1;
    }
    if constexpr (!Sh::PRIVATE) {
      lds_barrier();  // every wave's copy of this row (and the block sum) is in LDS;
                      // every wave is done with the previous row's slot
    } else {
      // this wave's own reads of the previous row's slot (refilled below) are done
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    {
      const int64_t ahead = row + PF * G;
      const int fill = slot == 0 ? NBUF - 1 : slot - 1;  // the previous row's slot
      if (ahead < p.R) issued += p1_stage<KS, NC>(p, ahead, ring + fill * Sh::SLOT, w, l);
      mark[PF - 1] = issued;
    }

    // scores C[(s, j)][i] over this wave's hidden slice (two 16-row tiles of A;
    // even and odd k-steps accumulate separately), and sums of squares. B
    // columns past the row's sources read a real source row: a column of C
    // depends only on its own column of B, and those columns are not used.
    float ss0 = 0.f, ss1 = 0.f;
    const __bf16* bsrc = cur + (size_t)(col < NC ? col : NC - 1) * STRIDE + w * (D / kP1Waves) + 8 * kg;
    f32x4_t c[4];
    #pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t gacc = f32x4_t{0.f, 0.f, 0.f, 0.f};  // NF: G[k][i] = b_k . b_i over the slice
    // Both A tiles every k-step (the second is zero for S <= 4): a branch here
    // would keep the compiler from issuing the next LDS reads ahead of the
    // current products.
    #pragma unroll
    for (int kk = 0; kk < KS / 2; ++kk) {
      const uint4 b = *reinterpret_cast<const uint4*>(bsrc + 32 * kk);
      float& ss = (kk & 1) ? ss1 : ss0;
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.x),
                                           __builtin_bit_cast(bf16x2v_t, b.x), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.y),
                                           __builtin_bit_cast(bf16x2v_t, b.y), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.z),
                                           __builtin_bit_cast(bf16x2v_t, b.z), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.w),
                                           __builtin_bit_cast(bf16x2v_t, b.w), ss, false);
      const int e = (kk & 1) * 2;
      c[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[2 * kk]),
                                                    __builtin_bit_cast(bf16x8_t, b), c[e], 0, 0, 0);
      c[e + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[2 * kk + 1]),
                                                        __builtin_bit_cast(bf16x8_t, b), c[e + 1], 0, 0, 0);
      if constexpr (NF)  // a lane's B fragment (column col, k-group kg) is also the A fragment of row col
        gacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                      __builtin_bit_cast(bf16x8_t, b), gacc, 0, 0, 0);
      if (kP1Fence > 0 && kk % kP1Fence == kP1Fence - 1)
        __builtin_amdgcn_sched_barrier(0);  // bound the LDS reads in flight
    }
    // sum of squares of source col over this wave's slice: add the four k-groups
    float ss = ss0 + ss1;
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (col < NC) {
      // D element r of lane l is row 4 (l / 16) + r, column l % 16 of its tile:
      // parts r = 0, 1, 2 of query 4 t + l / 16 (part 3 is zero)
      cred[(w * kP1MaxS + kg) * NC + col] = (c[0][0] + c[2][0]) + (c[0][1] + c[2][1]) + (c[0][2] + c[2][2]);
      cred[(w * kP1MaxS + 4 + kg) * NC + col] = (c[1][0] + c[3][0]) + (c[1][1] + c[3][1]) + (c[1][2] + c[3][2]);
      if (kg == 0) ssred[w * NC + col] = ss;
      if constexpr (NF) {
        float* gr = gram_buf + parity * (kP1Waves * NC * NC) + w * (NC * NC);
        #pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * kg + r < NC) gr[(4 * kg + r) * NC + col] = gacc[r];
      }
    }
    lds_barrier();

    // softmax, computed by every wave for itself: lane 8 s + i holds the score
    // of source i for query s
    const int i = l & 7, sq_ = l >> 3;
    float alpha;
    {
      const bool valid = i < NC && sq_ < S;
      float sc = -INFINITY;
      if (valid) {
        float dot[kP1Waves], sq[kP1Waves];
        #pragma unroll
        for (int ww = 0; ww < kP1Waves; ++ww) {
          dot[ww] = cred[(ww * kP1MaxS + sq_) * NC + i];
          sq[ww] = ssred[ww * NC + i];
        }
        #pragma unroll
        for (int h = kP1Waves / 2; h >= 1; h /= 2)
          #pragma unroll
          for (int ww = 0; ww < h; ++ww) {
            dot[ww] += dot[ww + h];
            sq[ww] += sq[ww + h];
          }
        sc = dot[0] * rsqrtf(sq[0] * p.invD + p.eps);
      }
      const float m = group8_max(sc);
      const float e = valid ? __expf(sc - m) : 0.f;
      const float z = group8_sum(e);
      alpha = e * (1.0f / z);
      if (w == 0 && i == 0 && sq_ < S) {
        if (p.m_out) p.m_out[(int64_t)sq_ * p.R + row] = m;
        p.lse_out[(int64_t)sq_ * p.R + row] = m + __logf(z);
      }
    }
    // NF: the sum of squares of output 0 over the whole row, as
    // alpha_0^T G alpha_0 from the reduced Gram matrix (lane 8 k + i takes
    // one term); every wave forms it for itself. It is taken from the fp32
    // output rather than the rounded one the norm is applied to: the two
    // differ by a relative O(2^-8 / sqrt(D)).
    float nf_inv = 0.f;
    if constexpr (NF) {
      const int gk = l >> 3, gi = l & 7;
      const float ak = __shfl(alpha, gk), ai = __shfl(alpha, gi);  // lanes 0..7 hold query 0's weights
      float t = 0.f;
      if (gk < NC && gi < NC) {
        const float* gr = gram_buf + parity * (kP1Waves * NC * NC) + gk * NC + gi;
        float gs = 0.f;
        #pragma unroll
        for (int ww = 0; ww < kP1Waves; ++ww) gs += gr[ww * (NC * NC)];
        t = ak * (ai * gs);
      }
      nf_inv = rsqrtf(wave_sum(t) * p.invD + p.nf_eps);
    }

    // outputs on the matrix cores: o_s[d] = sum_i alpha[s][i] b_i[d] as
    // 32x32x16 bf16 products with fp32 accumulation. A row 4 s + j holds
    // part j of alpha[s][0..7] (the exact three-part bf16 split; row 4 s + 3
    // and queries past S are zero) in k-group 0 for the first pass and in
    // k-group 1 for the second. B column n is the 8 sources at one element:
    // in the e-th product, element e of the vector of lane n (k-group 0) and
    // of lane n + 32 (k-group 1), so the first pass yields lane n's vector and
    // the second lane n + 32's. Accumulator r of lane l is row
    // 8 (r / 4) + 4 (l / 32) + r % 4: query 2 (r / 4) + l / 32, part r % 4 --
    // every lane ends with 8 consecutive outputs of 4 queries, stored as
    // 16-byte vectors. Non-finite sources make the whole wave's outputs
    // unspecified (a zero weight times Inf is NaN). Without an output buffer
    // (statistics only) the pass is skipped and nothing is counted.
    if (owner && p.out != nullptr) {
      uint4 x[8];
      #pragma unroll
      for (int k = 0; k < 8; ++k)
        x[k] = k < NC ? *reinterpret_cast<const uint4*>(cur + (size_t)k * STRIDE + tid * 8)
                      : make_uint4(0, 0, 0, 0);
      const int am = l & 31, as = am >> 2, aj = am & 3;
      // alpha[as][0..7] (lanes 8 as .. 8 as + 7) through this wave's LDS row
      float* arow = alpha_buf + w * 64;
      arow[l] = alpha;
      const float4 a0 = *reinterpret_cast<const float4*>(arow + 8 * as);
      const float4 a1 = *reinterpret_cast<const float4*>(arow + 8 * as + 4);
      const float al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float part[8];
      #pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = al[k];
        const float h1 = bf16_round(a);
        const float r1 = a - h1;  // exact
        const float h2 = bf16_round(r1);
        const float r2 = r1 - h2;  // exact
        part[k] = (as >= S || k >= NC) ? 0.f : aj == 0 ? h1 : aj == 1 ? h2 : aj == 2 ? r2 : 0.f;
      }
      const uint4 af = Bf16::pack(part);  // each part is a bf16 value: packing is exact
      const uint4 z4 = make_uint4(0, 0, 0, 0);
      const bool upper = l >= 32;
      const f32x16_t zero16 = {};
      #pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const uint4 A = (upper == (pass == 1)) ? af : z4;
        float o[4][8];
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          // (x_{2t}[e], x_{2t+1}[e]) for t = 0..3
          uint32_t bt[4];
          #pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t lo = (e < 2 ? x[2 * t].x : e < 4 ? x[2 * t].y : e < 6 ? x[2 * t].z : x[2 * t].w);
            const uint32_t hi = (e < 2 ? x[2 * t + 1].x : e < 4 ? x[2 * t + 1].y : e < 6 ? x[2 * t + 1].z
                                                                                   : x[2 * t + 1].w);
            bt[t] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          const f32x16_t c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, A), __builtin_bit_cast(bf16x8_t, make_uint4(bt[0], bt[1], bt[2], bt[3])),
              zero16, 0, 0, 0);
          #pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[q][e] = (c[4 * q] + c[4 * q + 1]) + c[4 * q + 2];
            asm volatile("" : "+v"(o[q][e]));  // reduce now: the 16 accumulators die here
          }
        }
        const int vec = w * 64 + am + 32 * pass;  // vector of the row this lane writes
        // The lane's 64-bit offset from query 2q's row (query 2q + 1, in the
        // upper lanes, lies R rows further: beyond 4 GB for large tensors),
        // the same for every q; formed per row, so that the compiler does not
        // hold one per query and pass across the row loop.
        int64_t loff = (upper ? p.R * rowbytes : 0) + (int64_t)vec * 16;
        asm volatile("" : "+v"(loff));
        #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sq = 2 * q + (upper ? 1 : 0);
          gchar_t* dst = uniform_ptr(static_cast<char*>(p.out) + ((int64_t)(2 * q) * p.R + row) * rowbytes) + loff;
          if (q == 0) {
            // Output 0 (the lower lanes) goes to out0 or, with NF, to nf_out
            // as round(gain * round(h) * inv); query 1 (the upper lanes) is
            // stored by the same instruction, so the wave issues one store
            // here whatever S is.
            uint4 hv = Bf16::pack(o[0]);
            if constexpr (NF) {
              float f[8];
              Bf16::unpack(hv, f);
              const float4 g0 = *reinterpret_cast<const float4*>(gam_buf + vec * 8);
              const float4 g1 = *reinterpret_cast<const float4*>(gam_buf + vec * 8 + 4);
              const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
              #pragma unroll
              for (int e = 0; e < 8; ++e) f[e] = gg[e] * (f[e] * nf_inv);
              if (!upper) hv = Bf16::pack(f);
            }
            void* const base0 = NF ? p.nf_out : p.out0 ? p.out0 : p.out;
            gchar_t* d0 = uniform_ptr(static_cast<char*>(base0) + row * rowbytes) + (uint32_t)(vec * 16);
            gchar_t* d1 = p.out1 ? uniform_ptr(static_cast<char*>(p.out1) + row * rowbytes) + (uint32_t)(vec * 16)
                                 : dst;
            if (!upper || S > 1) st16_global(upper ? d1 : d0, hv);
            continue;
          }
          if (2 * q < S && sq < S) {
            if (sq >= ATTNRES_P1_OUT_NT_FROM)
              st16_stream(dst, Bf16::pack(o[q]));
            else
              st16_global(dst, Bf16::pack(o[q]));
          }
        }
      }
      issued += 2 * ((S + 1) >> 1);
    }
    slot = slot == NBUF - 1 ? 0 : slot + 1;
    parity ^= 1;
  }
}

// ---------------------------------------------------------------------------
// Aggregate over any number of sources with one query [K3 (A1)-(A3); WC
// depth_summary/merge_summary/finish]. Sources are taken in register-resident
// groups of G; each group's scores are reduced across the row and folded into
// a running (m, z, numerator) triple by the online-softmax merge (OS2), so
// every source is read exactly once whatever n is.
// ---------------------------------------------------------------------------
struct AggParams {
  const void* src[64];
  int n;
  const float* w;  // [D]
  const float* gm; // [D] or null
  float eps;
  void* out;       // [R][D]
  float* m_out;    // [R] or null
  float* lse_out;  // [R] or null
  Close cl;        // close computing source n-1, or cl.v == null
  const void* o_init;     // [R][D] normalised output of an earlier group, or null
  const float* lse_init;  // [R] its log-sum-exp
  const float* nf_g = nullptr;  // with nf_out: the output is written as its sublayer's
  float nf_eps = 0.f;           // input norm to nf_out (and not to out)
  void* nf_out = nullptr;
  Geom g;
};

template <class T, int VPL, int G, bool PK>
__global__ __launch_bounds__(512) void aggregate_kernel(AggParams p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  constexpr int NV = 2 * G;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  const bool has_close = p.cl.v != nullptr;

  // this lane's slice of the folded query, reused for every row
  float q[VPL][EPV];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V) {
      load_query<EPV>(p.w, p.gm, (int64_t)vec * EPV, q[c]);
    } else {
      #pragma unroll
      for (int e = 0; e < EPV; ++e) q[c][e] = 0.f;
    }
  }

  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    // loads are unconditional (a row past the end reads row 0, a lane past
    // the row's end reads vector 0; both are discarded), so no branch hides
    // them from the compiler's wait counting and a group's loads are waited
    // for together
    const int64_t base = (rv ? row : 0) * rowbytes;
    int64_t voff[VPL];
    bool in_row[VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      in_row[c] = vec < g.V;
      voff[c] = base + (int64_t)(in_row[c] ? vec : 0) * 16;
    }
    // the closing source b = round(p + v) (or v), formed and stored before
    // the group loads
    uint4 bcl[VPL];
    if (has_close) {
      const char* pp = static_cast<const char*>(p.cl.p ? p.cl.p : p.cl.v);
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const uint4 v = ld16_stream(static_cast<const char*>(p.cl.v) + voff[c]);
        const uint4 a = ld16_stream(pp + voff[c]);
        float fa[EPV], fv[EPV];
        T::unpack(a, fa);
        T::unpack(v, fv);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) fa[e] = p.cl.p ? fa[e] + fv[e] : fv[e];
        bcl[c] = T::pack(fa);  // rounded to the I/O dtype, as the block sum is stored
        if (rv && in_row[c]) st16_stream(static_cast<char*>(p.cl.b) + voff[c], bcl[c]);
      }
    }
    float num[VPL][EPV];
    float m_run = -FLT_MAX, z_run = 0.f;
    if (p.o_init) {
      // start from an earlier group's summary (lse, z = 1, u = o): the
      // single-triple form of a normalised group [K3 9.4 (OS1)]
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const uint4 u = ld16_stream(static_cast<const char*>(p.o_init) + voff[c]);
        T::unpack(u, num[c]);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) num[c][e] = in_row[c] ? num[c][e] : 0.f;
      }
      m_run = p.lse_init[rv ? row : 0];
      z_run = 1.f;
    } else {
      #pragma unroll
      for (int c = 0; c < VPL; ++c)
        #pragma unroll
        for (int e = 0; e < EPV; ++e) num[c][e] = 0.f;
    }

    for (int i0 = 0; i0 < p.n; i0 += G) {
      uint4 u[G][VPL];
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        // slots past n and the closing source (already in bcl) read the
        // sink's first 16 bytes, which stay in cache
        const int i = i0 + j;
        const bool live = i < p.n && !(has_close && i == p.n - 1);
        const char* sp = static_cast<const char*>(p.src[live ? i : 0]);
        #pragma unroll
        for (int c = 0; c < VPL; ++c)
          u[j][c] = ld16_stream(live ? sp + voff[c] : reinterpret_cast<const char*>(g_store_sink));
      }
      // With PK the group's sources stay packed and each use unpacks them
      // again; otherwise they are unpacked once and held. Masked either way:
      // slots past n and lanes past the row's end contribute zero. Packed, the
      // 8-source group at 2 vectors per lane takes 160 VGPRs instead of 217
      // (3 waves per SIMD instead of 2) for twice the unpacking.
      float x[PK ? 1 : G][PK ? 1 : VPL][EPV];
      if constexpr (PK) {
        // the closing source takes its slot's registers once
        #pragma unroll
        for (int j = 0; j < G; ++j)
          if (has_close && i0 + j == p.n - 1)
            #pragma unroll
            for (int c = 0; c < VPL; ++c) u[j][c] = bcl[c];
      }
      auto unpack_keep = [&](int j, int c, float* xo) {
        const bool closing = !PK && has_close && i0 + j == p.n - 1;
        T::unpack(closing ? bcl[c] : u[j][c], xo);
        const bool keep = i0 + j < p.n && in_row[c];
        #pragma unroll
        for (int e = 0; e < EPV; ++e) xo[e] = keep ? xo[e] : 0.f;
      };
      float red[NV];
      #pragma unroll
      for (int k = 0; k < NV; ++k) red[k] = 0.f;
      if constexpr (PK) {
        #pragma unroll
        for (int j = 0; j < G; ++j)
          #pragma unroll
          for (int c = 0; c < VPL; ++c) {
            float xt[EPV];
            unpack_keep(j, c, xt);
            #pragma unroll
            for (int e = 0; e < EPV; ++e) {
              red[j] += q[c][e] * xt[e];
              red[G + j] += xt[e] * xt[e];
            }
          }
        // the packed registers look new here, so the unpacked values above
        // are not kept alive for the numerators below
        #pragma unroll
        for (int j = 0; j < G; ++j)
          #pragma unroll
          for (int c = 0; c < VPL; ++c)
            asm volatile("" : "+v"(u[j][c].x), "+v"(u[j][c].y), "+v"(u[j][c].z), "+v"(u[j][c].w));
      } else {
        #pragma unroll
        for (int j = 0; j < G; ++j)
          #pragma unroll
          for (int c = 0; c < VPL; ++c) unpack_keep(j, c, x[j][c]);
        #pragma unroll
        for (int j = 0; j < G; ++j)
          #pragma unroll
          for (int c = 0; c < VPL; ++c)
            #pragma unroll
            for (int e = 0; e < EPV; ++e) {
              red[j] += q[c][e] * x[j][c][e];
              red[G + j] += x[j][c][e] * x[j][c][e];
            }
      }
      row_reduce<NV>(red, lds, ln.slot, ln.wr, g.W);
      float sc[G];
      float m_new = m_run;
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        sc[j] = red[j] * rsqrtf(red[G + j] * g.invD + p.eps);
        if (i0 + j < p.n) m_new = fmaxf(m_new, sc[j]);
      }
      const float rescale = __expf(m_run - m_new);
      z_run *= rescale;
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        sc[j] = (i0 + j < p.n) ? __expf(sc[j] - m_new) : 0.f;
        z_run += sc[j];
      }
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        #pragma unroll
        for (int e = 0; e < EPV; ++e) num[c][e] *= rescale;
        #pragma unroll
        for (int j = 0; j < G; ++j) {
          float xt[EPV];
          if constexpr (PK) unpack_keep(j, c, xt);
          #pragma unroll
          for (int e = 0; e < EPV; ++e) num[c][e] += sc[j] * (PK ? xt[e] : x[PK ? 0 : j][PK ? 0 : c][e]);
        }
      }
      m_run = m_new;
    }
    if (p.nf_out) {
      // the sublayer input norm of the rounded output [ZZ block listing:
      // attn(attn_norm(h))]: its sum of squares over the row, then gamma_f h / rms
      const float rz = 1.0f / z_run;
      uint4 hv[VPL];
      float hss[1] = {0.f};
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float o[EPV];
        #pragma unroll
        for (int e = 0; e < EPV; ++e) o[e] = num[c][e] * rz;
        hv[c] = T::pack(o);
        T::unpack(hv[c], o);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) hss[0] += in_row[c] ? o[e] * o[e] : 0.f;
      }
      row_reduce<1>(hss, lds, ln.slot, ln.wr, g.W);
      if (rv) {
        const float inv = rsqrtf(hss[0] * g.invD + p.nf_eps);
        char* orow = static_cast<char*>(p.nf_out) + row * rowbytes;
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          const int vec = c * ln.stride + ln.t;
          if (vec < g.V) {
            float o[EPV], gn[EPV];
            T::unpack(hv[c], o);
            load_gain<EPV>(p.nf_g, (int64_t)vec * EPV, gn);
            #pragma unroll
            for (int e = 0; e < EPV; ++e) o[e] = gn[e] * (o[e] * inv);
            st16(orow + (int64_t)vec * 16, T::pack(o));
          }
        }
      }
    } else if (rv) {
      const float rz = 1.0f / z_run;
      char* orow = static_cast<char*>(p.out) + row * rowbytes;
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int vec = c * ln.stride + ln.t;
        if (vec < g.V) {
          float o[EPV];
          #pragma unroll
          for (int e = 0; e < EPV; ++e) o[e] = num[c][e] * rz;
          st16_stream(orow + (int64_t)vec * 16, T::pack(o));
        }
      }
    }
    if (rv && ln.t == 0) {
      if (p.m_out) p.m_out[row] = m_run;
      if (p.lse_out) p.lse_out[row] = m_run + __logf(z_run);
    }
  }
}

// ---------------------------------------------------------------------------
// Aggregate backward with recomputation [K3 "Attention Residual" eqs. A1-A3
// differentiated; the course's fused backward that recomputes the softmax
// instead of storing it]. Nothing of the forward is kept: per row the scores
// are recomputed from the sources, and with a_i = softmax(s)_i,
// g_i = dh . V_i and ds_i = a_i (g_i - sum_j a_j g_j) (dh . h is sum_j a_j g_j,
// so h itself is never formed):
//   dV_i = a_i dh + (ds_i / r_i) q~ - (ds_i s_i / (D r_i^2)) V_i
//   dq~ += (ds_i / r_i) V_i
// One row reduction yields the 3n sums q~.V_i, V_i.V_i and dh.V_i. With n <= G
// the sources stay in registers (raw 16-byte vectors) between the reduction
// and the gradient pass, so each source is read once; beyond G they are
// streamed twice (groups of G), the per-source statistics kept in LDS.
// dq~ is summed over rows per (workgroup, row slot) into `partial`, which a
// fixed-order reduction turns into dw = (sum_rows dq~) * gamma and
// dgamma = (sum_rows dq~) * w: the summation order depends only on the
// shape, so the result is deterministic.
// ---------------------------------------------------------------------------
struct AggBwdParams {
  const void* src[64];
  float* dV[64];       // [R][D] fp32 each
  int n;
  int accumulate;      // nonzero: dV_i += gradient
  const float* w;      // [D]
  const float* gm;     // [D] or null
  float eps;
  const void* dh;      // [R][D] in the I/O dtype
  const float* dh_scale;  // [R] or null: the upstream gradient is dh_scale[r] * dh[r]
  const float* dlse;      // [R] or null: gradient of the group's log-sum-exp, added to every score's
  float* partial;      // [gridDim.x * RPW][D]
  Geom g;
};

// per-source row statistics of the backward: score, 1/r, dh . V
struct BwdStat {
  float s, ri, gd;
};

// A row-uniform value moved into a scalar register (frees a vector register).
__device__ __forceinline__ float uniformf(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Opaque to the optimiser: the value must be re-read from these registers,
// so values derived from it earlier (unpacked copies) are not kept alive.
__device__ __forceinline__ void pin(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void pin(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }

// Four-element vectors of the backward. A lane's fp32 gradient of one vector
// is then 16 contiguous bytes, and a wave's gradient store covers 1 KiB with
// no gaps (with eight-element bf16 vectors each lane would write 32 bytes in
// two strided halves, which measured 1.6x the algorithmic write traffic).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2_t gu32x2_t;
struct Bf16x4 {
  typedef uint2 raw;
  static constexpr int kBytes = 8;
  static __device__ __forceinline__ raw load(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
  }
  static __device__ __forceinline__ raw zero() { return make_uint2(0, 0); }
  static __device__ __forceinline__ void unpack(const raw& v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};
struct F32x4 {
  typedef uint4 raw;
  static constexpr int kBytes = 16;
  static __device__ __forceinline__ raw load(const void* p) { return ld16_stream(p); }
  static __device__ __forceinline__ raw zero() { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ void unpack(const raw& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

#ifndef ATTNRES_BWD_DV_NT
#define ATTNRES_BWD_DV_NT 1  // gradients are written once: non-temporal stores
#endif

// dV = A dh + B q~ + C x for the 4 elements of one vector, written (or added)
// as 16 bytes of fp32 at dst.
template <class F, bool ACC>
__device__ __forceinline__ void bwd_store_dv(float* __restrict__ dst, const typename F::raw& dhr,
                                             const float* q, const typename F::raw& xr, float A,
                                             float B, float C) {
  float dh[4], x[4];
  F::unpack(dhr, dh);
  F::unpack(xr, x);
  float o[4];
  #pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = A * dh[k] + B * q[k] + C * x[k];
  if constexpr (ACC) {
    const uint4 u = ld16_stream(dst);
    o[0] += __uint_as_float(u.x); o[1] += __uint_as_float(u.y);
    o[2] += __uint_as_float(u.z); o[3] += __uint_as_float(u.w);
  }
  const uint4 u = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                             __float_as_uint(o[3]));
#if ATTNRES_BWD_DV_NT
  st16_stream(dst, u);
#else
  st16(dst, u);
#endif
}

// dq~ += B x over the 4 elements of one vector
template <class F>
__device__ __forceinline__ void bwd_acc_dq(float* dq, const typename F::raw& xr, float B) {
  float x[4];
  F::unpack(xr, x);
  #pragma unroll
  for (int e = 0; e < 4; ++e) dq[e] += B * x[e];
}

// Geometry: g.V counts four-element vectors; lane t holds vectors
// c * 64W + t (c < VPL) of its row.
#ifndef ATTNRES_BWD_WAVES_PER_EU
#define ATTNRES_BWD_WAVES_PER_EU 1  // minimum waves per SIMD the register budget must allow
#endif

// ACC: the gradients are added to dV (a compile-time choice, so the plain
// form has no branch around its stores).
template <class F, int VPL, int G, bool RES, bool ACC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(ATTNRES_BWD_WAVES_PER_EU)))
void aggregate_bwd_kernel(AggBwdParams p) {
  extern __shared__ float lds[];
  typedef typename F::raw raw;
  constexpr int NV = 3 * G;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * F::kBytes;
  // per-wave statistics of every source (streamed form only), after the
  // row-reduction scratch
  BwdStat* stat = reinterpret_cast<BwdStat*>(lds + (size_t)g.RPW * g.W * NV) +
                  (size_t)(threadIdx.x >> 6) * 64;

  float q[VPL][4], dq[VPL][4];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V) {
      load_query<4>(p.w, p.gm, (int64_t)vec * 4, q[c]);
    } else {
      #pragma unroll
      for (int e = 0; e < 4; ++e) q[c][e] = 0.f;
    }
    #pragma unroll
    for (int e = 0; e < 4; ++e) dq[c][e] = 0.f;
  }

  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    raw dhr[VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      dhr[c] = (rv && vec < g.V)
                   ? F::load(static_cast<const char*>(p.dh) + row * rowbytes + (int64_t)vec * F::kBytes)
                   : F::zero();
    }

    // pass 1: the 3 row sums of every source (one group when resident)
    raw x[G][VPL];
    float m_run = -FLT_MAX, z_run = 0.f, eg_run = 0.f;  // streamed form: online softmax
    BwdStat st[G];
    for (int i0 = 0; i0 < p.n; i0 += G) {
      #pragma unroll
      for (int j = 0; j < G; ++j)
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          const int vec = c * ln.stride + ln.t;
          x[j][c] = (rv && i0 + j < p.n && vec < g.V)
                        ? F::load(static_cast<const char*>(p.src[i0 + j]) + row * rowbytes +
                                  (int64_t)vec * F::kBytes)
                        : F::zero();
        }
      float red[NV];
      #pragma unroll
      for (int k = 0; k < NV; ++k) red[k] = 0.f;
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float dh[4];
        F::unpack(dhr[c], dh);
        #pragma unroll
        for (int j = 0; j < G; ++j) {
          float xf[4];
          F::unpack(x[j][c], xf);
          #pragma unroll
          for (int e = 0; e < 4; ++e) {
            red[j] += q[c][e] * xf[e];
            red[G + j] += xf[e] * xf[e];
            red[2 * G + j] += dh[e] * xf[e];
          }
        }
      }
      row_reduce<NV>(red, lds, ln.slot, ln.wr, g.W);
      const float gscale = p.dh_scale ? p.dh_scale[rv ? row : 0] : 1.f;
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        const float ri = rsqrtf(uniformf(red[G + j]) * g.invD + p.eps);
        st[j].ri = uniformf(ri);
        st[j].s = uniformf(uniformf(red[j]) * ri);
        st[j].gd = uniformf(gscale * uniformf(red[2 * G + j]));
      }
      if (RES) {
        #pragma unroll
        for (int j = 0; j < G; ++j)
          #pragma unroll
          for (int c = 0; c < VPL; ++c) pin(x[j][c]);
        #pragma unroll
        for (int c = 0; c < VPL; ++c) pin(dhr[c]);
      } else {
        if (ln.lane == 0) {
          #pragma unroll
          for (int j = 0; j < G; ++j)
            if (i0 + j < p.n) stat[i0 + j] = st[j];
        }
        float m_new = m_run;
        #pragma unroll
        for (int j = 0; j < G; ++j)
          if (i0 + j < p.n) m_new = fmaxf(m_new, st[j].s);
        const float rescale = __expf(m_run - m_new);
        z_run *= rescale;
        eg_run *= rescale;
        #pragma unroll
        for (int j = 0; j < G; ++j)
          if (i0 + j < p.n) {
            const float e = __expf(st[j].s - m_new);
            z_run += e;
            eg_run += e * st[j].gd;
          }
        m_run = uniformf(m_new);
        z_run = uniformf(z_run);
        eg_run = uniformf(eg_run);
      }
    }
    if (!rv) continue;  // uniform per row slot; no barrier follows in this iteration
    // the upstream gradient's row scale (its weight in a merge downstream) and
    // the gradient of the group's log-sum-exp: d lse / d s_i = a_i
    const float gs = uniformf(p.dh_scale ? p.dh_scale[row] : 1.f);
    const float dl = uniformf(p.dlse ? p.dlse[row] : 0.f);

    if (RES) {
      // softmax over the n resident sources
      float m = -FLT_MAX;
      #pragma unroll
      for (int j = 0; j < G; ++j)
        if (j < p.n) m = fmaxf(m, st[j].s);
      float a[G], z = 0.f;
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        a[j] = j < p.n ? __expf(st[j].s - m) : 0.f;
        z += a[j];
      }
      const float rz = 1.0f / z;
      float gbar = 0.f;
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        a[j] = uniformf(a[j] * rz);
        gbar += a[j] * st[j].gd;
      }
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        if (j >= p.n) continue;
        // one source at a time: keeps its unpacked values short-lived
        __builtin_amdgcn_sched_barrier(0);
        const float ds = a[j] * (st[j].gd - gbar + dl);
        const float B = uniformf(ds * st[j].ri);
        const float C = uniformf(-B * st[j].s * st[j].ri * g.invD);
        const float A = uniformf(a[j] * gs);
        float* dst = p.dV[j] + row * g.D;
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          // a lane past the row's end holds zeros (nothing added to dq~) and
          // stores to the sink
          const int vec = c * ln.stride + ln.t;
          float* to = reinterpret_cast<float*>(
              store_target(vec < g.V, reinterpret_cast<char*>(dst + (int64_t)vec * 4)));
          bwd_store_dv<F, ACC>(to, dhr[c], q[c], x[j][c], A, B, C);
          bwd_acc_dq<F>(dq[c], x[j][c], B);
        }
      }
    } else {
      // pass 2: stream the sources again with the statistics of pass 1
      const float rz = 1.0f / z_run;
      const float gbar = eg_run * rz;
      for (int i = 0; i < p.n; ++i) {
        const BwdStat si = stat[i];
        const float a = uniformf(__expf(si.s - m_run) * rz);
        const float ds = a * (si.gd - gbar + dl);
        const float B = uniformf(ds * si.ri);
        const float C = uniformf(-B * si.s * si.ri * g.invD);
        const float A = uniformf(a * gs);
        const char* srow = static_cast<const char*>(p.src[i]) + row * rowbytes;
        float* dst = p.dV[i] + row * g.D;
        raw xr[VPL];
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          const int vec = c * ln.stride + ln.t;
          xr[c] = F::load(srow + (int64_t)(vec < g.V ? vec : 0) * F::kBytes);
          if (!(vec < g.V)) xr[c] = F::zero();
        }
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          const int vec = c * ln.stride + ln.t;
          float* to = reinterpret_cast<float*>(
              store_target(vec < g.V, reinterpret_cast<char*>(dst + (int64_t)vec * 4)));
          bwd_store_dv<F, ACC>(to, dhr[c], q[c], xr[c], A, B, C);
          bwd_acc_dq<F>(dq[c], xr[c], B);
        }
      }
    }
  }

  // this (workgroup, row slot)'s sum of dq~ over its rows
  float* prow = p.partial + ((int64_t)blockIdx.x * g.RPW + ln.slot) * g.D;
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V)
      st16(prow + (int64_t)vec * 4, make_uint4(__float_as_uint(dq[c][0]), __float_as_uint(dq[c][1]),
                                               __float_as_uint(dq[c][2]), __float_as_uint(dq[c][3])));
  }
}

// ---------------------------------------------------------------------------
// Backward of one Phase-2 merge [K3 9.4 (OS2) and the single-source triple,
// differentiated; recomputation as in the aggregate backward]. The merge is
// a two-term softmax: h = a o + c p with (a, c) = softmax(lse, s_p) and
// s_p = q~ . p / r_p, r_p = sqrt(mean_d p^2 + eps). Per row, with the
// upstream gradient dh and gh = dh . h = a (dh . o) + c (dh . p):
//   d lse = a (dh . o - gh),   d s_p = c (dh . p - gh)
//   dp    = c dh + (d s_p / r_p) q~ - (d s_p s_p / (D r_p^2)) p
//   dq~  += (d s_p / r_p) p
// and the group's output o receives a dh (returned as the weight a, so the
// Phase-1 backward scales dh itself). One row reduction gives q~.p, p.p,
// dh.o and dh.p; g_out = g_in + dp (the partial's gradient accumulated from
// its later uses, the partial chain p_{j+1} = p_j + v_j).
// ---------------------------------------------------------------------------
struct MergeBwdParams {
  const void* o;
  const float* lse;
  const void* ps;
  const float* w;
  const float* gm;
  float eps;
  const void* dh;
  const float* g_in;
  float* g_out;
  float* a_out;
  float* dlse_out;
  float* partial;  // [gridDim.x * RPW][D]
  Geom g;
};

template <class F, int VPL>
__global__ __launch_bounds__(512) void merge_bwd_kernel(MergeBwdParams p) {
  extern __shared__ float lds[];
  typedef typename F::raw raw;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * F::kBytes;
  float q[VPL][4], dq[VPL][4];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V) {
      load_query<4>(p.w, p.gm, (int64_t)vec * 4, q[c]);
    } else {
      #pragma unroll
      for (int e = 0; e < 4; ++e) q[c][e] = 0.f;
    }
    #pragma unroll
    for (int e = 0; e < 4; ++e) dq[c][e] = 0.f;
  }
  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    const int64_t base = (rv ? row : 0) * rowbytes;
    raw orw[VPL], prw[VPL], dhr[VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      const int64_t off = base + (int64_t)(vec < g.V ? vec : 0) * F::kBytes;
      orw[c] = F::load(static_cast<const char*>(p.o) + off);
      prw[c] = F::load(static_cast<const char*>(p.ps) + off);
      dhr[c] = F::load(static_cast<const char*>(p.dh) + off);
    }
    float red[4] = {0.f, 0.f, 0.f, 0.f};  // q~.p, p.p, dh.o, dh.p
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const bool in_row = c * ln.stride + ln.t < g.V;
      float fo[4], fp[4], fd[4];
      F::unpack(orw[c], fo);
      F::unpack(prw[c], fp);
      F::unpack(dhr[c], fd);
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = in_row ? fp[e] : 0.f, de = in_row ? fd[e] : 0.f;
        red[0] += q[c][e] * pe;
        red[1] += pe * pe;
        red[2] += de * fo[e];
        red[3] += de * pe;
      }
    }
    row_reduce<4>(red, lds, ln.slot, ln.wr, g.W);
    if (!rv) continue;  // uniform per row slot; no barrier follows in this iteration
    const float rp = rsqrtf(red[1] * g.invD + p.eps);  // 1 / r_p
    const float sp = red[0] * rp;
    const float l = p.lse[row];
    const float M = fmaxf(l, sp);
    float a = __expf(l - M), cw = __expf(sp - M);
    const float rz = 1.0f / (a + cw);
    a *= rz;
    cw *= rz;
    const float gh = a * red[2] + cw * red[3];
    const float dl = a * (red[2] - gh);
    const float dsp = cw * (red[3] - gh);
    const float B = uniformf(dsp * rp);
    const float C = uniformf(-B * sp * rp * g.invD);
    const float A = uniformf(cw);
    float* gout = p.g_out + row * g.D;
    const float* gin = p.g_in ? p.g_in + row * g.D : nullptr;
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      if (vec < g.V) {
        float fp[4], fd[4], o4[4];
        F::unpack(prw[c], fp);
        F::unpack(dhr[c], fd);
        if (gin) {
          const uint4 u = ld16_stream(gin + (int64_t)vec * 4);
          o4[0] = __uint_as_float(u.x); o4[1] = __uint_as_float(u.y);
          o4[2] = __uint_as_float(u.z); o4[3] = __uint_as_float(u.w);
        } else {
          o4[0] = o4[1] = o4[2] = o4[3] = 0.f;
        }
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
          o4[e] += A * fd[e] + B * q[c][e] + C * fp[e];
          dq[c][e] += B * fp[e];
        }
        st16_stream(gout + (int64_t)vec * 4, make_uint4(__float_as_uint(o4[0]), __float_as_uint(o4[1]),
                                                        __float_as_uint(o4[2]), __float_as_uint(o4[3])));
      }
    }
    if (ln.t == 0) {
      p.a_out[row] = a;
      p.dlse_out[row] = dl;
    }
  }
  float* prow = p.partial + ((int64_t)blockIdx.x * g.RPW + ln.slot) * g.D;
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V)
      st16(prow + (int64_t)vec * 4, make_uint4(__float_as_uint(dq[c][0]), __float_as_uint(dq[c][1]),
                                               __float_as_uint(dq[c][2]), __float_as_uint(dq[c][3])));
  }
}

// ---------------------------------------------------------------------------
// Batched Phase-1 backward [K3 9.4 step 1 and 9.1 (A1)-(A3) differentiated]:
// the S queries of a block, each an aggregate over the same n sources, take
// their gradients in one pass over the sources. Query j's output received
// a_j dh_j (a_j the merge weight of its group, dh_j the upstream gradient of
// its sublayer) and its log-sum-exp the merge's d lse_j. Per row and query,
// with s_ji = q~_j . V_i / r_i, alpha = softmax_i(s_j), g_ji = a_j dh_j . V_i:
//   ds_ji = alpha_ji (g_ji - sum_i alpha_ji g_ji + d lse_j)
//   dV_i += sum_j [ alpha_ji a_j dh_j + (ds_ji / r_i) q~_j ]
//           - (sum_j ds_ji s_ji / (D r_i^2)) V_i
//   dq~_j += sum_i (ds_ji / r_i) V_i   (per-workgroup partial rows)
// One workgroup row at a time, two 4-element vectors per lane (rows of at
// most 2 x 64 x 8 vectors), up to 8 queries per launch (a template
// parameter, so no argument array is indexed at run time):
//  - every load of a row is issued first, the dV_i it adds to included;
//  - each wave reduces the 2 S n + n row sums one (query, source) pair at a
//    time (q~.V in fp32, dh.V and V.V as v_dot2 on the bf16 pairs) into an
//    LDS table, double-buffered by row parity: one barrier per row;
//  - the coefficients are formed one (query, source) pair per lane (lane
//    8 j + i; the softmax over a query's sources is an 8-lane reduction) and
//    broadcast as scalars: computed as uniform values, every lane would run
//    the whole table;
//  - the folded queries live in LDS, each lane owning its elements (no
//    barrier); from global memory, each use of a query would wait for its
//    load. The dq~ sums do too with up to 4 queries; with more, the queries
//    alone fill 128 KiB at 4096 elements and the sums stay in registers.
// Sources and upstream gradients are read once; each dV_i is read and written
// once (added to), instead of once per query.
// ---------------------------------------------------------------------------
constexpr int kP1BwdQ = 8;  // queries per launch (the queries in LDS)
#ifndef ATTNRES_P1BWD_LATE_MAXN
#define ATTNRES_P1BWD_LATE_MAXN 2  // sources up to which more than 4 queries prefetch the next row
#endif
constexpr int kP1BwdVpl = 2;  // four-element vectors per lane
constexpr int kP1BwdMaxN = 8;  // sources

struct P1BwdParams {
  const void* src[kP1BwdMaxN];
  int n;
  int S;
  const void* dh[kP1BwdQ];
  const float* dh_scale[kP1BwdQ];  // [R] or null (1)
  const float* dlse[kP1BwdQ];      // [R] or null (0)
  const float* w[kP1BwdQ];         // [D] each
  const float* gm[kP1BwdQ];        // [D] or null
  float eps;
  float* dV[kP1BwdMaxN];           // [R][D] fp32, added to
  float* partial;                  // [S][gridDim.x][D]
  Geom g;
};

template <int NC, int SQ>
__global__ __launch_bounds__(512) void phase1_bwd_kernel(P1BwdParams p) {
  typedef Bf16x4 F;
  typedef F::raw raw;
  constexpr int VPL = kP1BwdVpl;
  // q~_j = w_j * gamma_j for this lane's four elements: both loads are issued
  // unconditionally (w stands in for a missing gain), since a load under a
  // branch makes the compiler wait for every load in flight
  auto query = [&](int j, int64_t el, float* q) {
    const float4 a = ldf4(p.w[j] + el);
    const float4 b = ldf4((p.gm[j] ? p.gm[j] : p.w[j]) + el);
    const bool hg = p.gm[j] != nullptr;
    q[0] = hg ? a.x * b.x : a.x;
    q[1] = hg ? a.y * b.y : a.y;
    q[2] = hg ? a.z * b.z : a.z;
    q[3] = hg ? a.w * b.w : a.w;
  };
  // row sums: q~_j.x_i [SQ][NC], dh_j.x_i [SQ][NC], x_i.x_i [NC]
  constexpr int NR = (2 * SQ + 1) * NC;
  // the dq~ sums of this workgroup's rows in registers (more than 4 queries)
  // or in LDS
  constexpr bool DQR = SQ > 4;
  // [SQ][D] folded queries, [SQ][D] dq~ sums (in LDS), then the wave sums
  // [2 (row parity)][W][NR]
  extern __shared__ float lds[];
  const Geom& g = p.g;
  float* qs = lds;
  float* dqs = lds + SQ * g.D;
  float* wsum = lds + (DQR ? 1 : 2) * SQ * g.D;
  const int t = threadIdx.x, wr = t >> 6, lane = t & 63, stride = 64 * g.W;
  const int64_t rowbytes = (int64_t)g.V * F::kBytes;  // a bf16 row
  const int64_t growbytes = (int64_t)g.D * 4;         // an fp32 gradient row
  bool in_row[VPL];
  int vec[VPL];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    vec[c] = c * stride + t;
    in_row[c] = vec[c] < g.V;
    if (!in_row[c]) vec[c] = 0;  // reads vector 0; its values are discarded
  }
  // Every row of every stream is addressed as a wave-uniform base plus one
  // 32-bit lane offset per vector (8 bytes a bf16 vector, 16 an fp32 one):
  // 64-bit lane addresses per stream, hoisted out of the row loop, took two
  // registers per stream and vector and spilled with 8 queries.
  auto ld_x = [&](const void* base, int64_t r, int c) -> raw {
    const gchar_t* b = uniform_ptr(static_cast<const char*>(base) + r * rowbytes);
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const gu32x2_t*>(b + (uint32_t)vec[c] * 8u));
    return make_uint2(v.x, v.y);
  };
  auto g_row = [&](float* base, int64_t r) { return uniform_ptr(reinterpret_cast<char*>(base) + r * growbytes); };
  // each lane owns its elements of the queries and of the dq~ sums: no
  // barrier is needed for either. The queries are read from LDS in every
  // row (from global memory, each first use would wait for its load).
  #pragma unroll
  for (int j = 0; j < SQ; ++j)
    #pragma unroll
    for (int c = 0; c < VPL; ++c)
      if (in_row[c]) {
        float q[4];
        query(j, (int64_t)vec[c] * 4, q);
        *reinterpret_cast<float4*>(qs + j * g.D + vec[c] * 4) = make_float4(q[0], q[1], q[2], q[3]);
        if constexpr (!DQR) *reinterpret_cast<float4*>(dqs + j * g.D + vec[c] * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
  float dqr[DQR ? SQ : 1][VPL][4];
  #pragma unroll
  for (int j = 0; j < (DQR ? SQ : 1); ++j)
    #pragma unroll
    for (int c = 0; c < VPL; ++c)
      #pragma unroll
      for (int e = 0; e < 4; ++e) dqr[j][c][e] = 0.f;
  // this lane's query elements (lanes past the row's end read element 0)
  auto qload = [&](int j, int c, float* q) {
    const float4 v = *reinterpret_cast<const float4*>(qs + j * g.D + vec[c] * 4);
    q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
  };

  // With few enough sources and queries, the next row's sources (PFX) and
  // upstream gradients (PFD) are loaded while this row's gradients are
  // formed (the registers of the two rows fit); otherwise each row's loads
  // come first in that row. With more than 4 queries (LATE), the source
  // gradients a row adds to are loaded after its row sums instead of with
  // its sources, which frees their registers for the next row's loads,
  // issued behind them. With 8 queries that fits up to 4 sources, but from 3
  // sources the compiler then waits for each query's row scale on its own,
  // so LATE stops at ATTNRES_P1BWD_LATE_MAXN sources (1..2 measured 0.7%
  // faster over the stack backward; 3 and 4 keep the loads at the row start).
  constexpr bool LATE = DQR && NC <= ATTNRES_P1BWD_LATE_MAXN;
  constexpr bool PFD = NC + SQ <= 10 || LATE;
  constexpr bool PFX = NC + SQ <= 10 || (LATE && NC + SQ <= 11);
  constexpr bool PF = PFX || PFD;
  raw xn[PFX ? NC : 1][VPL], dn[PFD ? SQ : 1][VPL];
  auto load_xd = [&](int64_t r, raw (&xs)[PFX ? NC : 1][VPL], raw (&ds)[PFD ? SQ : 1][VPL]) {
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      if constexpr (PFX) {
        #pragma unroll
        for (int i = 0; i < NC; ++i) xs[i][c] = ld_x(p.src[i], r, c);
      }
      if constexpr (PFD) {
        #pragma unroll
        for (int j = 0; j < SQ; ++j) ds[j][c] = ld_x(p.dh[j], r, c);
      }
    }
  };
  if constexpr (PF) load_xd(blockIdx.x < g.R ? (int64_t)blockIdx.x : 0, xn, dn);
  if constexpr (LATE) {
    // as many stores behind the first row's loads as every later row has
    // behind its prefetch (its gradients'), each to its own 16 bytes of the
    // sink so none is merged away: the wait for a row's data then counts the
    // same on the loop's entry and on its back edge, and leaves those stores
    // in flight
    static_assert(NC * VPL * 16 <= sizeof(g_store_sink), "one sink slot per store");
    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
    for (int k = 0; k < NC * VPL; ++k) st16_stream((gchar_t*)g_store_sink + 16 * k, make_uint4(0u, 0u, 0u, 0u));
  }

  int parity = 0;
  for (int64_t row = blockIdx.x; row < g.R; row += gridDim.x, parity ^= 1) {
    // every load of the row first: sources, upstream gradients (loaded
    // during the previous row with PF), and the source gradients this row
    // adds to (used after the reduction)
    raw x[NC][VPL], d[SQ][VPL];
    uint4 dv[NC][VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      #pragma unroll
      for (int i = 0; i < NC; ++i) x[i][c] = PFX ? xn[PFX ? i : 0][c] : ld_x(p.src[i], row, c);
      #pragma unroll
      for (int j = 0; j < SQ; ++j) d[j][c] = PFD ? dn[PFD ? j : 0][c] : ld_x(p.dh[j], row, c);
      if constexpr (!LATE) {
        #pragma unroll
        for (int i = 0; i < NC; ++i) {
          const u32x4_t v = __builtin_nontemporal_load(
              reinterpret_cast<const gu32x4_t*>(g_row(p.dV[i], row) + (uint32_t)vec[c] * 16u));
          dv[i][c] = make_uint4(v.x, v.y, v.z, v.w);
        }
      }
    }
    // lanes past the row's end read vector 0: a zero source there zeroes
    // every term those lanes add (scores, gradient dots, sums of squares, dq~)
    #pragma unroll
    for (int c = 0; c < VPL; ++c)
      #pragma unroll
      for (int i = 0; i < NC; ++i) {
        x[i][c].x = in_row[c] ? x[i][c].x : 0u;
        x[i][c].y = in_row[c] ? x[i][c].y : 0u;
      }
    // The sources and upstream gradients stay packed (bf16) and are unpacked
    // where they are used: the empty asm makes them look new to every query,
    // so the compiler does not keep their fp32 unpacking alive across queries.
    auto launder = [&]() {
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        #pragma unroll
        for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(x[i][c].x), "+v"(x[i][c].y));
        #pragma unroll
        for (int j = 0; j < SQ; ++j) asm volatile("" : "+v"(d[j][c].x), "+v"(d[j][c].y));
      }
    };
    // the row sums, one (query, source) pair at a time: each wave reduces
    // its lanes and writes its sums to LDS
    float* ws = wsum + (parity * g.W + wr) * NR;
    float xx[NC];
    #pragma unroll
    for (int i = 0; i < NC; ++i) xx[i] = 0.f;
    #pragma unroll
    for (int j = 0; j < SQ; ++j) {
      launder();
      // q~.x in fp32 (q~ is fp32); dh.x and x.x directly on the bf16 pairs
      // (v_dot2_f32_bf16: exact products, fp32 accumulation)
      float qf[VPL][4];
      #pragma unroll
      for (int c = 0; c < VPL; ++c) qload(j, c, qf[c]);
      #pragma unroll
      for (int i = 0; i < NC; ++i) {
        float a = 0.f, b = 0.f;
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          float xf[4];
          F::unpack(x[i][c], xf);
          #pragma unroll
          for (int e = 0; e < 4; ++e) a += qf[c][e] * xf[e];
          b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, x[i][c].x),
                                              __builtin_bit_cast(bf16x2v_t, d[j][c].x), b, false);
          b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, x[i][c].y),
                                              __builtin_bit_cast(bf16x2v_t, d[j][c].y), b, false);
          if (j == 0) {
            xx[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, x[i][c].x),
                                                    __builtin_bit_cast(bf16x2v_t, x[i][c].x), xx[i], false);
            xx[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, x[i][c].y),
                                                    __builtin_bit_cast(bf16x2v_t, x[i][c].y), xx[i], false);
          }
        }
        a = wave_sum(a);
        b = wave_sum(b);
        if (lane == 0) {
          ws[j * NC + i] = a;
          ws[(SQ + j) * NC + i] = b;
        }
      }
    }
    #pragma unroll
    for (int i = 0; i < NC; ++i) {
      const float v = wave_sum(xx[i]);
      if (lane == 0) ws[2 * SQ * NC + i] = v;
    }
    // one barrier per row: the sums alternate between two halves by row
    // parity, so a wave may write the next row's sums while another still
    // reads these
    __syncthreads();
    // each query's row scale and log-sum-exp gradient (uniform per query; 1
    // and 0 where none is given), loaded ahead of the loads issued next, so
    // waiting for them does not wait for those
    const int jl = lane >> 3, il = lane & 7;
    float gs = 1.f, dl = 0.f;
    #pragma unroll
    for (int j = 0; j < SQ; ++j) {
      const float gj = p.dh_scale[j] ? p.dh_scale[j][row] : 1.f;
      const float dj = p.dlse[j] ? p.dlse[j][row] : 0.f;
      gs = jl == j ? gj : gs;
      dl = jl == j ? dj : dl;
    }
    if constexpr (LATE) {
      #pragma unroll
      for (int c = 0; c < VPL; ++c)
        #pragma unroll
        for (int i = 0; i < NC; ++i) {
          const u32x4_t v = __builtin_nontemporal_load(
              reinterpret_cast<const gu32x4_t*>(g_row(p.dV[i], row) + (uint32_t)vec[c] * 16u));
          dv[i][c] = make_uint4(v.x, v.y, v.z, v.w);
        }
      __builtin_amdgcn_sched_barrier(0);  // the gradients' loads ahead of the next row's
    }
    if constexpr (PF) {
      // the next row's sources and upstream gradients (this row again at the
      // end: in bounds, unused)
      const int64_t nr = row + gridDim.x;
      load_xd(nr < g.R ? nr : row, xn, dn);
    }
    // The per-row coefficients, one (query, source) pair per lane: lane
    // 8 j + i takes query j and source i; the softmax over a query's sources
    // is a reduction over its 8-lane group. (Computed as uniform values they
    // would cost every lane the whole table.)
    const bool valid = jl < SQ && il < NC;
    float tq = 0.f, tg = 0.f, tv = 0.f;
    if (valid) {
      const float* w0 = wsum + parity * g.W * NR;
      for (int w = 0; w < g.W; ++w) {
        tq += w0[w * NR + jl * NC + il];
        tg += w0[w * NR + (SQ + jl) * NC + il];
        tv += w0[w * NR + 2 * SQ * NC + il];
      }
    }
    const float rl = rsqrtf(tv * g.invD + p.eps);
    const float sc = valid ? tq * rl : -FLT_MAX;
    const float mx = group8_max(sc);
    const float ex = valid ? __expf(sc - mx) : 0.f;
    const float al = ex * (1.0f / group8_sum(ex));
    const float gbar = group8_sum(al * (gs * tg));
    const float Al = al * gs;
    const float Bl = al * (gs * tg - gbar + dl) * rl;
    // cc_i = sum over queries of B sc r / D: the lanes 8 j + i
    float ccl = valid ? Bl * sc * rl * g.invD : 0.f;
    if constexpr (SQ > 1) ccl += __shfl_xor(ccl, 8);
    if constexpr (SQ > 2) ccl += __shfl_xor(ccl, 16);
    if constexpr (SQ > 4) ccl += __shfl_xor(ccl, 32);
    auto lane_val = [&](float v, int k) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
    };
    float cc[NC];
    #pragma unroll
    for (int i = 0; i < NC; ++i) cc[i] = lane_val(ccl, i);
    #pragma unroll
    for (int j = 0; j < SQ; ++j) {
      float A[NC], B[NC];
      #pragma unroll
      for (int i = 0; i < NC; ++i) {
        A[i] = lane_val(Al, 8 * j + i);
        B[i] = lane_val(Bl, 8 * j + i);
      }
      launder();
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float q[4], dh[4], dq[4] = {0.f, 0.f, 0.f, 0.f};
        qload(j, c, q);
        F::unpack(d[j][c], dh);
        #pragma unroll
        for (int i = 0; i < NC; ++i) {
          float xf[4];
          F::unpack(x[i][c], xf);
          float o[4] = {__uint_as_float(dv[i][c].x), __uint_as_float(dv[i][c].y), __uint_as_float(dv[i][c].z),
                        __uint_as_float(dv[i][c].w)};
          #pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] += A[i] * dh[e] + B[i] * q[e];
            dq[e] += B[i] * xf[e];
          }
          dv[i][c] = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                __float_as_uint(o[3]));
        }
        if constexpr (DQR) {
          #pragma unroll
          for (int e = 0; e < 4; ++e) dqr[DQR ? j : 0][c][e] += dq[e];
        } else if (in_row[c]) {
          float4* acc = reinterpret_cast<float4*>(dqs + j * g.D + vec[c] * 4);
          float4 a = *acc;
          a.x += dq[0]; a.y += dq[1]; a.z += dq[2]; a.w += dq[3];
          *acc = a;
        }
      }
    }
    launder();
    #pragma unroll
    for (int i = 0; i < NC; ++i)
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float xf[4];
        F::unpack(x[i][c], xf);
        float o[4] = {__uint_as_float(dv[i][c].x), __uint_as_float(dv[i][c].y), __uint_as_float(dv[i][c].z),
                      __uint_as_float(dv[i][c].w)};
        #pragma unroll
        for (int e = 0; e < 4; ++e) o[e] -= cc[i] * xf[e];
        // lanes past the row's end store to the sink (a branch here costs
        // the 8-query variants their registers)
        gchar_t* dst = g_row(p.dV[i], row) + (uint32_t)vec[c] * 16u;
        dst = in_row[c] ? dst : (gchar_t*)g_store_sink;
        st16_stream(dst, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                    __float_as_uint(o[3])));
      }
  }
  #pragma unroll
  for (int j = 0; j < SQ; ++j)
    #pragma unroll
    for (int c = 0; c < VPL; ++c)
      if (in_row[c]) {
        float* prow = p.partial + ((int64_t)j * gridDim.x + blockIdx.x) * g.D + vec[c] * 4;
        const float4 a = DQR ? make_float4(dqr[DQR ? j : 0][c][0], dqr[DQR ? j : 0][c][1], dqr[DQR ? j : 0][c][2],
                                           dqr[DQR ? j : 0][c][3])
                             : *reinterpret_cast<const float4*>(dqs + j * g.D + vec[c] * 4);
        st16(prow, make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                              __float_as_uint(a.w)));
      }
}

// Column sums of a [rows][D] fp32 matrix over consecutive row chunks, each in
// ascending row order: out[k][d] = sum of in[r][d] for r in chunk k. With
// FINISH the single chunk's sum t gives dw = t * gamma (t without a gain) and
// dgamma = t * w, written or added. One thread owns four columns.
// blockIdx.z selects one of several queries whose partial rows lie qin
// floats apart (their chunk sums qout apart; w, gamma, dw and dgamma rows D
// apart); bit q of acc_mask says whether query q adds to dw / dgamma.
template <bool FINISH>
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const float* __restrict__ in,
                                                         int64_t rows, int64_t D, int64_t chunk,
                                                         float* __restrict__ out,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ gm,
                                                         float* __restrict__ dw,
                                                         float* __restrict__ dgamma,
                                                         unsigned acc_mask, int64_t qin, int64_t qout) {
  const int64_t d = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (d >= D) return;
  const int q = blockIdx.z;
  in += q * qin;
  if (!FINISH) out += q * qout;
  if (FINISH) {
    if (w) w += q * D;
    if (gm) gm += q * D;
    dw += q * D;
    if (dgamma) dgamma += q * D;
  }
  const int accumulate = (acc_mask >> q) & 1u;
  const int64_t r0 = (int64_t)blockIdx.y * chunk;
  const int64_t r1 = r0 + chunk < rows ? r0 + chunk : rows;
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    const float4 a = ldf4(in + r * D + d), b = ldf4(in + (r + 1) * D + d);
    const float4 c = ldf4(in + (r + 2) * D + d), e = ldf4(in + (r + 3) * D + d);
    t.x += a.x; t.y += a.y; t.z += a.z; t.w += a.w;
    t.x += b.x; t.y += b.y; t.z += b.z; t.w += b.w;
    t.x += c.x; t.y += c.y; t.z += c.z; t.w += c.w;
    t.x += e.x; t.y += e.y; t.z += e.z; t.w += e.w;
  }
  for (; r < r1; ++r) {
    const float4 a = ldf4(in + r * D + d);
    t.x += a.x; t.y += a.y; t.z += a.z; t.w += a.w;
  }
  if (!FINISH) {
    *reinterpret_cast<float4*>(out + (int64_t)blockIdx.y * D + d) = t;
    return;
  }
  const float4 gv = gm ? ldf4(gm + d) : make_float4(1.f, 1.f, 1.f, 1.f);
  float4 o = make_float4(t.x * gv.x, t.y * gv.y, t.z * gv.z, t.w * gv.w);
  if (accumulate) {
    const float4 prev = ldf4(dw + d);
    o.x += prev.x; o.y += prev.y; o.z += prev.z; o.w += prev.w;
  }
  *reinterpret_cast<float4*>(dw + d) = o;
  if (dgamma) {
    const float4 wv = ldf4(w + d);
    float4 og = make_float4(t.x * wv.x, t.y * wv.y, t.z * wv.z, t.w * wv.w);
    if (accumulate) {
      const float4 prev = ldf4(dgamma + d);
      og.x += prev.x; og.y += prev.y; og.z += prev.z; og.w += prev.w;
    }
    *reinterpret_cast<float4*>(dgamma + d) = og;
  }
}

// ---------------------------------------------------------------------------
// Phase 1 streamed over any number of sources [K3 9.4 step 1; RH 4.2 Phase 1]:
// up to SQ queries stay in registers while the row's sources stream through in
// register groups of G. Each group's SQ x G scores come from one row
// reduction, and every query folds them into its own running (m, z,
// numerator) by the online-softmax merge (OS2), so each source is read once
// for all SQ queries whatever n is. Used where the matrix-core kernel does not
// apply: more than 8 sources, more than 8 queries, fp32 I/O, or other row
// widths. Loads are unconditional and stores branch-free (see the aggregate
// kernel).
//
// More than SQ queries run in passes of SQ. When the rows alone do not fill
// the grid (few rows, as in decode), the passes run side by side in one
// launch: workgroup b runs pass (b / 8) % passes for row walker
// b % 8 + 8 (b / (8 passes)). Consecutive workgroups go to the 8 XCDs in
// turn, so all passes of one walker sit on one XCD and walk the same rows at
// about the same time, and the later reads of a row's sources are served by
// that XCD's L2. Every pass of the launch forms a fused block close in
// registers; pass 0 stores it. With many rows the passes run as consecutive
// launches, which measured twice as fast at 131072 rows of 7168 as 6 side-by-
// side passes; launches after the first read the stored block sum.
// ---------------------------------------------------------------------------
struct Phase1SParams {
  const void* src[64];
  int n;
  int S;            // queries of the launch (all its passes)
  int passes;       // passes of the launch: ceil(S / SQ)
  int walkers;      // row walkers per pass (a multiple of 8)
  const float* Wq;  // [S][D]
  const float* G;   // [S][D] or null
  float eps;
  void* out;        // [S][R][D]
  float* m_out;     // [S][R] or null
  float* lse_out;   // [S][R]
  Close cl;         // close computing source n-1, or cl.v == null
  Geom g;
};

template <class T, int VPL, int G, int SQ, int PD>
__global__ __launch_bounds__(512) void phase1_stream_kernel(Phase1SParams p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  constexpr int NV = SQ * G + G;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  const bool has_close = p.cl.v != nullptr;
  const int rest = (int)(blockIdx.x >> 3);
  const int pass = rest % p.passes;
  const int64_t walker = (int64_t)(blockIdx.x & 7) + 8 * (int64_t)(rest / p.passes);
  const int s0 = pass * SQ;
  const int Sp = p.S - s0 < SQ ? p.S - s0 : SQ;  // queries of this pass

  float q[SQ][VPL][EPV];
  #pragma unroll
  for (int s = 0; s < SQ; ++s)
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      if (s < Sp && vec < g.V) {
        load_query<EPV>(p.Wq, p.G, (int64_t)(s0 + s) * g.D + (int64_t)vec * EPV, q[s][c]);
      } else {
        #pragma unroll
        for (int e = 0; e < EPV; ++e) q[s][c][e] = 0.f;
      }
    }

  // Byte offsets of this lane's vectors in row `grp`'s slot (row 0 past the
  // end, vector 0 past the row's end: loads stay in bounds and unconditional).
  bool in_row[VPL];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) in_row[c] = c * ln.stride + ln.t < g.V;
  auto row_off = [&](int64_t grp, int c) -> int64_t {
    const int64_t row = grp * g.RPW + ln.slot;
    const int64_t rr = (grp < g.groups && row < g.R) ? row : 0;
    return rr * rowbytes + (int64_t)(in_row[c] ? c * ln.stride + ln.t : 0) * 16;
  };
  // Raw vectors of sources i0 .. i0 + G - 1 of row `grp`; slots past n and
  // the closing source read the sink's first 16 bytes.
  auto issue = [&](int64_t grp, int i0, uint4 (&u)[G][VPL]) {
    #pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = i0 + j;
      const bool live = i < p.n && !(has_close && i == p.n - 1);
      const char* sp = static_cast<const char*>(p.src[live ? i : 0]);
      #pragma unroll
      for (int c = 0; c < VPL; ++c)
        u[j][c] = ld16_stream(live ? sp + row_off(grp, c) : reinterpret_cast<const char*>(g_store_sink));
    }
  };

  // The next PD groups' loads are in flight while a group reduces. Groups are
  // taken in one sequence over this workgroup's rows (row k's groups, then
  // row k + 1's): flat index f is group f % gpr of the workgroup's row f / gpr.
  const int gpr = (p.n + G - 1) / G;
  auto issue_flat = [&](int64_t f, uint4 (&u)[G][VPL]) {
    const int64_t k = f / gpr;
    issue(walker + k * p.walkers, (int)(f - k * gpr) * G, u);
  };
  uint4 ring[PD][G][VPL];
  #pragma unroll
  for (int d = 0; d < PD; ++d) issue_flat(d, ring[d]);
  int64_t f_next = PD;
  for (int64_t grp = walker; grp < g.groups; grp += p.walkers) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    // the closing source b = round(p + v) (or v), formed and stored first
    uint4 bcl[VPL];
    if (has_close) {
      const char* pp = static_cast<const char*>(p.cl.p ? p.cl.p : p.cl.v);
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int64_t off = row_off(grp, c);
        const uint4 v = ld16_stream(static_cast<const char*>(p.cl.v) + off);
        const uint4 a = ld16_stream(pp + off);
        float fa[EPV], fv[EPV];
        T::unpack(a, fa);
        T::unpack(v, fv);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) fa[e] = p.cl.p ? fa[e] + fv[e] : fv[e];
        bcl[c] = T::pack(fa);
        st16_stream(store_target(rv && in_row[c] && pass == 0, static_cast<char*>(p.cl.b) + off), bcl[c]);
      }
    }

    float m_run[SQ], z_run[SQ], num[SQ][VPL][EPV];
    #pragma unroll
    for (int s = 0; s < SQ; ++s) {
      m_run[s] = -FLT_MAX;
      z_run[s] = 0.f;
      #pragma unroll
      for (int c = 0; c < VPL; ++c)
        #pragma unroll
        for (int e = 0; e < EPV; ++e) num[s][c][e] = 0.f;
    }
    for (int i0 = 0; i0 < p.n; i0 += G) {
      uint4 u[G][VPL];
      #pragma unroll
      for (int j = 0; j < G; ++j)
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          u[j][c] = ring[0][j][c];
          #pragma unroll
          for (int d = 0; d + 1 < PD; ++d) ring[d][j][c] = ring[d + 1][j][c];
        }
      issue_flat(f_next++, ring[PD - 1]);
      float x[G][VPL][EPV];
      #pragma unroll
      for (int j = 0; j < G; ++j) {
        const int i = i0 + j;
        const bool closing = has_close && i == p.n - 1;
        #pragma unroll
        for (int c = 0; c < VPL; ++c) {
          T::unpack(closing ? bcl[c] : u[j][c], x[j][c]);
          const bool keep = i < p.n && in_row[c];
          #pragma unroll
          for (int e = 0; e < EPV; ++e) x[j][c][e] = keep ? x[j][c][e] : 0.f;
        }
      }
      float red[NV];
      #pragma unroll
      for (int k = 0; k < NV; ++k) red[k] = 0.f;
      #pragma unroll
      for (int j = 0; j < G; ++j)
        #pragma unroll
        for (int c = 0; c < VPL; ++c)
          #pragma unroll
          for (int e = 0; e < EPV; ++e) {
            red[SQ * G + j] += x[j][c][e] * x[j][c][e];
            #pragma unroll
            for (int s = 0; s < SQ; ++s) red[s * G + j] += q[s][c][e] * x[j][c][e];
          }
      row_reduce<NV>(red, lds, ln.slot, ln.wr, g.W);
      float ri[G];
      #pragma unroll
      for (int j = 0; j < G; ++j) ri[j] = rsqrtf(red[SQ * G + j] * g.invD + p.eps);
      #pragma unroll
      for (int s = 0; s < SQ; ++s) {
        float sc[G];
        float m_new = m_run[s];
        #pragma unroll
        for (int j = 0; j < G; ++j) {
          sc[j] = red[s * G + j] * ri[j];
          if (i0 + j < p.n) m_new = fmaxf(m_new, sc[j]);
        }
        const float rescale = __expf(m_run[s] - m_new);
        z_run[s] *= rescale;
        #pragma unroll
        for (int j = 0; j < G; ++j) {
          sc[j] = (i0 + j < p.n) ? __expf(sc[j] - m_new) : 0.f;
          z_run[s] += sc[j];
        }
        #pragma unroll
        for (int c = 0; c < VPL; ++c)
          #pragma unroll
          for (int e = 0; e < EPV; ++e) {
            float a = num[s][c][e] * rescale;
            #pragma unroll
            for (int j = 0; j < G; ++j) a += sc[j] * x[j][c][e];
            num[s][c][e] = a;
          }
        m_run[s] = m_new;
      }
    }
    #pragma unroll
    for (int s = 0; s < SQ; ++s) {
      if (s >= Sp) continue;
      const float rz = 1.0f / z_run[s];
      char* orow = static_cast<char*>(p.out) + (int64_t)(s0 + s) * g.R * rowbytes;
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float o[EPV];
        #pragma unroll
        for (int e = 0; e < EPV; ++e) o[e] = num[s][c][e] * rz;
        st16(store_target(rv && in_row[c], orow + row_off(grp, c)), T::pack(o));
      }
      if (rv && ln.t == 0) {
        if (p.m_out) p.m_out[(int64_t)(s0 + s) * g.R + row] = m_run[s];
        p.lse_out[(int64_t)(s0 + s) * g.R + row] = m_run[s] + __logf(z_run[s]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 1 for many queries over wide rows [K3 9.4 step 1; RH 4.2 Phase 1],
// bf16, n <= 16 sources, up to 32 queries, in two passes over the sources:
//
// Scores. For a tile of rows, the scores of every query against every source
// of every row form one product C = Qp B, where Qp is [32 MT, D]: row
// 4 q + j holds part j of query q (parts: the exact three-way bf16 split of
// the fp32 query, row j = 3 zero), and B is [D, rows x 8]: column 8 r + i is
// source i of row r. It runs on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation): each wave owns 16 columns and all 2 MT 16-row tiles
// of Qp (4 queries each). Both operands pass through LDS in steps of 64
// hidden elements (see phase1_gemm_scores_kernel). In k-step ks of a step,
// k-group g of a lane holds elements 32 ks + 8 g .. 32 ks + 8 g + 7 (A and B
// alike). Sums of squares come from the same B registers (v_dot2). After the
// last step each lane holds,
// for its column, the three parts of one query per tile; their sum scaled by
// the source's 1 / rms is the score. A row takes NPR columns, the smallest of
// 1, 2, 4, 8 or 16 that holds its n sources (so a tile holds 16 / NPR rows
// per wave), and the softmax is an NPR-lane reduction. The weights alpha
// [S][R][AST] (AST = 8, or 16 for n > 8; entries i < NPR, zero from n on)
// and the statistics m, lse are written.
//
// Outputs. o_s = sum_i alpha[s][i] b_i, one row per wave group: the row's n
// sources stay in registers and every query's output is formed from them
// (as fp32 for n <= 8; packed, one vector per lane, for n > 8).
//
// Together the passes move (2 n + S) D-vectors per row where query passes of
// 4 in registers would move (passes x n + S). A block close runs before them
// as a launch of its own.
// ---------------------------------------------------------------------------
constexpr int kGWaves = 16;   // waves per scores workgroup, 16 source columns each
constexpr int kGChunk = 128;  // rows are a whole number of 2 x 128 elements

struct QSplitParams {
  const float* W;  // [S][D]
  const float* G;  // [S][D] or null
  int S, MT;
  int64_t D;
  __bf16* qp;      // [32 MT][D]
};

__global__ void qsplit_kernel(QSplitParams p) {
  const int64_t total = (int64_t)p.MT * 32 * p.D;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / p.D, d = idx - m * p.D;
    const int s = 8 * (int)(m >> 5) + (int)((m & 31) >> 2), j = (int)(m & 3);
    float part = 0.f;
    if (s < p.S && j < 3) {
      const int64_t off = (int64_t)s * p.D + d;
      const float q = p.G ? p.W[off] * p.G[off] : p.W[off];
      const float h1 = bf16_round(q);
      const float r1 = q - h1;  // exact
      const float h2 = bf16_round(r1);
      part = j == 0 ? h1 : j == 1 ? h2 : r1 - h2;  // r1 - h2 is exact and a bf16 value
    }
    p.qp[idx] = (__bf16)part;
  }
}

struct P1GParams {
  const void* src[16];
  int n;
  int S;
  const __bf16* qp;  // [32 MT][D]
  float eps;
  float invD;
  int64_t R;
  int D;
  float* alpha;      // [S][R][AST], AST = 8 (NPR <= 8) or 16
  float* m_out;      // [S][R] or null
  float* lse_out;    // [S][R]
};

// The scores pass stages its operands in LDS. A step is 64 hidden elements:
// 128 bytes of each of a wave's 16 source columns and of each of the 32 MT Qp
// rows. Both are copied with global_load_lds_dwordx4, 16 bytes per lane, so
// that one instruction moves whole 128-byte lines (eight of them per KiB):
// loading the sources straight into the matrix-core operand layout left each
// load touching 16 half-lines, and the address unit then stalled on the L1.
// A copy lane fetches piece s ^ f(r) of its row r (f(r) = (r >> 1) & 7) into
// slot s, so the operand reads (16 lanes, one per row, the same piece) meet 16
// different bank groups.
constexpr int kGStep = 64;  // hidden elements per step
#ifndef ATTNRES_GEMM_RING
#define ATTNRES_GEMM_RING 4
#endif
// source steps per wave in LDS (kGRing - 1 copies in flight); 16 waves x 4 x
// 2 KiB plus the Qp buffers of 4 tiles is the 160 KiB of a CU
constexpr int kGRing = ATTNRES_GEMM_RING;

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

// 16 bytes per lane from a per-lane global address into LDS at
// lds + 16 * lane; `nt` marks a stream read once. Issued as inline assembly,
// so the compiler adds no waits for it: the kernel counts its own copies
// (p1_wait). M0 is written here and nowhere else in the kernel.
template <bool NTC>
__device__ __forceinline__ void dma16_lane(const char* g, uint32_t lds) {
  if constexpr (NTC)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory");
}

template <int MT, int NPR>
__global__ __launch_bounds__(1024) void phase1_gemm_scores_kernel(P1GParams p) {
  constexpr int RW = 16 / NPR;          // rows per wave: NPR source columns each
  constexpr int RT = kGWaves * RW;      // rows per tile
  constexpr int AST = NPR > 8 ? 16 : 8; // row stride of the weights
  constexpr int AB = MT * 32 * 128;     // bytes of one Qp step
  __shared__ __attribute__((aligned(16))) char abuf[2][AB];
  __shared__ __attribute__((aligned(16))) char bbuf[kGWaves][kGRing][16 * 128];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, g4 = l >> 4;        // B column and k-group
  const int rl = col / NPR, i = col % NPR;    // row of the wave's RW, source
  const int64_t rowbytes = (int64_t)p.D * 2;
  const int nsteps = p.D / kGStep;
  const int64_t tiles = (p.R + RT - 1) / RT;
  // this workgroup's tiles blockIdx.x, blockIdx.x + gridDim.x, ...: their
  // steps form one sequence k = tile step * nsteps + step
  const int64_t my_tiles = blockIdx.x < tiles ? (tiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int64_t steps = my_tiles * nsteps;
  const int aw = w < 4 * MT ? 1 : 0;  // waves 0 .. 4 MT - 1 copy 8 Qp rows each per step

  // Copy lanes. Sources: instruction m (0, 1) of a step moves columns
  // 8 m .. 8 m + 7 of the wave, 8 lanes (one line) per column; a column past
  // n reads source 0 and a row past R reads row 0 (both discarded).
  const int cs = l & 7;
  const char* bsrc[2];
  int brl[2];
  #pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int c = 8 * m + (l >> 3);
    const int ic = c % NPR;
    brl[m] = c / NPR;
    bsrc[m] = static_cast<const char*>(p.src[ic < p.n ? ic : 0]) + 16 * (cs ^ gswz(c));
  }
  auto bcopy = [&](int64_t k) {
    const int64_t tj = k / nsteps;
    const int st = (int)(k - tj * nsteps);
    const int64_t tile = blockIdx.x + tj * gridDim.x;
    const uint32_t dst = lds_offset(&bbuf[w][(int)(k % kGRing)][0]);
    #pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int64_t r = tile * RT + w * RW + brl[m];
      dma16_lane<true>(bsrc[m] + (r < p.R ? r : 0) * rowbytes + (int64_t)st * 128, dst + 1024u * m);
    }
  };
  // Qp: rows 8 w .. 8 w + 7 (the same for every tile, so cached)
  const int ar = 8 * (aw ? w : 0) + (l >> 3);
  const char* asrc = reinterpret_cast<const char*>(p.qp) + (int64_t)ar * rowbytes + 16 * (cs ^ gswz(ar));
  auto acopy = [&](int64_t k) {
    if (aw) dma16_lane<false>(asrc + (int64_t)(k % nsteps) * 128, lds_offset(&abuf[(int)(k & 1)][w * 1024]));
  };

  // Order of a wave's copies (2 instructions per B step, aw per A step):
  // A(0), B(0) .. B(P - 1), then per step k: A(k+1), B(k+P), with P =
  // kGRing - 1. Step k needs B(k), after which at least 2 P + aw copies were
  // issued (2 P + aw at k = 0, up to 2 P + P aw later: waiting for fewer is
  // only stricter); its barrier needs A(k+1), after which come the 2 copies
  // of B(k+P) (and, at a tile's end, the weight stores).
  constexpr int P = kGRing - 1;
  acopy(0);
  #pragma unroll
  for (int j = 0; j < P; ++j) bcopy(j);
  p1_wait(2 * P);
  lds_barrier();

  f32x4_t acc[2 * MT];
  #pragma unroll
  for (int t = 0; t < 2 * MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ss0 = 0.f, ss1 = 0.f;
  int st = 0;  // step within the current tile
  int64_t tile = blockIdx.x;
  const int sw = gswz(col);  // the swizzle of this lane's operand row (A: 16 t + col; B: col)

  for (int64_t k = 0; k < steps; ++k) {
    acopy(k + 1);
    bcopy(k + P);
    p1_wait(2 * P + aw);
    asm volatile("" ::: "memory");  // the LDS reads below stay after the wait
    const char* bb = &bbuf[w][(int)(k % kGRing)][col * 128];
    const char* ab = &abuf[(int)(k & 1)][col * 128];
    #pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int slot = 16 * ((4 * ks + g4) ^ sw);
      const uint4 b = *reinterpret_cast<const uint4*>(bb + slot);
      float& ss = ks ? ss1 : ss0;
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.x), __builtin_bit_cast(bf16x2v_t, b.x),
                                           ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.y), __builtin_bit_cast(bf16x2v_t, b.y),
                                           ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.z), __builtin_bit_cast(bf16x2v_t, b.z),
                                           ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, b.w), __builtin_bit_cast(bf16x2v_t, b.w),
                                           ss, false);
      #pragma unroll
      for (int t = 0; t < 2 * MT; ++t) {
        const uint4 a = *reinterpret_cast<const uint4*>(ab + t * 16 * 128 + slot);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x8_t, b), acc[t], 0, 0, 0);
      }
    }
    if (++st == nsteps) {
      // scores, softmax over the row's NPR lanes, weights and statistics
      st = 0;
      const int64_t row = tile * RT + w * RW + rl;
      const bool rv = row < p.R;
      float ss = ss0 + ss1;
      ss += __shfl_xor(ss, 16);  // the four k-groups of this column
      ss += __shfl_xor(ss, 32);
      const float inv = rsqrtf(ss * p.invD + p.eps);
      const bool valid = i < p.n;
      #pragma unroll
      for (int t = 0; t < 2 * MT; ++t) {
        // accumulators 0..2 of k-group g4: parts 0..2 of query 4 t + g4
        const int s = 4 * t + g4;
        const float sc = ((acc[t][0] + acc[t][1]) + acc[t][2]) * inv;
        const float m = groupn_max<NPR>(valid ? sc : -INFINITY);
        const float e = valid ? __expf(sc - m) : 0.f;
        const float z = groupn_sum<NPR>(e);
        if (rv && s < p.S) {
          p.alpha[((int64_t)s * p.R + row) * AST + i] = e * (1.0f / z);
          if (i == 0) {
            if (p.m_out) p.m_out[(int64_t)s * p.R + row] = m;
            p.lse_out[(int64_t)s * p.R + row] = m + __logf(z);
          }
        }
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      ss0 = 0.f;
      ss1 = 0.f;
      tile += gridDim.x;
    }
    p1_wait(2);
    lds_barrier();  // A(k+1) is in LDS; every read of A(k) and B(k) is done
  }
  p1_wait(0);  // no copy may still be landing in LDS when the workgroup ends
}

struct P1OParams {
  const void* src[16];
  int S;
  const float* alpha;  // [S][R][8] (n <= 8) or [S][R][16]
  void* out;           // [S][R][D]
  Geom g;
};

template <int NC, bool NT>
__global__ __launch_bounds__(512) void phase1_gemm_outputs_kernel(P1OParams p) {
  constexpr int VPL = 2;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    // one row per wave group: uniform across the wave, so the weights are
    // scalar loads
    const int64_t row = __builtin_amdgcn_readfirstlane((int)(grp * g.RPW + ln.slot));
    const bool rv = row < g.R;
    const int64_t base = (rv ? row : 0) * rowbytes;
    float x[NC][VPL][8];
    bool own[VPL];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      own[c] = rv && vec < g.V;
      const int64_t off = base + (int64_t)(vec < g.V ? vec : 0) * 16;
      #pragma unroll
      for (int i = 0; i < NC; ++i) Bf16::unpack(ld16_stream(static_cast<const char*>(p.src[i]) + off), x[i][c]);
    }
    const float* arow = p.alpha + (rv ? row : 0) * 8;
    for (int s = 0; s < p.S; ++s) {
      const float4 a0 = *reinterpret_cast<const float4*>(arow + (int64_t)s * g.R * 8);
      const float4 a1 = *reinterpret_cast<const float4*>(arow + (int64_t)s * g.R * 8 + 4);
      const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      char* orow = static_cast<char*>(p.out) + (int64_t)s * g.R * rowbytes + base;
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        float o[8];
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          float acc = a[0] * x[0][c][e];
          #pragma unroll
          for (int i = 1; i < NC; ++i) acc = fmaf(a[i], x[i][c][e], acc);
          o[e] = acc;
        }
        char* dst = store_target(own[c], orow + (int64_t)(c * ln.stride + ln.t) * 16);
        if constexpr (NT) st16_stream(dst, Bf16::pack(o));
        else st16(dst, Bf16::pack(o));
      }
    }
  }
}

// The outputs pass for 9..16 sources: the row's sources stay packed in
// registers, one 16-byte vector per lane (up to 16 waves per row, so rows of
// up to 8192 elements); kept as fp32 they would not fit beside the
// accumulators. Queries go in pairs, so each source is unpacked once per
// pair: the pair's 32 weights are one load (lane 16 q + i holds weight i of
// query q; the weights are [S][R][16]) and reach the products as scalars.
// Each output sums its terms in source order, as the narrower pass does.
template <int NC, bool NT>
__global__ __launch_bounds__(1024) void phase1_gemm_outputs_wide_kernel(P1OParams p) {
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    // one row per wave group: uniform across the wave
    const int64_t row = __builtin_amdgcn_readfirstlane((int)(grp * g.RPW + ln.slot));
    const bool rv = row < g.R;
    const int64_t base = (rv ? row : 0) * rowbytes;
    const int vec = ln.t;
    const bool own = rv && vec < g.V;
    // each source row as a wave-uniform base plus a 32-bit lane offset, so
    // no 64-bit address per lane and source is kept
    const uint32_t loff = (uint32_t)(vec < g.V ? vec : 0) * 16u;
    u32x4_t x[NC];
    #pragma unroll
    for (int i = 0; i < NC; ++i) {
      const gchar_t* b = uniform_ptr(static_cast<const char*>(p.src[i]) + base);
      x[i] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4_t*>(b + loff));
    }
    char* dst0 = static_cast<char*>(p.out) + base + (int64_t)vec * 16;
    for (int s0 = 0; s0 < p.S; s0 += 2) {
      // the empty asm makes the packed sources look new to every pair, so
      // their unpacking is not hoisted out of this loop as NC x 8 floats
      #pragma unroll
      for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(x[i]));
      const int sq = s0 + (ln.lane >> 4);
      const float wv = (ln.lane < 32 && sq < p.S)
                           ? p.alpha[((int64_t)sq * g.R + (rv ? row : 0)) * 16 + (ln.lane & 15)]
                           : 0.f;
      float o0[8], o1[8];
      #pragma unroll
      for (int i = 0; i < NC; ++i) {
        float f[8];
        Bf16::unpack(uint4{x[i][0], x[i][1], x[i][2], x[i][3]}, f);
        const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), i));
        const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), 16 + i));
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          o0[e] = i == 0 ? a0 * f[e] : fmaf(a0, f[e], o0[e]);
          o1[e] = i == 0 ? a1 * f[e] : fmaf(a1, f[e], o1[e]);
        }
        // one source at a time: otherwise the scheduler unpacks them all
        // up front and runs out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
      char* dst = store_target(own, dst0 + (int64_t)s0 * g.R * rowbytes);
      if constexpr (NT) st16_stream(dst, Bf16::pack(o0));
      else st16(dst, Bf16::pack(o0));
      // unconditional (a missing second query stores to the sink): under a
      // branch the compiler would sink o1's products into it and keep every
      // unpacked source alive until then
      dst = store_target(own && s0 + 1 < p.S, dst0 + (int64_t)(s0 + 1) * g.R * rowbytes);
      if constexpr (NT) st16_stream(dst, Bf16::pack(o1));
      else st16(dst, Bf16::pack(o1));
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 2 (one intra-block merge step) [K3 9.4 step 2, OS2, single-source
// triple; RH 4.2 Phase 2]: p = p_prev + v_prev rounded to the I/O dtype (or
// p = v_prev on the first merge), the score of the rounded p, then
// h = (e^(lse-M) o + e^(s_p-M) p) / (e^(lse-M) + e^(s_p-M)). The o tile is
// loaded before the row reduction so its latency overlaps the reduction. The
// inputs are streamed (non-temporal loads); p and h are written with plain
// stores: both are read again soon (p by the next merge, h by the sublayer)
// and are rewritten in place every sublayer, so keeping them cacheable lets
// the last-level cache serve them (about 8% faster than non-temporal stores).
// Tensors far larger than that cache (NT: a row-set of more than
// ATTNRES_PHASE2_NT_BYTES) are written non-temporally like every other stream.
// ---------------------------------------------------------------------------
struct Phase2Params {
  const void* o;
  const float* lse;
  const float* w;
  const float* gm;
  float eps;
  const void* p_prev;  // null on the first merge of a block
  const void* v_prev;
  void* p_out;         // null iff p_prev is null
  void* h_out;         // may be null when hn_out is set
  const float* gf;     // [D] gain of the output norm, or null (ones)
  float eps_f;
  void* hn_out;        // RMSNorm(h) * gf, or null (no output norm)
  const void* xs;      // a completed source merged as one more single-source term, or null
  Geom g;
};

template <bool NT>
__device__ __forceinline__ void st16_out(char* p, const uint4& v) {
  if constexpr (NT) st16_stream(p, v);
  else st16(p, v);
}

#ifndef ATTNRES_PHASE2_MAX_WAVES
#define ATTNRES_PHASE2_MAX_WAVES 8  // waves per row in Phase 2 (more vectors per lane beyond)
#endif
#ifndef ATTNRES_PHASE2_LB
#define ATTNRES_PHASE2_LB 512  // launch bound of the Phase-2 kernel (64 * max waves per workgroup)
#endif

template <class T, int VPL, bool HAS_PREV, bool NORM, bool NT, bool EXTRA = false>
__global__ __launch_bounds__(ATTNRES_PHASE2_LB) void phase2_kernel(Phase2Params p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  const Geom& g = p.g;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;

  // this sublayer's folded query (and the output norm's gain), resident for
  // every row; zero past the row's end
  float q[VPL][EPV], gn[NORM ? VPL : 1][EPV];
  #pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int vec = c * ln.stride + ln.t;
    if (vec < g.V) {
      load_query<EPV>(p.w, p.gm, (int64_t)vec * EPV, q[c]);
      if (NORM) load_gain<EPV>(p.gf, (int64_t)vec * EPV, gn[c]);
    } else {
      #pragma unroll
      for (int e = 0; e < EPV; ++e) {
        q[c][e] = 0.f;
        if (NORM) gn[c][e] = 0.f;
      }
    }
  }

  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    const int64_t base = (rv ? row : 0) * rowbytes;
    // every load of the row is issued first and unconditionally (a row past
    // the end reads row 0, a lane past the row's end reads vector 0; both are
    // discarded), so no branch hides a load from the compiler's wait counting
    // and one wait covers them all
    uint4 vv[VPL], pp[VPL], ov[VPL], xv[EXTRA ? VPL : 1];
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      const int64_t off = base + (int64_t)(vec < g.V ? vec : 0) * 16;
      vv[c] = ld16_stream(static_cast<const char*>(p.v_prev) + off);
      if (HAS_PREV) pp[c] = ld16_stream(static_cast<const char*>(p.p_prev) + off);
      ov[c] = ld16_stream(static_cast<const char*>(p.o) + off);
      if (EXTRA) xv[c] = ld16_stream(static_cast<const char*>(p.xs) + off);
    }
    const float l = p.lse[rv ? row : 0];

    uint4 pv[VPL];
    // q~.p and p.p, then (with the extra source) q~.x and x.x
    float red[EXTRA ? 4 : 2];
    #pragma unroll
    for (int k = 0; k < (EXTRA ? 4 : 2); ++k) red[k] = 0.f;
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      const bool ok = rv && vec < g.V;
      if (HAS_PREV) {
        float fa[EPV], fv[EPV];
        T::unpack(pp[c], fa);
        T::unpack(vv[c], fv);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) fa[e] += fv[e];
        pv[c] = T::pack(fa);  // the partial, rounded to the I/O dtype
        st16_out<NT>(store_target(ok, static_cast<char*>(p.p_out) + base + (int64_t)vec * 16), pv[c]);
      } else {
        pv[c] = vv[c];
      }
      const bool in_row = vec < g.V;
      float f[EPV];
      T::unpack(pv[c], f);
      #pragma unroll
      for (int e = 0; e < EPV; ++e) {
        f[e] = in_row ? f[e] : 0.f;
        red[0] += q[c][e] * f[e];
        red[1] += f[e] * f[e];
      }
      if constexpr (EXTRA) {
        T::unpack(xv[c], f);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) {
          f[e] = in_row ? f[e] : 0.f;
          red[2] += q[c][e] * f[e];
          red[3] += f[e] * f[e];
        }
      }
    }
    row_reduce<EXTRA ? 4 : 2>(red, lds, ln.slot, ln.wr, g.W);
    const float sp = red[0] * rsqrtf(red[1] * g.invD + p.eps);
    // the extra source's score (a completed source the Phase-1 group did not
    // include): OS2 over three terms, the group, the source and the partial
    const float sx = EXTRA ? red[2] * rsqrtf(red[3] * g.invD + p.eps) : -FLT_MAX;
    const float M = fmaxf(fmaxf(l, sp), sx);
    float a = __expf(l - M), b = __expf(sp - M), cx = EXTRA ? __expf(sx - M) : 0.f;
    const float r = 1.0f / (a + b + cx);
    a *= r;
    b *= r;
    cx *= r;
    uint4 hv[VPL];
    float hss[1] = {0.f};
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      float fo[EPV], fp[EPV];
      T::unpack(ov[c], fo);
      T::unpack(pv[c], fp);
      #pragma unroll
      for (int e = 0; e < EPV; ++e) fo[e] = a * fo[e] + b * fp[e];
      if constexpr (EXTRA) {
        T::unpack(xv[c], fp);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) fo[e] += cx * fp[e];
      }
      hv[c] = T::pack(fo);  // h rounded to the I/O dtype
      if (p.h_out)
        st16_out<NT>(store_target(rv && vec < g.V, static_cast<char*>(p.h_out) + base + (int64_t)vec * 16),
                     hv[c]);
      if (NORM && vec < g.V) {
        T::unpack(hv[c], fo);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) hss[0] += fo[e] * fo[e];
      }
    }
    if constexpr (NORM) {
      // the sublayer's input norm on the rounded h: RMSNorm(h) * gf
      row_reduce<1>(hss, lds, ln.slot, ln.wr, g.W);
      const float inv = rsqrtf(hss[0] * g.invD + p.eps_f);
      #pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int vec = c * ln.stride + ln.t;
        float f[EPV];
        T::unpack(hv[c], f);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) f[e] = gn[c][e] * (f[e] * inv);
        st16_out<NT>(store_target(rv && vec < g.V, static_cast<char*>(p.hn_out) + base + (int64_t)vec * 16),
                     T::pack(f));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm of a token tensor, the input norm of the sublayer that consumes an
// aggregate [ZZ block listing: attn(attn_norm(h)), mlp(mlp_norm(h)); WC
// reference: eps inside the root, mean over the hidden axis]:
// out = x / sqrt(mean_d x^2 + eps) * gamma, rounded to the I/O dtype. x and
// out may be the same buffer (each lane reads its vectors before the row's
// reduction and writes them after it).
// ---------------------------------------------------------------------------
struct NormParams {
  const void* x;
  const float* g;  // [D] or null (ones)
  float eps;
  void* out;
  Geom geo;
};

template <class T, int VPL>
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormParams p) {
  extern __shared__ float lds[];
  constexpr int EPV = T::kEPV;
  const Geom& g = p.geo;
  const Lanes ln(g.W);
  const int64_t rowbytes = (int64_t)g.V * 16;
  for (int64_t grp = blockIdx.x; grp < g.groups; grp += gridDim.x) {
    const int64_t row = grp * g.RPW + ln.slot;
    const bool rv = row < g.R;
    const int64_t base = row * rowbytes;
    uint4 xv[VPL];
    float ss[1] = {0.f};
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      const bool ok = rv && vec < g.V;
      xv[c] = ok ? ld16_stream(static_cast<const char*>(p.x) + base + (int64_t)vec * 16) : make_uint4(0, 0, 0, 0);
      float f[EPV];
      T::unpack(xv[c], f);
      #pragma unroll
      for (int e = 0; e < EPV; ++e) ss[0] += f[e] * f[e];
    }
    row_reduce<1>(ss, lds, ln.slot, ln.wr, g.W);
    const float inv = rsqrtf(ss[0] * g.invD + p.eps);
    #pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vec = c * ln.stride + ln.t;
      if (rv && vec < g.V) {
        float f[EPV], gn[EPV];
        T::unpack(xv[c], f);
        load_gain<EPV>(p.g, (int64_t)vec * EPV, gn);
        #pragma unroll
        for (int e = 0; e < EPV; ++e) f[e] = gn[e] * (f[e] * inv);
        st16(static_cast<char*>(p.out) + base + (int64_t)vec * 16, T::pack(f));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stand-alone block close [K3 9.3 listing]: b = p + v rounded to the I/O
// dtype, or b = v when p is null. Elementwise over `nvec` vectors.
// ---------------------------------------------------------------------------
template <class T>
__global__ void close_kernel(const void* __restrict__ pp, const void* __restrict__ vv,
                             void* __restrict__ b, int64_t nvec) {
  constexpr int EPV = T::kEPV;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint4 v = ld16_stream(static_cast<const char*>(vv) + i * 16);
    if (pp) {
      uint4 a = ld16_stream(static_cast<const char*>(pp) + i * 16);
      float fa[EPV], fv[EPV];
      T::unpack(a, fa);
      T::unpack(v, fv);
      #pragma unroll
      for (int e = 0; e < EPV; ++e) fa[e] += fv[e];
      v = T::pack(fa);
    }
    st16_stream(static_cast<char*>(b) + i * 16, v);
  }
}

// A block's partial sums in one pass [K3 9.3 listing: p grows by each
// sublayer output, rounded to the I/O dtype after every add]: from
// in[0] = p_1 and the later outputs in[1..n-1], out[t] = p_{t+1} =
// round(p_t + in[t]) for t = 1..n-1, the same adds and roundings as a chain
// of block closes, with each partial read from registers instead of memory.
// Inputs are loaded eight at a time and unconditionally (an index past n
// reads the last input again and is discarded).
struct PartialsParams {
  const void* in[kPartialsMax];
  void* out[kPartialsMax];  // out[0] unused
  int n;
  int64_t nvec;  // 16-byte vectors per tensor
};

template <class T>
__global__ void partials_kernel(PartialsParams p) {
  constexpr int EPV = T::kEPV;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t off = i * 16;
    float fa[EPV];
    T::unpack(ld16_stream(static_cast<const char*>(p.in[0]) + off), fa);
    for (int t0 = 1; t0 < p.n; t0 += 8) {
      uint4 x[8];
      #pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = t0 + u < p.n ? t0 + u : p.n - 1;
        x[u] = ld16_stream(static_cast<const char*>(p.in[t]) + off);
      }
      #pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t0 + u < p.n) {  // uniform across the grid
          float fv[EPV];
          T::unpack(x[u], fv);
          #pragma unroll
          for (int e = 0; e < EPV; ++e) fa[e] += fv[e];
          const uint4 v = T::pack(fa);  // the partial, rounded to the I/O dtype
          T::unpack(v, fa);
          st16_stream(static_cast<char*>(p.out[t0 + u]) + off, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from api.hip).
// ---------------------------------------------------------------------------

#ifndef ATTNRES_PHASE2_NT_BYTES
// [R, D] tensors larger than this are written non-temporally by Phase 2 and
// by the Phase-1 outputs pass
#define ATTNRES_PHASE2_NT_BYTES (1024.0 * 1024.0 * 1024.0)
#endif

#ifndef ATTNRES_PHASE2_VPL
#define ATTNRES_PHASE2_VPL 2  // preferred vectors per lane in Phase 2 (rows take up to 8 waves)
#endif
#ifndef ATTNRES_PHASE2_VPL_WIDE
// Vectors per lane of the merges that do less memory work per row reduction
// (the fused norm's second reduction; a block's first merge, which reads no
// partial), over at least ATTNRES_PHASE2_WIDE_ROWS rows whose vectors fill
// whole waves at this width: fewer waves per row cost less per reduction.
// At config 3's shape (4 vectors per lane, 2 waves per row) the normed merge
// went 106.6 -> 98.5 us and the first merge 68 -> 62 us, while the merge with
// a partial is fastest at 2; with few rows (decode, 128) the merge is a
// latency chain and 4 vectors per lane took it from 4.7 to 5.2 us.
#define ATTNRES_PHASE2_VPL_WIDE 4
#endif
#ifndef ATTNRES_PHASE2_WIDE_ROWS
#define ATTNRES_PHASE2_WIDE_ROWS 4096
#endif

static Geom make_geom(int64_t R, int64_t D, int esize, int vpl, int waves_per_group_max) {
  Geom g;
  g.R = R;
  g.D = (int)D;
  g.V = (int)(D * esize / 16);
  g.W = (g.V + 64 * vpl - 1) / (64 * vpl);
  g.RPW = g.W >= waves_per_group_max ? 1 : waves_per_group_max / g.W;
  g.groups = (R + g.RPW - 1) / g.RPW;
  g.invD = 1.0f / (float)D;
  return g;
}

static unsigned grid_for(const Geom& g) {
  // one workgroup per row group; the hardware spreads them over the 256 CUs
  // (round-robin across the 8 XCDs); cap keeps the grid-stride loop short
  const int64_t cap = 1 << 20;
  return (unsigned)(g.groups < cap ? g.groups : cap);
}

template <typename K, typename... Args>
static hipError_t launch(const Launch& L, K kernel, dim3 grid, dim3 block, size_t lds,
                         Args... args) {
  if (L.start || L.stop) {
    // the start/stop events take the timestamps of this kernel's own dispatch
    // (either may be null: a sequence of launches is timed first to last)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, L.stream, L.start, L.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, L.stream, args...);
  }
  return hipGetLastError();
}

hipError_t launch_fold(const float* w, const float* g, float* q, int64_t count, const Launch& L) {
  const int64_t blocks = (count + 255) / 256;
  return launch(L, fold_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, w,
                g, q, count);
}

template <class T, int VPL, int NMAX, int SB>
static hipError_t launch_phase1_t(Phase1Params& p, const Launch& L) {
  const int nv = SB * NMAX + NMAX;
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * nv * sizeof(float) : 0;
  return launch(L, phase1_kernel<T, VPL, NMAX, SB>, dim3(grid_for(p.g)),
                dim3(64 * p.g.W * p.g.RPW), lds, p);
}

// Phase 1 for n <= 16 sources. Returns hipErrorInvalidValue if the shape is
// beyond the register-resident kernel (the caller then falls back).
template <class T>
static hipError_t launch_phase1_dt(const Phase1Args& a, const Launch& L) {
  Phase1Params p;
  for (int i = 0; i < 16; ++i) p.src[i] = i < a.n ? a.src[i] : nullptr;
  p.n = a.n; p.S = a.S; p.Wq = a.W; p.G = a.G; p.eps = a.eps;
  p.out = a.out; p.m_out = a.m_out; p.lse_out = a.lse_out;
  p.cl = Close{a.close_p, a.close_v, a.close_b};
  if (a.n <= 8) {
    p.g = make_geom(a.R, a.D, T::kBytes, 2, 4);
    if (p.g.W > 8) return hipErrorInvalidValue;
    // exact source count: no idle register slots; the query batch shrinks as
    // the resident sources grow so the kernel stays within 256 VGPRs
    switch (a.n) {
      case 1: return launch_phase1_t<T, 2, 1, 8>(p, L);
      case 2: return launch_phase1_t<T, 2, 2, 8>(p, L);
      case 3: return launch_phase1_t<T, 2, 3, 8>(p, L);
      case 4: return launch_phase1_t<T, 2, 4, 8>(p, L);
      case 5: return launch_phase1_t<T, 2, 5, 4>(p, L);
      case 6: return launch_phase1_t<T, 2, 6, 4>(p, L);
      case 7: return launch_phase1_t<T, 2, 7, 2>(p, L);
      default: return launch_phase1_t<T, 2, 8, 2>(p, L);
    }
  }
  if (a.n <= 16) {
    p.g = make_geom(a.R, a.D, T::kBytes, 1, 4);
    if (p.g.W > 8) return hipErrorInvalidValue;
    return launch_phase1_t<T, 1, 16, 1>(p, L);
  }
  return hipErrorInvalidValue;
}

bool phase1_mfma_eligible(int dtype, int n, int S, int64_t D) {
  return dtype == 1 && n >= 1 && n <= kP1MaxN && S >= 1 && S <= kP1MaxS &&
         (D == 1024 || D == 2048 || D == 3072 || D == 4096);
}

template <int KS, int NC>
static hipError_t launch_phase1_mfma_t(const Phase1MParams& p, const Launch& L) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = p.R < cus ? p.R : cus;  // one workgroup per CU, each walks rows
  if (p.nf_out) {
    if constexpr (P1Shape<KS, NC, true>::FITS)
      return launch(L, phase1_mfma_kernel<KS, NC, true>, dim3((unsigned)grid), dim3(64 * kP1Waves), 0, p);
    else
      return hipErrorInvalidValue;
  }
  return launch(L, phase1_mfma_kernel<KS, NC, false>, dim3((unsigned)grid), dim3(64 * kP1Waves), 0, p);
}

template <int KS>
static bool phase1_mfma_norm_fits_k(int n) {
  switch (n) {
    case 1: return P1Shape<KS, 1, true>::FITS;
    case 2: return P1Shape<KS, 2, true>::FITS;
    case 3: return P1Shape<KS, 3, true>::FITS;
    case 4: return P1Shape<KS, 4, true>::FITS;
    case 5: return P1Shape<KS, 5, true>::FITS;
    case 6: return P1Shape<KS, 6, true>::FITS;
    case 7: return P1Shape<KS, 7, true>::FITS;
    default: return P1Shape<KS, 8, true>::FITS;
  }
}

// Whether the register-tile kernel holds the gain and the Gram partials of
// the fused input norm beside two ring slots (not at D = 4096 with 8 sources).
static bool phase1_mfma_norm_fits(int n, int64_t D) {
  switch (D) {
    case 1024: return phase1_mfma_norm_fits_k<8>(n);
    case 2048: return phase1_mfma_norm_fits_k<16>(n);
    case 3072: return phase1_mfma_norm_fits_k<24>(n);
    default: return phase1_mfma_norm_fits_k<32>(n);
  }
}

template <int KS>
static hipError_t launch_phase1_mfma_k(const Phase1MParams& p, const Launch& L) {
  switch (p.n) {
    case 1: return launch_phase1_mfma_t<KS, 1>(p, L);
    case 2: return launch_phase1_mfma_t<KS, 2>(p, L);
    case 3: return launch_phase1_mfma_t<KS, 3>(p, L);
    case 4: return launch_phase1_mfma_t<KS, 4>(p, L);
    case 5: return launch_phase1_mfma_t<KS, 5>(p, L);
    case 6: return launch_phase1_mfma_t<KS, 6>(p, L);
    case 7: return launch_phase1_mfma_t<KS, 7>(p, L);
    default: return launch_phase1_mfma_t<KS, 8>(p, L);
  }
}

static hipError_t launch_phase1_mfma(const Phase1Args& a, const Launch& L) {
  Phase1MParams p;
  for (int i = 0; i < kP1MaxN; ++i) p.src[i] = i < a.n ? a.src[i] : nullptr;
  p.n = a.n; p.S = a.S; p.Wq = a.W; p.G = a.G; p.eps = a.eps;
  p.out = a.out; p.m_out = a.m_out; p.lse_out = a.lse_out;
  p.cl = Close{a.close_p, a.close_v, a.close_b};
  p.R = a.R; p.D = (int)a.D; p.invD = 1.0f / (float)a.D;
  p.nf_g = a.nf_g; p.nf_eps = a.nf_eps; p.nf_out = a.out ? a.nf_out : nullptr;
  p.out0 = a.out0;
  p.out1 = a.out1;
  if (a.nf_out && (!a.out || !phase1_mfma_norm_fits(a.n, a.D))) return hipErrorInvalidValue;
  switch (a.D) {
    case 1024: return launch_phase1_mfma_k<8>(p, L);
    case 2048: return launch_phase1_mfma_k<16>(p, L);
    case 3072: return launch_phase1_mfma_k<24>(p, L);
    default: return launch_phase1_mfma_k<32>(p, L);
  }
}

#ifndef ATTNRES_P1_SINGLE_VPL
#define ATTNRES_P1_SINGLE_VPL 2  // 16-byte vectors per lane of the one-source statistics pass
#endif
#ifndef ATTNRES_P1_SINGLE_GROUPS
#define ATTNRES_P1_SINGLE_GROUPS 2048  // workgroups of the one-source statistics pass
#endif
#ifndef ATTNRES_P1_SINGLE_AHEAD
#define ATTNRES_P1_SINGLE_AHEAD 1  // rows loaded ahead by the one-source statistics pass
#endif

template <class T>
static hipError_t launch_phase1_single(const Phase1Args& a, const Launch& L) {
  Phase1Params p;
  for (int i = 0; i < 16; ++i) p.src[i] = i < a.n ? a.src[i] : nullptr;
  p.n = a.n; p.S = a.S; p.Wq = a.W; p.G = a.G; p.eps = a.eps;
  p.out = nullptr; p.m_out = a.m_out; p.lse_out = a.lse_out;
  p.cl = Close{nullptr, nullptr, nullptr};
  p.nf_g = a.nf_g; p.nf_eps = a.nf_eps; p.nf_out = a.nf_out;
  p.g = make_geom(a.R, a.D, T::kBytes, ATTNRES_P1_SINGLE_VPL, 4);
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * 9 * sizeof(float) : 0;
  const int64_t grid = p.g.groups < ATTNRES_P1_SINGLE_GROUPS ? p.g.groups : ATTNRES_P1_SINGLE_GROUPS;
  return launch(L, phase1_single_kernel<T, ATTNRES_P1_SINGLE_VPL, 8, ATTNRES_P1_SINGLE_AHEAD>,
                dim3((unsigned)grid),
                dim3(64 * p.g.W * p.g.RPW), lds, p);
}

static bool phase1_single_eligible(int dtype, const Phase1Args& a) {
  return !a.out && a.n == 1 && !a.close_v && a.S <= 8 &&
         make_geom(1, a.D, dtype == 1 ? 2 : 4, ATTNRES_P1_SINGLE_VPL, 4).W <= 8;
}

#ifndef ATTNRES_P1_STREAM_GROUPS
#define ATTNRES_P1_STREAM_GROUPS 512  // workgroups of a streamed Phase-1 pass (each walks many rows)
#endif

// Streamed Phase 1: elements per lane E = VPL x (elements per vector); the
// query tile, the SQ numerators and a group of G sources each take E registers
// per query or source, so wider rows take fewer queries per pass.
// At 16 elements per lane with 4 queries (D = 7168 bf16), sources in pairs
// with one pair in flight: 7% faster at 131072 rows and 10% at 128 rows than
// single sources three ahead (the registers hold one or the other).
#ifndef ATTNRES_P1_STREAM_G16
#define ATTNRES_P1_STREAM_G16 2
#endif
#ifndef ATTNRES_P1_STREAM_AHEAD16
#define ATTNRES_P1_STREAM_AHEAD16 1
#endif
#ifndef ATTNRES_P1_STREAM_AHEAD
#define ATTNRES_P1_STREAM_AHEAD 3  // source groups in flight ahead of the one being reduced
#endif

template <class T, int VPL, int G, int SQ, int PD>
static hipError_t launch_phase1_stream_t(Phase1SParams& p, const Phase1Args& a, const Launch& L) {
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * (SQ * G + G) * sizeof(float) : 0;
  const int64_t row_bytes = a.D * T::kBytes;
  // Passes per launch: as many as fit side by side in about
  // ATTNRES_P1_STREAM_GROUPS workgroups, one walker per row group each.
  const int passes = (a.S + SQ - 1) / SQ;
  const int64_t budget = a.max_groups > 0 ? a.max_groups : ATTNRES_P1_STREAM_GROUPS;
  const int64_t busy = p.g.groups < budget ? p.g.groups : budget;
  int per = (int)(budget / busy);
  per = per < 1 ? 1 : per > passes ? passes : per;
  for (int s0 = 0; s0 < a.S; s0 += per * SQ) {
    // later launches read the block sum the first one stored
    if (s0 > 0 && p.cl.v) {
      p.src[a.n - 1] = p.cl.b;
      p.cl = Close{nullptr, nullptr, nullptr};
    }
    p.S = a.S - s0 < per * SQ ? a.S - s0 : per * SQ;
    p.passes = (p.S + SQ - 1) / SQ;
    int64_t walkers = budget / p.passes;
    if (walkers > p.g.groups) walkers = p.g.groups;
    walkers = (walkers + 7) / 8 * 8;  // a multiple of the 8 XCDs
    p.walkers = (int)walkers;
    p.Wq = a.W + (int64_t)s0 * a.D;
    p.G = a.G ? a.G + (int64_t)s0 * a.D : nullptr;
    p.out = static_cast<char*>(a.out) + (int64_t)s0 * a.R * row_bytes;
    p.m_out = a.m_out ? a.m_out + (int64_t)s0 * a.R : nullptr;
    p.lse_out = a.lse_out + (int64_t)s0 * a.R;
    // timed from the first launch's start to the last launch's end
    const Launch Ls{L.stream, s0 == 0 ? L.start : nullptr, s0 + per * SQ >= a.S ? L.stop : nullptr};
    hipError_t e = launch(Ls, phase1_stream_kernel<T, VPL, G, SQ, PD>,
                          dim3((unsigned)(walkers * p.passes)), dim3(64 * p.g.W * p.g.RPW), lds, p);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The smallest of 8, 16 or 32 elements per lane whose row fits eight waves;
// returns the vectors per lane (0: the row is too wide).
static int stream_vpl(int esize, int64_t D, int* E) {
  const int epv = 16 / esize;
  for (int e = 8; e <= 32; e *= 2) {
    const int vpl = e / epv;
    if (make_geom(1, D, esize, vpl, 8).W <= 8) {
      *E = e;
      return vpl;
    }
  }
  return 0;
}

template <class T>
static hipError_t launch_phase1_stream(const Phase1Args& a, const Launch& L) {
  Phase1SParams p;
  for (int i = 0; i < 64; ++i) p.src[i] = i < a.n ? a.src[i] : nullptr;
  p.n = a.n; p.eps = a.eps;
  p.cl = Close{a.close_p, a.close_v, a.close_b};
  int E = 0;
  const int vpl = stream_vpl(T::kBytes, a.D, &E);
  if (!vpl) return hipErrorInvalidValue;
  p.g = make_geom(a.R, a.D, T::kBytes, vpl, 8);
  constexpr int epv = T::kEPV;
  // The kernel is bound by vector-ALU issue, which scales with the query
  // tile, so the tile is the smallest that covers S (or the largest that fits
  // the registers, in passes); smaller tiles leave room for larger source
  // groups. bf16 keeps ATTNRES_P1_STREAM_AHEAD groups in flight at 8 and 16
  // elements per lane (the 4-query tile at 16: ATTNRES_P1_STREAM_G16 sources
  // per group, ATTNRES_P1_STREAM_AHEAD16 groups ahead); fp32 vectors (and the
  // widest rows) take twice the registers and keep one.
  constexpr int PD = T::kBytes == 2 ? ATTNRES_P1_STREAM_AHEAD : 1;
  if (E == 8) {
    if (a.S <= 2) return launch_phase1_stream_t<T, 8 / epv, 4, 2, PD>(p, a, L);
    if (a.S <= 4) return launch_phase1_stream_t<T, 8 / epv, 4, 4, PD>(p, a, L);
    return launch_phase1_stream_t<T, 8 / epv, 2, 8, PD>(p, a, L);
  }
  if (E == 16) {
    if (a.S <= 1) return launch_phase1_stream_t<T, 16 / epv, 2, 1, PD>(p, a, L);
    if (a.S <= 2) return launch_phase1_stream_t<T, 16 / epv, 2, 2, PD>(p, a, L);
    return launch_phase1_stream_t<T, 16 / epv, ATTNRES_P1_STREAM_G16, 4,
                                  T::kBytes == 2 ? ATTNRES_P1_STREAM_AHEAD16 : 1>(p, a, L);
  }
  if constexpr (T::kBytes == 2) {
    if (a.S >= 2) return launch_phase1_stream_t<T, 32 / epv, 1, 2, 1>(p, a, L);
  }
  return launch_phase1_stream_t<T, 32 / epv, 1, 1, 1>(p, a, L);
}

#ifndef ATTNRES_P1_GEMM_MIN_ROWS
#define ATTNRES_P1_GEMM_MIN_ROWS 4096  // fewer rows: the streamed kernel (its passes run side by side)
#endif

static int gemm_tiles(int S) { return (S + 7) / 8; }
constexpr int kGMaxN = 16;  // sources per row of the scores/outputs passes

bool phase1_gemm_shape(int dtype, int S, int64_t D, int64_t R) {
  // (the outputs pass keeps its row index in a 32-bit scalar register)
  return dtype == 1 && S >= 1 && S <= 32 && D % (2 * kGChunk) == 0 && D <= 8192 &&
         R >= ATTNRES_P1_GEMM_MIN_ROWS && R <= INT32_MAX;
}

// More than 8 sources take the two passes only with at least 4 queries: the
// scores pass reads the sources once more, which with fewer queries costs
// more than the streamed kernel's arithmetic (the Full schedule at C = 2 went
// 4.49 -> 4.83 ms that way).
bool phase1_gemm_eligible(int dtype, int n, int S, int64_t D, int64_t R) {
  return n >= 1 && n <= kGMaxN && (n <= 8 || S >= 4) && phase1_gemm_shape(dtype, S, D, R) &&
         !phase1_mfma_eligible(dtype, n, S, D);
}

int phase1_gemm_needed(int dtype, int S, int64_t D, int64_t R, int nmax) {
  int most = 0;
  if (S < 2 || !phase1_gemm_shape(dtype, S, D, R)) return 0;
  for (int n = 1; n <= nmax && n <= kGMaxN; ++n)
    if (phase1_gemm_eligible(dtype, n, S, D, R)) most = n;
  return most;
}

static size_t gemm_qp_bytes(int S, int64_t D) {
  return ((size_t)32 * gemm_tiles(S) * D * 2 + 255) & ~(size_t)255;
}

size_t phase1_gemm_workspace(int S, int64_t R, int64_t D, int nmax) {
  return gemm_qp_bytes(S, D) + (size_t)S * R * (nmax > 8 ? 16 : 8) * sizeof(float);
}

template <int MT, int NPR>
static hipError_t launch_gemm_scores_t(const P1GParams& g, const Launch& L) {
  const int64_t tiles = (g.R + kGWaves * (16 / NPR) - 1) / (kGWaves * (16 / NPR));
  const unsigned grid = (unsigned)(tiles < (1 << 20) ? tiles : (1 << 20));
  return launch(L, phase1_gemm_scores_kernel<MT, NPR>, dim3(grid), dim3(64 * kGWaves), 0, g);
}

// Source columns per row: the smallest of 1, 2, 4, 8 or 16 that holds the n
// sources, so a 16-column tile takes 16 / NPR rows.
template <int MT>
static hipError_t launch_gemm_scores(const P1GParams& g, const Launch& L) {
  if (g.n <= 1) return launch_gemm_scores_t<MT, 1>(g, L);
  if (g.n <= 2) return launch_gemm_scores_t<MT, 2>(g, L);
  if (g.n <= 4) return launch_gemm_scores_t<MT, 4>(g, L);
  if (g.n <= 8) return launch_gemm_scores_t<MT, 8>(g, L);
  return launch_gemm_scores_t<MT, 16>(g, L);
}

template <int NC>
static hipError_t launch_gemm_outputs(const P1OParams& o, bool nt, const Launch& L) {
  const unsigned grid = grid_for(o.g);
  const dim3 block(64 * o.g.W * o.g.RPW);
  if constexpr (NC > 8) {
    if (nt) return launch(L, phase1_gemm_outputs_wide_kernel<NC, true>, dim3(grid), block, 0, o);
    return launch(L, phase1_gemm_outputs_wide_kernel<NC, false>, dim3(grid), block, 0, o);
  } else {
    if (nt) return launch(L, phase1_gemm_outputs_kernel<NC, true>, dim3(grid), block, 0, o);
    return launch(L, phase1_gemm_outputs_kernel<NC, false>, dim3(grid), block, 0, o);
  }
}

// Phase 1 as a query split, a matrix-core scores pass and an outputs pass
// (see phase1_gemm_scores_kernel); without an output buffer (statistics
// only) the outputs pass is skipped. The sources must be materialised (no
// fused close); `ws` holds phase1_gemm_workspace(S, R, D, n) bytes.
hipError_t launch_phase1_gemm(const Phase1Args& a, void* ws, const Launch& L) {
  if (a.close_v || !phase1_gemm_eligible(1, a.n, a.S, a.D, a.R)) return hipErrorInvalidValue;
  const int MT = gemm_tiles(a.S);
  __bf16* qp = static_cast<__bf16*>(ws);
  float* alpha = reinterpret_cast<float*>(static_cast<char*>(ws) + gemm_qp_bytes(a.S, a.D));
  // timed from the split's start to the outputs pass's end
  const Launch first{L.stream, L.start, nullptr}, last{L.stream, nullptr, L.stop};
  const Launch mid{L.stream, nullptr, a.out ? nullptr : L.stop};
  {
    QSplitParams q{a.W, a.G, a.S, MT, a.D, qp};
    const int64_t blocks = ((int64_t)MT * 32 * a.D + 255) / 256;
    hipError_t e = launch(first, qsplit_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, q);
    if (e != hipSuccess) return e;
  }
  {
    P1GParams g;
    for (int i = 0; i < kGMaxN; ++i) g.src[i] = i < a.n ? a.src[i] : a.src[0];
    g.n = a.n; g.S = a.S; g.qp = qp; g.eps = a.eps; g.invD = 1.0f / (float)a.D;
    g.R = a.R; g.D = (int)a.D; g.alpha = alpha; g.m_out = a.m_out; g.lse_out = a.lse_out;
    hipError_t e;
    switch (MT) {
      case 1: e = launch_gemm_scores<1>(g, mid); break;
      case 2: e = launch_gemm_scores<2>(g, mid); break;
      case 3: e = launch_gemm_scores<3>(g, mid); break;
      default: e = launch_gemm_scores<4>(g, mid); break;
    }
    if (e != hipSuccess) return e;
  }
  if (!a.out) return hipSuccess;
  P1OParams o;
  for (int i = 0; i < kGMaxN; ++i) o.src[i] = i < a.n ? a.src[i] : a.src[0];
  o.S = a.S; o.alpha = alpha; o.out = a.out;
  // two vectors per lane up to 8 sources (at most 8 waves per row), one
  // vector per lane beyond (at most 16)
  o.g = a.n > 8 ? make_geom(a.R, a.D, 2, 1, 16) : make_geom(a.R, a.D, 2, 2, 8);
  if (o.g.W > (a.n > 8 ? 16 : 8)) return hipErrorInvalidValue;
  const bool nt = (double)a.R * a.D * 2 > (double)ATTNRES_PHASE2_NT_BYTES;
  switch (a.n) {
    case 1: return launch_gemm_outputs<1>(o, nt, last);
    case 2: return launch_gemm_outputs<2>(o, nt, last);
    case 3: return launch_gemm_outputs<3>(o, nt, last);
    case 4: return launch_gemm_outputs<4>(o, nt, last);
    case 5: return launch_gemm_outputs<5>(o, nt, last);
    case 6: return launch_gemm_outputs<6>(o, nt, last);
    case 7: return launch_gemm_outputs<7>(o, nt, last);
    case 8: return launch_gemm_outputs<8>(o, nt, last);
    case 9: return launch_gemm_outputs<9>(o, nt, last);
    case 10: return launch_gemm_outputs<10>(o, nt, last);
    case 11: return launch_gemm_outputs<11>(o, nt, last);
    case 12: return launch_gemm_outputs<12>(o, nt, last);
    case 13: return launch_gemm_outputs<13>(o, nt, last);
    case 14: return launch_gemm_outputs<14>(o, nt, last);
    case 15: return launch_gemm_outputs<15>(o, nt, last);
    default: return launch_gemm_outputs<16>(o, nt, last);
  }
}

#ifndef ATTNRES_P1_STREAM
#define ATTNRES_P1_STREAM 1  // 0: the register-resident vector-ALU Phase 1 where it applies
#endif

hipError_t launch_phase1(int dtype, const Phase1Args& a, const Launch& L) {
  if (phase1_single_eligible(dtype, a))
    return dtype == 1 ? launch_phase1_single<Bf16>(a, L) : launch_phase1_single<F32>(a, L);
  if (phase1_mfma_eligible(dtype, a.n, a.S, a.D)) return launch_phase1_mfma(a, L);
  if (a.out && (ATTNRES_P1_STREAM || a.n > 16))
    return dtype == 1 ? launch_phase1_stream<Bf16>(a, L) : launch_phase1_stream<F32>(a, L);
  return dtype == 1 ? launch_phase1_dt<Bf16>(a, L) : launch_phase1_dt<F32>(a, L);
}

// The one-source statistics kernel writes the norm from the sum of squares
// it forms anyway; the register-tile kernel takes output 0's sum of squares
// from the Gram matrix of the row's sources, reduced with the scores, so the
// norm needs no exchange between waves of its own.
bool phase1_out01_supported(int dtype, const Phase1Args& a, bool gemm) {
  return !gemm && a.out && !phase1_single_eligible(dtype, a) && phase1_mfma_eligible(dtype, a.n, a.S, a.D);
}

bool phase1_norm_fused(int dtype, const Phase1Args& a, bool gemm) {
  if (gemm) return false;
  if (phase1_single_eligible(dtype, a)) return true;
  return a.out && phase1_mfma_eligible(dtype, a.n, a.S, a.D) && phase1_mfma_norm_fits(a.n, a.D);
}

const char* phase1_kernel_name(int dtype, const Phase1Args& a, bool gemm) {
  if (gemm) return a.out ? "phase1_gemm_scores_kernel+phase1_gemm_outputs_kernel" : "phase1_gemm_scores_kernel";
  if (phase1_single_eligible(dtype, a)) return "phase1_single_kernel";
  if (phase1_mfma_eligible(dtype, a.n, a.S, a.D)) return "phase1_mfma_kernel";
  if (a.out && (ATTNRES_P1_STREAM || a.n > 16)) return "phase1_stream_kernel";
  return "phase1_kernel";
}

bool phase1_stats_supported(int dtype, int n, int S, int64_t D) {
  if (phase1_mfma_eligible(dtype, n, S, D)) return true;
  if (n < 1 || n > 8) return false;
  return make_geom(1, D, dtype == 1 ? 2 : 4, 2, 4).W <= 8;
}

bool phase1_supported(int dtype, int n, int S, int64_t D) {
  if (phase1_mfma_eligible(dtype, n, S, D)) return true;
  if (n < 1 || n > 64) return false;
  int E = 0;
  return stream_vpl(dtype == 1 ? 2 : 4, D, &E) != 0;
}

#ifndef ATTNRES_AGG_PACKED_MIN_D
#define ATTNRES_AGG_PACKED_MIN_D 2048  // narrower rows keep the 8-source group unpacked
#endif

template <class T, int VPL, int G, bool PK = false>
static hipError_t launch_agg_t(AggParams& p, const Launch& L) {
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * 2 * G * sizeof(float) : 0;
  return launch(L, aggregate_kernel<T, VPL, G, PK>, dim3(grid_for(p.g)), dim3(64 * p.g.W * p.g.RPW),
                lds, p);
}

template <class T>
static hipError_t launch_aggregate_dt(const AggArgs& a, const Launch& L) {
  AggParams p;
  for (int i = 0; i < 64; ++i) p.src[i] = i < a.n ? a.src[i] : nullptr;
  p.n = a.n; p.w = a.w; p.gm = a.g; p.eps = a.eps;
  p.out = a.out; p.m_out = a.m_out; p.lse_out = a.lse_out;
  p.cl = Close{a.close_p, a.close_v, a.close_b};
  p.o_init = a.o_init; p.lse_init = a.lse_init;
  p.nf_g = a.nf_g; p.nf_eps = a.nf_eps; p.nf_out = a.nf_out;
  p.g = make_geom(a.R, a.D, T::kBytes, 2, 4);
  if (p.g.W > 8) {
    // widest rows: four vectors per lane and groups of four sources
    p.g = make_geom(a.R, a.D, T::kBytes, 4, 4);
    if (p.g.W > 8) return hipErrorInvalidValue;
    return launch_agg_t<T, 4, 4>(p, L);
  }
  if (a.n <= 2) return launch_agg_t<T, 2, 2>(p, L);
  if (a.n <= 4) return launch_agg_t<T, 2, 4>(p, L);
  // one group of 5..8 sources over rows of at least ATTNRES_AGG_PACKED_MIN_D
  // elements: packed (config 3's final aggregate 244 -> 222 us); two or more
  // groups, or narrower rows, measured slower that way
  if (a.n <= 8 && a.D >= ATTNRES_AGG_PACKED_MIN_D) return launch_agg_t<T, 2, 8, true>(p, L);
  return launch_agg_t<T, 2, 8>(p, L);
}

hipError_t launch_aggregate(int dtype, const AggArgs& a, const Launch& L) {
  return dtype == 1 ? launch_aggregate_dt<Bf16>(a, L) : launch_aggregate_dt<F32>(a, L);
}

template <class T, int VPL, bool HP>
#ifndef ATTNRES_PHASE2_MAX_GROUPS
#define ATTNRES_PHASE2_MAX_GROUPS (1 << 20)  // workgroups of a Phase-2 launch (rows per group beyond: grid-stride)
#endif

static hipError_t launch_ph2_t(Phase2Params& p, const Launch& L) {
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * 2 * sizeof(float) : 0;
  if (p.xs) {
    // with an extra source: four row sums; written with plain stores (this
    // variant serves the few-row decode schedule)
    const size_t lds4 = 2 * lds;
    const unsigned grid4 = (unsigned)(p.g.groups < ATTNRES_PHASE2_MAX_GROUPS ? p.g.groups
                                                                              : ATTNRES_PHASE2_MAX_GROUPS);
    if (p.hn_out)
      return launch(L, phase2_kernel<T, VPL, HP, true, false, true>, dim3(grid4),
                    dim3(64 * p.g.W * p.g.RPW), lds4, p);
    return launch(L, phase2_kernel<T, VPL, HP, false, false, true>, dim3(grid4),
                  dim3(64 * p.g.W * p.g.RPW), lds4, p);
  }
  const unsigned grid = (unsigned)(p.g.groups < ATTNRES_PHASE2_MAX_GROUPS ? p.g.groups
                                                                           : ATTNRES_PHASE2_MAX_GROUPS);
  const dim3 block(64 * p.g.W * p.g.RPW);
  if ((double)p.g.R * p.g.V * 16 > (double)ATTNRES_PHASE2_NT_BYTES) {
    if (p.hn_out) return launch(L, phase2_kernel<T, VPL, HP, true, true>, dim3(grid), block, lds, p);
    return launch(L, phase2_kernel<T, VPL, HP, false, true>, dim3(grid), block, lds, p);
  }
  if (p.hn_out) return launch(L, phase2_kernel<T, VPL, HP, true, false>, dim3(grid), block, lds, p);
  return launch(L, phase2_kernel<T, VPL, HP, false, false>, dim3(grid), block, lds, p);
}

template <class T, bool HP>
static hipError_t launch_ph2_vpl(Phase2Params& p, int vpl, const Launch& L) {
  if (p.xs) {
    // the extra-source variant exists for 2, 4 and 8 vectors per lane
    switch (vpl) {
      case 2: return launch_ph2_t<T, 2, HP>(p, L);
      case 4: return launch_ph2_t<T, 4, HP>(p, L);
      case 8: return launch_ph2_t<T, 8, HP>(p, L);
      default: return hipErrorInvalidValue;
    }
  }
  switch (vpl) {
    case 1: return launch_ph2_t<T, 1, HP>(p, L);
    case 2: return launch_ph2_t<T, 2, HP>(p, L);
    case 3: return launch_ph2_t<T, 3, HP>(p, L);
    case 4: return launch_ph2_t<T, 4, HP>(p, L);
    case 5: return launch_ph2_t<T, 5, HP>(p, L);
    case 6: return launch_ph2_t<T, 6, HP>(p, L);
    case 7: return launch_ph2_t<T, 7, HP>(p, L);
    default: return launch_ph2_t<T, 8, HP>(p, L);
  }
}

template <class T>
static hipError_t launch_phase2_dt(const Phase2Args& a, const Launch& L) {
  Phase2Params p;
  p.o = a.o; p.lse = a.lse; p.w = a.w; p.gm = a.g; p.eps = a.eps;
  p.p_prev = a.p_prev; p.v_prev = a.v_prev; p.p_out = a.p_out; p.h_out = a.h_out;
  p.gf = a.gf; p.eps_f = a.eps_f; p.hn_out = a.hn_out; p.xs = a.xs;
  // ATTNRES_PHASE2_VPL vectors per lane (ATTNRES_PHASE2_VPL_WIDE for the
  // normed and first merges over many rows), more when a row would need
  // over MW waves (rows are at most 2048 vectors, so at most 8 per lane);
  // with an extra source the next of 2, 4 or 8
  const int V = (int)(a.D * T::kBytes / 16);
  constexpr int MW = ATTNRES_PHASE2_MAX_WAVES;
  const bool wide = (a.hn_out || !a.p_prev) && a.R >= ATTNRES_PHASE2_WIDE_ROWS &&
                    V % (64 * ATTNRES_PHASE2_VPL_WIDE) == 0;
  int vpl = wide ? ATTNRES_PHASE2_VPL_WIDE : ATTNRES_PHASE2_VPL;
  if (64 * MW * vpl < V) vpl = (V + 64 * MW - 1) / (64 * MW);
  if (a.xs) vpl = vpl <= 2 ? 2 : vpl <= 4 ? 4 : 8;
  p.g = make_geom(a.R, a.D, T::kBytes, vpl, 4);
  if (p.g.W > MW || vpl > 8 || 64 * p.g.W * p.g.RPW > ATTNRES_PHASE2_LB) return hipErrorInvalidValue;
  return a.p_prev ? launch_ph2_vpl<T, true>(p, vpl, L) : launch_ph2_vpl<T, false>(p, vpl, L);
}

hipError_t launch_phase2(int dtype, const Phase2Args& a, const Launch& L) {
  return dtype == 1 ? launch_phase2_dt<Bf16>(a, L) : launch_phase2_dt<F32>(a, L);
}

template <class T, int VPL>
static hipError_t launch_norm_t(const NormParams& p, const Launch& L) {
  const size_t lds = p.geo.W > 1 ? (size_t)p.geo.RPW * p.geo.W * sizeof(float) : 0;
  return launch(L, rmsnorm_kernel<T, VPL>, dim3(grid_for(p.geo)), dim3(64 * p.geo.W * p.geo.RPW), lds, p);
}

template <class T>
static hipError_t launch_rmsnorm_dt(const void* x, int64_t R, int64_t D, const float* g, float eps,
                                    void* out, const Launch& L) {
  NormParams p{x, g, eps, out, Geom{}};
  const int V = (int)(D * T::kBytes / 16);
  int vpl = 2;
  if (64 * 4 * vpl < V) vpl = (V + 255) / 256;
  p.geo = make_geom(R, D, T::kBytes, vpl, 4);
  if (p.geo.W > 4 || vpl > 8) return hipErrorInvalidValue;
  switch (vpl) {
    case 1: return launch_norm_t<T, 1>(p, L);
    case 2: return launch_norm_t<T, 2>(p, L);
    case 3: return launch_norm_t<T, 3>(p, L);
    case 4: return launch_norm_t<T, 4>(p, L);
    case 5: return launch_norm_t<T, 5>(p, L);
    case 6: return launch_norm_t<T, 6>(p, L);
    case 7: return launch_norm_t<T, 7>(p, L);
    default: return launch_norm_t<T, 8>(p, L);
  }
}

hipError_t launch_rmsnorm(int dtype, const void* x, int64_t R, int64_t D, const float* g, float eps,
                          void* out, const Launch& L) {
  return dtype == 1 ? launch_rmsnorm_dt<Bf16>(x, R, D, g, eps, out, L)
                    : launch_rmsnorm_dt<F32>(x, R, D, g, eps, out, L);
}

#ifndef ATTNRES_CLOSE_MAX_GROUPS
#define ATTNRES_CLOSE_MAX_GROUPS (1 << 20)  // workgroups of a standalone close: one vector per lane (grid-stride beyond)
#endif

hipError_t launch_partials(int dtype, const void* const* in, void* const* out, int n, int64_t R, int64_t D,
                           const Launch& L) {
  if (n < 2 || n > kPartialsMax) return hipErrorInvalidValue;
  PartialsParams p;
  for (int t = 0; t < kPartialsMax; ++t) {
    p.in[t] = t < n ? in[t] : in[0];
    p.out[t] = t < n ? out[t] : nullptr;
  }
  p.n = n;
  p.nvec = R * D * (dtype == 1 ? 2 : 4) / 16;
  if (p.nvec == 0) return hipSuccess;
  int64_t blocks = (p.nvec + 255) / 256;
  if (blocks > ATTNRES_CLOSE_MAX_GROUPS) blocks = ATTNRES_CLOSE_MAX_GROUPS;
  if (dtype == 1) return launch(L, partials_kernel<Bf16>, dim3((unsigned)blocks), dim3(256), 0, p);
  return launch(L, partials_kernel<F32>, dim3((unsigned)blocks), dim3(256), 0, p);
}

hipError_t launch_close(int dtype, const void* p, const void* v, void* b, int64_t R, int64_t D,
                        const Launch& L) {
  const int64_t nvec = R * D * (dtype == 1 ? 2 : 4) / 16;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > ATTNRES_CLOSE_MAX_GROUPS) blocks = ATTNRES_CLOSE_MAX_GROUPS;
  if (dtype == 1) return launch(L, close_kernel<Bf16>, dim3((unsigned)blocks), dim3(256), 0, p, v, b, nvec);
  return launch(L, close_kernel<F32>, dim3((unsigned)blocks), dim3(256), 0, p, v, b, nvec);
}

// ---------------------------------------------------------------------------
// aggregate backward: plan (geometry, grid, workspace) and launches
// ---------------------------------------------------------------------------
#ifndef ATTNRES_BWD_MAX_GROUPS
#define ATTNRES_BWD_MAX_GROUPS 1024  // workgroups of the backward (bounds the dq~ partials)
#endif
#ifndef ATTNRES_BWD_CHUNK
#define ATTNRES_BWD_CHUNK 32  // partial rows summed per first-stage thread
#endif

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

#ifndef ATTNRES_BWD_BF16_VPL
#define ATTNRES_BWD_BF16_VPL 4  // four-element bf16 vectors per lane (32 bytes of a source)
#endif
#ifndef ATTNRES_BWD_F32_VPL
#define ATTNRES_BWD_F32_VPL 2  // four-element fp32 vectors per lane (32 bytes of a source)
#endif

#ifndef ATTNRES_BWD_AGG_BF16_VPL
// The aggregate backward (one reduction of 3n sums per row, then the
// gradient pass) over bf16 rows that 2 vectors per lane spread over 4..8
// waves: 7 sources at 16384 x 4096 took 573 us at 4 vectors per lane and
// 554 us at 2. The merge backward stays at ATTNRES_BWD_BF16_VPL (at 2 the
// stack backward went 18.4 -> 19.6 ms).
#define ATTNRES_BWD_AGG_BF16_VPL 2
#endif

// Four-element vectors (V = D / 4 per row): VPL of them per lane, doubled
// (then quadrupled) for rows too wide for eight waves. The aggregate
// backward over bf16 takes ATTNRES_BWD_AGG_BF16_VPL where that fills 4..8
// waves and both widths take one row per workgroup: the merge backward
// shares the plan's grid and dq~ partial rows (grid x rows per workgroup),
// so the two geometries must agree on rows per workgroup.
static Geom bwd_geom(int dtype, int64_t R, int64_t D, int* vpl, bool agg = false) {
  int v = dtype == 1 ? ATTNRES_BWD_BF16_VPL : ATTNRES_BWD_F32_VPL;
  Geom g = make_geom(R, D, 4, v, 4);
  while (g.W > 8 && v < 16) {
    v *= 2;
    g = make_geom(R, D, 4, v, 4);
  }
  if (agg && dtype == 1) {
    const Geom ga = make_geom(R, D, 4, ATTNRES_BWD_AGG_BF16_VPL, 4);
    if (ga.W >= 4 && ga.W <= 8 && ga.RPW == g.RPW) {
      *vpl = ATTNRES_BWD_AGG_BF16_VPL;
      return ga;
    }
  }
  *vpl = v;
  return g;
}

BwdPlan plan_aggregate_bwd(int dtype, int64_t R, int64_t D) {
  BwdPlan pl;
  int vpl = 0;
  const Geom g = bwd_geom(dtype, R, D, &vpl, true);
  pl.vpl = vpl;
  pl.supported = g.W <= 8;
  pl.grid = (unsigned)(g.groups < ATTNRES_BWD_MAX_GROUPS ? g.groups : ATTNRES_BWD_MAX_GROUPS);
  pl.P = (int64_t)pl.grid * g.RPW;
  pl.chunk = ATTNRES_BWD_CHUNK;
  pl.P2 = pl.P > pl.chunk ? (pl.P + pl.chunk - 1) / pl.chunk : 0;
  pl.partial_bytes = align256((size_t)pl.P * D * 4);
  pl.bytes = pl.partial_bytes + align256((size_t)pl.P2 * D * 4);
  return pl;
}

template <class T, int VPL, int G, bool RES>
static hipError_t launch_bwd_t(const AggBwdParams& p, unsigned grid, const Launch& L) {
  const int waves = p.g.W * p.g.RPW;
  const size_t lds = (size_t)p.g.RPW * p.g.W * 3 * G * sizeof(float) +
                     (RES ? 0 : (size_t)waves * 64 * sizeof(BwdStat));
  if (p.accumulate)
    return launch(L, aggregate_bwd_kernel<T, VPL, G, RES, true>, dim3(grid), dim3(64 * waves), lds, p);
  return launch(L, aggregate_bwd_kernel<T, VPL, G, RES, false>, dim3(grid), dim3(64 * waves), lds, p);
}

// n <= G sources stay resident; wider rows (more vectors per lane) keep
// groups of four
template <class F, int VPL, bool WIDE>
static hipError_t launch_bwd_vpl(const AggBwdParams& p, int n, unsigned grid, const Launch& L) {
  if constexpr (WIDE) {
    if (n <= 4) return launch_bwd_t<F, VPL, 4, true>(p, grid, L);
    return launch_bwd_t<F, VPL, 4, false>(p, grid, L);
  } else {
    // resident groups; sizes measured at 16384 rows of 4096 bf16: exact
    // groups for 1-4 and 7, a group of 8 for 5 and 6 (exact groups of 5 and 6
    // ran no faster, 6 about 11% slower)
    switch (n) {
      case 1: return launch_bwd_t<F, VPL, 1, true>(p, grid, L);
      case 2: return launch_bwd_t<F, VPL, 2, true>(p, grid, L);
      case 3: return launch_bwd_t<F, VPL, 3, true>(p, grid, L);
      case 4: return launch_bwd_t<F, VPL, 4, true>(p, grid, L);
      case 7: return launch_bwd_t<F, VPL, 7, true>(p, grid, L);
      case 5:
      case 6:
      case 8: return launch_bwd_t<F, VPL, 8, true>(p, grid, L);
      default: break;
    }
    if (n <= 16) return launch_bwd_t<F, VPL, 16, true>(p, grid, L);
    return launch_bwd_t<F, VPL, 8, false>(p, grid, L);
  }
}

template <class F, int SMALL>
static hipError_t launch_bwd_dt(const BwdArgs& a, const BwdPlan& pl, const Launch& L) {
  AggBwdParams p;
  for (int i = 0; i < 64; ++i) {
    p.src[i] = i < a.n ? a.src[i] : nullptr;
    p.dV[i] = i < a.n ? a.dV[i] : nullptr;
  }
  p.n = a.n; p.accumulate = a.accumulate;
  p.w = a.w; p.gm = a.g; p.eps = a.eps; p.dh = a.dh;
  p.dh_scale = a.dh_scale; p.dlse = a.dlse;
  p.partial = static_cast<float*>(a.workspace);
  int vpl = 0;
  p.g = bwd_geom(F::kBytes == 8 ? 1 : 0, a.R, a.D, &vpl, true);
  if constexpr (F::kBytes == 8 && ATTNRES_BWD_AGG_BF16_VPL < SMALL) {
    if (vpl == ATTNRES_BWD_AGG_BF16_VPL) return launch_bwd_vpl<F, ATTNRES_BWD_AGG_BF16_VPL, false>(p, a.n, pl.grid, L);
  }
  if (vpl == SMALL) return launch_bwd_vpl<F, SMALL, false>(p, a.n, pl.grid, L);
  if (vpl == 2 * SMALL) return launch_bwd_vpl<F, 2 * SMALL, true>(p, a.n, pl.grid, L);
  if constexpr (SMALL * 4 <= 8) {
    if (vpl == 4 * SMALL) return launch_bwd_vpl<F, 4 * SMALL, true>(p, a.n, pl.grid, L);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_aggregate_bwd(int dtype, const BwdArgs& a, const BwdPlan& pl, const Launch& L) {
  if (pl.grid == 0) return hipSuccess;
  return dtype == 1 ? launch_bwd_dt<Bf16x4, ATTNRES_BWD_BF16_VPL>(a, pl, L)
                    : launch_bwd_dt<F32x4, ATTNRES_BWD_F32_VPL>(a, pl, L);
}

hipError_t launch_bwd_reduce(const BwdArgs& a, const BwdPlan& pl, int stage, const Launch& L) {
  const float* partial = static_cast<const float*>(a.workspace);
  float* stage1 = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + pl.partial_bytes);
  const unsigned bx = (unsigned)((a.D / 4 + 255) / 256);
  if (stage == 0) {
    if (pl.P2 == 0) return hipSuccess;
    return launch(L, bwd_colsum_kernel<false>, dim3(bx, (unsigned)pl.P2), dim3(256), 0, partial,
                  pl.P, a.D, pl.chunk, stage1, (const float*)nullptr, (const float*)nullptr,
                  (float*)nullptr, (float*)nullptr, 0u, (int64_t)0, (int64_t)0);
  }
  const float* in = pl.P2 ? stage1 : partial;
  const int64_t rows = pl.P2 ? pl.P2 : pl.P;
  return launch(L, bwd_colsum_kernel<true>, dim3(bx, 1), dim3(256), 0, in, rows, a.D, rows,
                (float*)nullptr, a.w, a.g, a.dw, a.dgamma,
                (unsigned)((a.accumulate_q < 0 ? a.accumulate : a.accumulate_q) ? 1 : 0), (int64_t)0, (int64_t)0);
}

// The query-gradient reductions of nq aggregates in one launch per stage:
// query q's dq~ partial rows (the plan's layout, its first-stage sums after
// them) start q * slot bytes into ws; w, g, dw and dgamma are the first
// query's rows, the others D apart. Timed from the first stage's start to
// the second's end.
hipError_t launch_bwd_reduce_queries(const BwdPlan& pl, void* ws, size_t slot, int nq, int64_t D,
                                     const float* w, const float* g, float* dw, float* dgamma,
                                     unsigned acc_mask, const Launch& L) {
  if (nq < 1 || nq > 32 || slot % sizeof(float)) return hipErrorInvalidValue;
  const unsigned bx = (unsigned)((D / 4 + 255) / 256);
  const int64_t qs = (int64_t)(slot / sizeof(float));
  const float* partial = static_cast<const float*>(ws);
  float* stage1 = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.partial_bytes);
  if (pl.P2) {
    hipError_t e = launch(Launch{L.stream, L.start, nullptr}, bwd_colsum_kernel<false>,
                          dim3(bx, (unsigned)pl.P2, (unsigned)nq), dim3(256), 0, partial, pl.P, D, pl.chunk,
                          stage1, (const float*)nullptr, (const float*)nullptr, (float*)nullptr, (float*)nullptr,
                          0u, qs, qs);
    if (e != hipSuccess) return e;
  }
  const float* in = pl.P2 ? stage1 : partial;
  const int64_t rows = pl.P2 ? pl.P2 : pl.P;
  return launch(Launch{L.stream, pl.P2 ? nullptr : L.start, L.stop}, bwd_colsum_kernel<true>,
                dim3(bx, 1, (unsigned)nq), dim3(256), 0, in, rows, D, rows, (float*)nullptr, w, g, dw, dgamma,
                acc_mask, qs, (int64_t)0);
}

#ifndef ATTNRES_P1BWD_GROUPS
#define ATTNRES_P1BWD_GROUPS 512  // workgroups of the batched Phase-1 backward (each walks rows)
#endif

// up to 8 sources (the coefficients take one 8-lane group per query); rows
// of at most 2 x 64 x 8 four-element vectors
bool phase1_bwd_eligible(int dtype, int n, int64_t D) {
  const int64_t V = D / 4;
  return dtype == 1 && n >= 1 && n <= kP1BwdMaxN && D % 4 == 0 && V <= 64 * 8 * kP1BwdVpl;
}

// With 8 queries, up to 6 sources fit the registers (244 VGPRs at 6); 7 and
// 8 sources spill inside the row loop from 7 queries, so they take 4.
int phase1_bwd_max_queries(int n) { return n <= 6 ? kP1BwdQ : 4; }

size_t phase1_bwd_workspace(int64_t R, int64_t D) {
  const int64_t grid = R < ATTNRES_P1BWD_GROUPS ? (R > 0 ? R : 1) : ATTNRES_P1BWD_GROUPS;
  const int64_t chunks = (grid + ATTNRES_BWD_CHUNK - 1) / ATTNRES_BWD_CHUNK;
  return align256((size_t)kP1BwdQ * grid * D * 4) + align256((size_t)kP1BwdQ * chunks * D * 4);
}

template <int NC, int SQ>
static hipError_t launch_p1bwd_q(const P1BwdParams& p, unsigned grid, const Launch& L) {
  const size_t lds = ((size_t)(SQ > 4 ? 1 : 2) * SQ * p.g.D + (size_t)2 * p.g.W * (2 * SQ + 1) * NC) * sizeof(float);
  return launch(L, phase1_bwd_kernel<NC, SQ>, dim3(grid), dim3(64 * p.g.W), lds, p);
}

template <int NC>
static hipError_t launch_p1bwd_t(const P1BwdParams& p, unsigned grid, const Launch& L) {
  switch (p.S) {
    case 1: return launch_p1bwd_q<NC, 1>(p, grid, L);
    case 2: return launch_p1bwd_q<NC, 2>(p, grid, L);
    case 3: return launch_p1bwd_q<NC, 3>(p, grid, L);
    case 4: return launch_p1bwd_q<NC, 4>(p, grid, L);
    case 5: return launch_p1bwd_q<NC, 5>(p, grid, L);
    case 6: return launch_p1bwd_q<NC, 6>(p, grid, L);
    case 7: return launch_p1bwd_q<NC, 7>(p, grid, L);
    default: return launch_p1bwd_q<NC, 8>(p, grid, L);
  }
}

hipError_t launch_phase1_bwd(const Phase1BwdArgs& a, void* ws, const Launch& L, const Launch& Lred) {
  if (!phase1_bwd_eligible(1, a.n, a.D) || a.S < 1 || a.S > kP1BwdQ) return hipErrorInvalidValue;
  if (a.R == 0) return hipSuccess;
  P1BwdParams p;
  for (int i = 0; i < kP1BwdMaxN; ++i) {
    p.src[i] = i < a.n ? a.src[i] : a.src[0];
    p.dV[i] = i < a.n ? a.dV[i] : nullptr;
  }
  p.n = a.n; p.S = a.S; p.eps = a.eps;
  for (int j = 0; j < kP1BwdQ; ++j) {
    const int jj = j < a.S ? j : 0;
    p.dh[j] = a.dh[jj];
    p.dh_scale[j] = j < a.S ? a.dh_scale[j] : nullptr;
    p.dlse[j] = j < a.S ? a.dlse[j] : nullptr;
    p.w[j] = a.w + (int64_t)jj * a.D;
    p.gm[j] = a.g ? a.g + (int64_t)jj * a.D : nullptr;
  }
  const unsigned grid = (unsigned)(a.R < ATTNRES_P1BWD_GROUPS ? a.R : ATTNRES_P1BWD_GROUPS);
  p.partial = static_cast<float*>(ws);
  p.g = make_geom(a.R, a.D, 4, kP1BwdVpl, 1);  // four-element vectors (V = D / 4)
  p.g.RPW = 1;
  p.g.groups = a.R;
  hipError_t e;
  switch (a.n) {
    case 1: e = launch_p1bwd_t<1>(p, grid, L); break;
    case 2: e = launch_p1bwd_t<2>(p, grid, L); break;
    case 3: e = launch_p1bwd_t<3>(p, grid, L); break;
    case 4: e = launch_p1bwd_t<4>(p, grid, L); break;
    case 5: e = launch_p1bwd_t<5>(p, grid, L); break;
    case 6: e = launch_p1bwd_t<6>(p, grid, L); break;
    case 7: e = launch_p1bwd_t<7>(p, grid, L); break;
    default: e = launch_p1bwd_t<8>(p, grid, L); break;
  }
  if (e != hipSuccess) return e;
  // each query's partial rows [grid][D] -> dw, dgamma (written or added)
  float* stage1 = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)kP1BwdQ * grid * a.D * 4));
  const unsigned bx = (unsigned)((a.D / 4 + 255) / 256);
  const int64_t chunk = ATTNRES_BWD_CHUNK;
  const int64_t P2 = grid > chunk ? ((int64_t)grid + chunk - 1) / chunk : 0;
  // every query in one launch per stage (blockIdx.z = query), timed from the
  // first stage's start to the second's end
  unsigned mask = 0;
  for (int j = 0; j < a.S; ++j) mask |= (a.accumulate_q[j] ? 1u : 0u) << j;
  const int64_t qpart = (int64_t)grid * a.D;
  if (P2) {
    e = launch(Launch{Lred.stream, Lred.start, nullptr}, bwd_colsum_kernel<false>, dim3(bx, (unsigned)P2, a.S),
               dim3(256), 0, (const float*)p.partial, (int64_t)grid, a.D, chunk, stage1, (const float*)nullptr,
               (const float*)nullptr, (float*)nullptr, (float*)nullptr, 0u, qpart, P2 * a.D);
    if (e != hipSuccess) return e;
  }
  const float* in = P2 ? stage1 : p.partial;
  const int64_t rows = P2 ? P2 : grid;
  return launch(Launch{Lred.stream, P2 ? nullptr : Lred.start, Lred.stop}, bwd_colsum_kernel<true>,
                dim3(bx, 1, a.S), dim3(256), 0, in, rows, a.D, rows, (float*)nullptr, a.w, a.g, a.dw, a.dgamma,
                mask, P2 ? P2 * a.D : qpart, (int64_t)0);
}

template <class F, int VPL>
static hipError_t launch_merge_bwd_t(const MergeBwdParams& p, unsigned grid, const Launch& L) {
  const size_t lds = p.g.W > 1 ? (size_t)p.g.RPW * p.g.W * 4 * sizeof(float) : 0;
  return launch(L, merge_bwd_kernel<F, VPL>, dim3(grid), dim3(64 * p.g.W * p.g.RPW), lds, p);
}

template <class F, int SMALL>
static hipError_t launch_merge_bwd_dt(const MergeBwdArgs& a, const BwdPlan& pl, const Launch& L) {
  MergeBwdParams p;
  p.o = a.o; p.lse = a.lse; p.ps = a.ps; p.w = a.w; p.gm = a.g; p.eps = a.eps; p.dh = a.dh;
  p.g_in = a.g_in; p.g_out = a.g_out; p.a_out = a.a_out; p.dlse_out = a.dlse_out;
  p.partial = static_cast<float*>(a.workspace);
  int vpl = 0;
  p.g = bwd_geom(F::kBytes == 8 ? 1 : 0, a.R, a.D, &vpl);
  if (vpl == SMALL) return launch_merge_bwd_t<F, SMALL>(p, pl.grid, L);
  if (vpl == 2 * SMALL) return launch_merge_bwd_t<F, 2 * SMALL>(p, pl.grid, L);
  if constexpr (SMALL * 4 <= 8) {
    if (vpl == 4 * SMALL) return launch_merge_bwd_t<F, 4 * SMALL>(p, pl.grid, L);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge_bwd(int dtype, const MergeBwdArgs& a, const BwdPlan& pl, const Launch& L) {
  if (pl.grid == 0) return hipSuccess;
  return dtype == 1 ? launch_merge_bwd_dt<Bf16x4, ATTNRES_BWD_BF16_VPL>(a, pl, L)
                    : launch_merge_bwd_dt<F32x4, ATTNRES_BWD_F32_VPL>(a, pl, L);
}

}  // namespace attnres
