// gen.hip -- seeded synthetic inputs for tests and benchmarks (libattnres_inputs.so).
//
// This module holds no AttnRes arithmetic. It fills device tensors with
// counter-based pseudo-random normals, gathers token rows, and provides
// sublayer callbacks that hand pre-generated or freshly generated sublayer
// outputs to attnres_block_stack_forward. The same generator is written out in
// numpy in inputs/__init__.py (the CPU twin).
//
// Generator (every operation mod 2^64):
//   mix64(z)   = SplitMix64 output function (Steele, Lea & Flood, "Fast
//                splittable pseudorandom number generators", OOPSLA 2014):
//                z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
//                z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
//   key        = mix64(seed * G + mix64(role << 32 | layer)),  G = 0x9E3779B97F4A7C15
//   bits(i)    = mix64(key + (i + 1) * G)     for element index i = row * D + col
//   u1 = ((bits >> 40) + 1) / 2^24 in (0, 1],  u2 = ((bits >> 16) & 0xFFFFFF) / 2^24
//   z  = sqrt(-2 ln u1) * cos(2 pi u2)        (Box-Muller, fp64)
//   value = round-to-nearest-even(scale * z) in the tensor dtype.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "inputs.h"

#define INPUTS_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint32_t role, uint32_t layer) {
  return mix64(seed * kGolden + mix64(((uint64_t)role << 32) | layer));
}

__device__ inline double normal_at(uint64_t key, uint64_t idx) {
  const uint64_t b = mix64(key + (idx + 1) * kGolden);
  const double u1 = (double)((b >> 40) + 1) * 0x1p-24;
  const double u2 = (double)((b >> 16) & 0xFFFFFFull) * 0x1p-24;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

// nearest-even rounding of a double to bf16, on the bit pattern
__device__ inline uint16_t bf16_rne(double x) {
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48);  // signed zero
  uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = b >> 63;
  b &= 0x7FFFFFFFFFFFFFFFull;
  b += (1ull << 44) - 1 + ((b >> 45) & 1);
  const int e = (int)(b >> 52) - 1023 + 127;
  const uint32_t mant = (uint32_t)(b >> 45) & 0x7F;
  return (uint16_t)((sign << 15) | ((uint32_t)e << 7) | mant);
}

// Fill rows of a [rows, D] tensor; row r of dst holds generated row ids[r]
// (or r when ids is null). One thread per 16-byte vector.
__global__ void fill_normal_kernel(void* __restrict__ dst, int dtype, int64_t rows, int64_t D,
                                   const int64_t* __restrict__ ids, uint64_t key, double scale) {
  const int epv = dtype == 1 ? 8 : 4;
  const int64_t vpr = D / epv;
  const int64_t nvec = rows * vpr;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / vpr;
    const int64_t col = (v - r * vpr) * epv;
    const int64_t grow = ids ? ids[r] : r;
    const uint64_t base = (uint64_t)(grow * D + col);
    uint32_t w[4];
    if (dtype == 1) {
      for (int k = 0; k < 4; ++k) {
        const uint16_t lo = bf16_rne(scale * normal_at(key, base + 2 * k));
        const uint16_t hi = bf16_rne(scale * normal_at(key, base + 2 * k + 1));
        w[k] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
    } else {
      for (int k = 0; k < 4; ++k) w[k] = __float_as_uint((float)(scale * normal_at(key, base + k)));
    }
    reinterpret_cast<uint4*>(dst)[v] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void gather_rows_kernel(void* __restrict__ dst, const void* __restrict__ src,
                                   const int64_t* __restrict__ ids, int64_t nrows,
                                   int64_t row_vecs) {
  const int64_t n = nrows * row_vecs;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / row_vecs, c = v - r * row_vecs;
    reinterpret_cast<uint4*>(dst)[v] = reinterpret_cast<const uint4*>(src)[ids[r] * row_vecs + c];
  }
}

unsigned blocks_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 16384 ? (b > 0 ? b : 1) : 16384);
}

}  // namespace

INPUTS_API int attnres_inputs_fill_normal(void* dst, int dtype, int64_t rows, int64_t D,
                                          const int64_t* row_ids, uint64_t seed, uint32_t role,
                                          uint32_t layer, double scale, void* stream) {
  if (!dst || (dtype != 0 && dtype != 1) || rows < 0 || D < 1) return -1;
  const int epv = dtype == 1 ? 8 : 4;
  if (D % epv) return -1;
  if (rows == 0) return 0;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(blocks_for(rows * (D / epv))), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dst, dtype, rows, D, row_ids,
                     stream_key(seed, role, layer), scale);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

INPUTS_API int attnres_inputs_gather_rows(void* dst, const void* src, const int64_t* row_ids,
                                          int64_t nrows, int64_t row_bytes, void* stream) {
  if (!dst || !src || !row_ids || nrows < 0 || row_bytes % 16) return -1;
  if (nrows == 0) return 0;
  const int64_t rv = row_bytes / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks_for(nrows * rv)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dst, src, row_ids, nrows, rv);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Sublayer callback: v_l = scales[l-1] * N(0,1), generated into ring slot l % 3.
INPUTS_API int attnres_inputs_ring_sublayer(void* ctx, int l, const void* h, const void** v_out,
                                            void* stream) {
  (void)h;
  attnres_inputs_ring* r = static_cast<attnres_inputs_ring*>(ctx);
  if (!r || !v_out || l < 1 || l > r->L) return 1;
  void* slot = r->slots[l % 3];
  if (attnres_inputs_fill_normal(slot, r->dtype, r->R, r->D, nullptr, r->seed, r->role,
                                 (uint32_t)l, r->scales[l - 1], stream) != 0)
    return 2;
  *v_out = slot;
  return 0;
}

// Sublayer callback that records rows of every h_l, then defers to an inner callback.
INPUTS_API int attnres_inputs_record_sublayer(void* ctx, int l, const void* h, const void** v_out,
                                              void* stream) {
  attnres_inputs_recorder* r = static_cast<attnres_inputs_recorder*>(ctx);
  if (!r || l < 1 || l > r->L) return 1;
  if (r->nrows > 0) {
    char* dst = static_cast<char*>(r->rec) + (int64_t)(l - 1) * r->nrows * r->row_bytes;
    if (attnres_inputs_gather_rows(dst, h, r->rows, r->nrows, r->row_bytes, stream) != 0) return 2;
  }
  return r->inner(r->inner_ctx, l, h, v_out, stream);
}
