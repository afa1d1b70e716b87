// device.hpp -- device-side building blocks of the AttnRes kernels (gfx950, wave64).
//
// Element formats, 16-byte vector memory access, and the row reductions every
// kernel needs: the score of a source is a dot product and a sum of squares
// over the whole hidden axis, so each token row ends in a reduction across the
// lanes (and waves) that hold its columns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16 element format: 8 elements per 16-byte vector, widened exactly to fp32,
// narrowed nearest-even by the hardware conversion (v_cvt_pk_bf16_f32).
struct Bf16 {
  static constexpr int kEPV = 8;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
  }
  // Exact widening of element e (0..7) of a vector.
  static __device__ __forceinline__ float elem(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

// fp32 element format: 4 elements per 16-byte vector.
struct F32 {
  static constexpr int kEPV = 4;
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  static __device__ __forceinline__ float elem(const uint4& v, int e) {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Streaming (non-temporal) 16-byte access for tensors touched once per
// kernel: the loads and stores carry the nt hint, so several concurrent
// [R,D] streams do not thrash the caches. Queries and gains use ld16/ldf4.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_stream(void* p, const uint4& v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// Four consecutive fp32 values (one 16-byte load).
__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// Sum of x over the 64 lanes of the wave, returned wave-uniform. Quad swaps and
// row rotations give every lane its 16-lane row sum; the two row broadcasts
// chain the rows into lane 63. All 64 lanes must be active. The summation
// order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float x) {
  x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x124, 0xF>(x);  // row_ror:4
  x = dpp_add<0x128, 0xF>(x);  // row_ror:8
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Reduce NV per-lane partial sums across the W waves that share a token row.
// Each wave reduces its lanes with wave_sum; lane 0 of each wave writes the
// wave's sums to `lds` ([slots][W][NV] floats, one slot per row handled by the
// workgroup). After a barrier, lane k of every wave sums entry k over the W
// waves in wave order and the totals are broadcast from lane k, so a lane
// reads W values instead of W x NV (for NV > 64 every lane sums every entry).
// Either way the order of the additions is the same. Must be reached by every
// thread of the workgroup (it contains barriers).
template <int NV>
__device__ __forceinline__ void row_reduce(float (&v)[NV], float* lds, int slot, int wave_in_row,
                                           int W) {
  #pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
  if (W == 1) return;
  float* base = lds + (size_t)slot * W * NV;
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    #pragma unroll
    for (int k = 0; k < NV; ++k) base[wave_in_row * NV + k] = v[k];
  }
  __syncthreads();
  if constexpr (NV <= 64) {
    float s = 0.f;
    if (lane < NV) {
      s = base[lane];
      for (int w = 1; w < W; ++w) s += base[w * NV + lane];
    }
    #pragma unroll
    for (int k = 0; k < NV; ++k)
      v[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), k));
  } else {
    #pragma unroll
    for (int k = 0; k < NV; ++k) {
      float s = base[k];
      for (int w = 1; w < W; ++w) s += base[w * NV + k];
      v[k] = s;
    }
  }
  __syncthreads();
}

}  // namespace attnres
