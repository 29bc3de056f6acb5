// Device-side helpers shared by the gfx950 kernels of liblf_attn: element loads and stores for the two
// input types, and the fp32 MFMA tile used by every matrix product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its uint16_t bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(static_cast<uint32_t>(x.bits) << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

// float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    r.bits = static_cast<uint16_t>((u >> 16) | 0x40u);
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = static_cast<uint16_t>(u >> 16);
  }
  return r;
}

// One 16x16x4 fp32 MFMA step: acc += A(16x4) * B(4x16).
// Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; the 16x16 accumulator lives in lane l as rows
// 4*(l/16) + {0,1,2,3} of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Four consecutive elements as float4 (16-byte aligned for float, 8-byte aligned for bf16).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16_t* p, float4 v) {
  const bf16_t a = from_f32<bf16_t>(v.x), b = from_f32<bf16_t>(v.y), c = from_f32<bf16_t>(v.z),
               d = from_f32<bf16_t>(v.w);
  uint2 u;
  u.x = static_cast<uint32_t>(a.bits) | (static_cast<uint32_t>(b.bits) << 16);
  u.y = static_cast<uint32_t>(c.bits) | (static_cast<uint32_t>(d.bits) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

// Barrier for data exchanged through LDS only: waits for this wave's LDS operations, not for its global loads and
// stores (the fence of __syncthreads() also drains those, so a store or prefetch in flight would cost its full
// latency at every barrier of a loop).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

}  // namespace lf
