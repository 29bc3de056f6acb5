// Split-fp16 helpers shared by the kernels that run fp32 products on the fp16 MFMA (gfx950): an fp32 value x is
// carried as x = hi + lo, two fp16 values (about 22 significant bits), and A B ~= A_hi B_hi + A_hi B_lo + A_lo B_hi
// with fp32 accumulation (v_mfma_f32_16x16x32_f16).
#pragma once

#include "lf_device.h"

namespace lf {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ short4v lds_read_tr(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Splits fp32 values into fp16 halves, two at a time: hi = round_f16(v) and lo = round_f16(v - hi) (v - hi is
// exact in fp32, so lo is its correctly rounded fp16 value). Written with vector conversions (a pack conversion
// for each half pair) so that the compiler sees every instruction and keeps the wait states MFMA results need.
__device__ __forceinline__ void split2(f32x2 v, half2v& h, half2v& l) {
  h = __builtin_convertvector(v, half2v);
  l = __builtin_convertvector(v - __builtin_convertvector(h, f32x2), half2v);
}

__device__ __forceinline__ void split4(f32x4 v, half4& h, half4& l) {
  half2v h0, l0, h1, l1;
  split2(f32x2{v[0], v[1]}, h0, l0);
  split2(f32x2{v[2], v[3]}, h1, l1);
  h = half4{h0[0], h0[1], h1[0], h1[1]};
  l = half4{l0[0], l0[1], l1[0], l1[1]};
}

// Largest exponent e of an fp32 value (v = f * 2^e, f in [1, 2)) for v > 0; -126 for 0 and subnormals.
__device__ __forceinline__ int exp_of(float v) {
  const int b = static_cast<int>((__float_as_uint(v) >> 23) & 0xffu);
  return (b == 0 ? 1 : b) - 127;
}

// Storage exponent for an iterate whose largest entry is about mx: entries land in [2^12, 2^13).
__device__ __forceinline__ int store_exp(float mx) { return mx > 0.f ? exp_of(mx) - 12 : 0; }

// Maximum over the wave of a non-negative value, returned wave-uniform: DPP steps inside each row of 16 lanes
// (quad swaps, then rotations by 4 and 8), then the four row results through scalar registers.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);  // non-negative floats order like their bit patterns
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false));   // quad_perm [1, 0, 3, 2]
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false));   // quad_perm [2, 3, 0, 1]
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false));  // row_ror:8
  const int a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const int c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return __int_as_float(max(max(a, b), max(c, d)));
}

// v * s split into fp16 halves (hi + lo), four values at a time.
__device__ __forceinline__ void split_scaled4(f32x4 a, float s, half4& h, half4& l) {
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = a[r] * s;
  split4(v, h, l);
}

}  // namespace lf
