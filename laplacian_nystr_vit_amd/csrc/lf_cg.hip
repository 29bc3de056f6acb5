// Conjugate gradients for W_eps X = I (m <= 64): the solver the Newton-Schulz iteration is compared against
// (LaplacianFormer reading note, Design 3 and the solver row of the ablation table).
//
// Every column j of X is an independent CG solve of W_eps x = e_j from x = 0. One block per slice, one wave per
// strip of 16 columns; a wave never talks to another wave until the optional residual reduction at the end.
//
// Layout. A wave keeps its strip of X, of the residual R and of the direction P in registers, in the accumulator
// layout of the 16x16x4 fp32 MFMA: row tile a (rows 16a .. 16a+15), lane (q = lane/16, c = lane%16) holds rows
// 16a + 4q + {0,1,2,3} of column c. W_eps is read once into registers as the A operand.
//
// Contraction order. k-step t (0..15) of a product W*P takes column index k = 16*(t/4) + 4q + t%4 from lane group
// q. With that order the B operand that lane (q, c) must supply at step t, P[k][c], is exactly the accumulator
// element it holds (row tile t/4, element t%4): the product needs neither LDS nor cross-lane moves. Steps whose
// smallest k is >= m and row tiles starting at >= m are skipped (their operands are zero).
//
// Per-column scalars (p.Wp, r.r) are sums over the 64 rows of a column: each lane sums its 16 rows, then two xor
// shuffles across the lane groups; addition being commutative, all four groups get the same bits.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {
namespace {

constexpr int kCgWaves = 4;

__device__ __forceinline__ float group_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float col_dot(const f32x4 u[4], const f32x4 v[4]) {
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a) s += u[a][0] * v[a][0] + u[a][1] * v[a][1] + u[a][2] * v[a][2] + u[a][3] * v[a][3];
  return group_sum(s);
}

// acc = W * M over the wave's column strip, M in accumulator layout (see the file comment).
__device__ __forceinline__ void strip_product(const float wa[4][16], const f32x4 M[4], f32x4 acc[4], int m) {
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (16 * (t >> 2) + (t & 3) >= m) continue;  // every k of this step is >= m
    const float b = M[t >> 2][t & 3];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (16 * a < m) acc[a] = mfma16x16x4(wa[a][t], b, acc[a]);
  }
}

__global__ __launch_bounds__(kCgWaves * 64) void k_cg(const float* __restrict__ We, float* __restrict__ Xout,
                                                     float* __restrict__ resid, int m, int iters) {
  __shared__ float sres[kCgWaves][kCgItersMax];
  const int g = blockIdx.x;
  const int ln = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int q = ln >> 4;
  const int c = 16 * wv + (ln & 15);
  const float* W = We + static_cast<size_t>(g) * m * m;

  if (resid && 16 * wv >= m)  // a wave without columns contributes zeros; an active wave writes every step
    for (int k = ln; k < iters; k += 64) sres[wv][k] = 0.f;

  if (16 * wv < m) {
    float wa[4][16];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int row = 16 * a + (ln & 15);
        const int k = 16 * (t >> 2) + 4 * q + (t & 3);
        const bool in = row < m && k < m;
        const float v = W[in ? row * m + k : 0];
        wa[a][t] = in ? v : 0.f;
      }

    f32x4 x[4], r[4], p[4], acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * a + 4 * q + e;
        x[a][e] = 0.f;
        r[a][e] = (row == c && c < m) ? 1.f : 0.f;
        p[a][e] = r[a][e];
      }
    float rr = c < m ? 1.f : 0.f;

    for (int it = 0; it < iters; ++it) {
      strip_product(wa, p, acc, m);  // acc = W p
      const float pq = col_dot(p, acc);
      const float step = rr > 0.f ? rr / (pq != 0.f ? pq : 1.f) : 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        x[a] = x[a] + p[a] * step;
        r[a] = r[a] - acc[a] * step;
      }
      const float rn = col_dot(r, r);
      const float beta = rr > 0.f ? rn / rr : 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) p[a] = r[a] + p[a] * beta;
      rr = rn;

      if (resid) {  // ||W x - I||^2 over this strip, from x itself
        strip_product(wa, x, acc, m);
        float s = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * a + 4 * q + e;
            const float ev = acc[a][e] - ((row == c && c < m) ? 1.f : 0.f);
            s += ev * ev;
          }
        s = group_sum(s);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 8, 64);
        if (ln == 0) sres[wv][it] = s;
      }
    }

    float* X = Xout + static_cast<size_t>(g) * m * m;
    if (c < m)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * a + 4 * q + e;
          if (row < m) X[row * m + c] = x[a][e];
        }
  }

  if (resid) {
    __syncthreads();
    for (int k = threadIdx.x; k < iters; k += blockDim.x)
      resid[static_cast<size_t>(g) * iters + k] = sqrtf((sres[0][k] + sres[1][k]) + (sres[2][k] + sres[3][k]));
  }
}

}  // namespace

bool cg_supported(const Shape& s) { return s.m >= 1 && s.m <= 64; }

hipError_t launch_cg(const Shape& s, const float* We, float* X, float* resid, int iters, hipStream_t st) {
  if (s.G == 0) return hipSuccess;
  hipLaunchKernelGGL(k_cg, dim3(s.G), dim3(kCgWaves * 64), 0, st, We, X, resid, s.m, iters);
  return hipGetLastError();
}

}  // namespace lf
