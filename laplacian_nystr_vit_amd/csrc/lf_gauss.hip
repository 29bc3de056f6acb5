// Gaussian-kernel variant of the similarity step: C[i][l] = exp(-||x_i - L_l||_2^2 / lambda) for the rows x of
// Q and K, and W_eps = k(L, L) + eps I. The papernotes.org LaplacianFormer note sets this kernel against the
// Laplacian one: its motivation section says the Gaussian kernel of earlier linear attentions decays with the
// squared l2 distance, and its key findings open with swapping that kernel for the Laplacian one. Everything
// after the kernel (landmarks, eps shift, Newton-Schulz, whitening, products, DWC) is shared with the Laplacian
// path.
//
// Unlike the l1 distance, the squared l2 distance is a dense contraction plus two norms:
//   ||x - l||^2 = ||x||^2 + ||l||^2 - 2 x.l,
// so the cross-kernels run on fp32 MFMA (v_mfma_f32_16x16x4_f32), which issues twice the fp32 work per cycle of a
// VALU difference-and-square loop. The landmark kernel W is computed from the differences themselves on the VALU:
// it is tiny (m^2 d per slice), and (a - b)^2 == (b - a)^2 in float32 makes W bitwise symmetric with an exact
// zero distance on its diagonal, which Newton-Schulz relies on.
#include <hip/hip_runtime.h>

#include <climits>

#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

// Grid: G * (tilesQ + tilesK) row blocks of 64 rows, then wblocks blocks of 256 landmark pairs.
// Row block (4 waves): the block stages its 64 rows of one source (Q or K) of one slice in LDS with coalesced
// 16-byte loads, together with their squared norms. Wave w then takes the 16-landmark tiles w, w + 4, ... and, for
// each, all four 16-row tiles: four independent MFMA accumulation chains that share one landmark operand. Lane
// (r16, q) = (lane % 16, lane / 16) supplies channels [q D/4, (q+1) D/4) of row r16 of a row tile and of landmark
// r16 of the landmark tile (read straight from L2: one slice's landmarks are m*D*4 bytes); in MFMA step t, k-slot
// q carries channel q D/4 + t for both operands, so no cross-lane exchange feeds the contraction. The accumulator
// of lane (r16, q) holds x.l for rows 4q + {0..3} of the row tile and landmark r16: adding the two norms and one
// v_exp_f32 gives four consecutive tokens of one landmark column, stored as one 16-byte write into the
// landmark-major C.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_gauss(const T* __restrict__ Q, const T* __restrict__ K,
                                               const float* __restrict__ L, float* __restrict__ CQ,
                                               float* __restrict__ CK, float* __restrict__ We, int N, int m,
                                               int tilesQ, int tilesK, int rowblocks, long npairs, float scale,
                                               float eps) {
  constexpr int CPL = D / 4;  // channels per lane
  constexpr int LDX = D + 4;  // LDS row stride: 16 lanes reading one column offset of 16 rows hit distinct banks
  __shared__ float sX[64 * LDX];
  __shared__ float sN[64];
  int b = static_cast<int>(blockIdx.x);
  {
    // Consecutive blocks on one XCD (blocks are dealt to the 8 XCDs round-robin): a slice's row blocks then share
    // its landmarks through one L2.
    const int full = (static_cast<int>(gridDim.x) / 8) * 8;
    if (b < full) b = (b % 8) * (full / 8) + b / 8;
  }
  if (b >= rowblocks) {
    // Landmark pairs: W[g][l][l2] = exp(-sum_c (L_lc - L_l2c)^2 / lambda) + eps [l == l2].
    const long e = static_cast<long>(b - rowblocks) * 256 + threadIdx.x;
    if (e >= npairs) return;
    const long mm = static_cast<long>(m) * m;
    const int g = static_cast<int>(e / mm);
    const int rem = static_cast<int>(e - static_cast<long>(g) * mm);
    const int l = rem / m, l2 = rem - l * m;
    const float* __restrict__ a = L + (static_cast<size_t>(g) * m + l) * D;
    const float* __restrict__ c = L + (static_cast<size_t>(g) * m + l2) * D;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int k = 0; k < D; k += 4) {
      const float4 u = load4(a + k), v = load4(c + k);
      const float d0 = u.x - v.x, d1 = u.y - v.y, d2 = u.z - v.z, d3 = u.w - v.w;
      s0 = fmaf(d0, d0, s0);
      s1 = fmaf(d1, d1, s1);
      s2 = fmaf(d2, d2, s2);
      s3 = fmaf(d3, d3, s3);
    }
    float val = __builtin_amdgcn_exp2f(((s0 + s1) + (s2 + s3)) * scale);
    if (l == l2) val += eps;
    We[e] = val;
    return;
  }

  const int per_slice = tilesQ + tilesK;
  const int g = b / per_slice;
  const int local = b - g * per_slice;
  const bool isq = local < tilesQ;
  const int tile = isq ? local : local - tilesQ;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = lane_id(), r16 = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int i0 = tile * 64;  // first row of the block
  const T* __restrict__ xg = (isq ? Q : K) + static_cast<size_t>(g) * N * D;

  // Stage the 64 rows (rows past N read as zero and are never stored).
  for (int e = tid; e < 16 * D; e += 256) {
    const int r = e / (D / 4), c4 = e - r * (D / 4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + r < N) v = load4(xg + static_cast<size_t>(i0 + r) * D + 4 * c4);
    *reinterpret_cast<float4*>(sX + r * LDX + 4 * c4) = v;
  }
  __syncthreads();
  {
    // Squared norm of row tid / 4 from its four channel quarters, summed in a fixed order.
    const float* src = sX + (tid >> 2) * LDX + (tid & 3) * CPL;
    float p = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + c);
      p = fmaf(v.x, v.x, p);
      p = fmaf(v.y, v.y, p);
      p = fmaf(v.z, v.z, p);
      p = fmaf(v.w, v.w, p);
    }
    p += __shfl_xor(p, 1);
    p += __shfl_xor(p, 2);
    if ((tid & 3) == 0) sN[tid >> 2] = p;
  }
  __syncthreads();

  const int ntiles = (m + 15) >> 4;
  if (w >= ntiles) return;
  // A operands: channels [q CPL, (q+1) CPL) of row rt*16 + r16, for the four row tiles.
  float xa[4][CPL];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(sX + (rt * 16 + r16) * LDX + q * CPL + c);
      xa[rt][c] = v.x;
      xa[rt][c + 1] = v.y;
      xa[rt][c + 2] = v.z;
      xa[rt][c + 3] = v.w;
    }
  // Norms of the rows each accumulator element belongs to: row rt*16 + 4q + j.
  float xr[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) xr[rt][j] = sN[rt * 16 + 4 * q + j];
  const bool vec = (N & 3) == 0;
  const float* __restrict__ Lg = L + static_cast<size_t>(g) * m * D;
  float* __restrict__ Cg = (isq ? CQ : CK) + static_cast<size_t>(g) * m * N;

  for (int lt = w; lt < ntiles; lt += 4) {
    float lb[CPL];
    {
      const float* __restrict__ src = Lg + static_cast<size_t>(min(lt * 16 + r16, m - 1)) * D + q * CPL;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        const float4 v = load4(src + c);
        lb[c] = v.x;
        lb[c + 1] = v.y;
        lb[c + 2] = v.z;
        lb[c + 3] = v.w;
      }
    }
    float ln = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) ln = fmaf(lb[c], lb[c], ln);
    ln += __shfl_xor(ln, 16);
    ln += __shfl_xor(ln, 32);  // ||L_{lt*16 + r16}||^2, identical bits in the four lanes of landmark r16

    f32x4 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < CPL; ++t)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma16x16x4(xa[rt][t], lb[t], acc[rt]);

    const int l = lt * 16 + r16;
    if (l < m) {
      float* __restrict__ dst = Cg + static_cast<size_t>(l) * N;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int rb = i0 + rt * 16 + 4 * q;  // first of this lane's four rows in this row tile
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d2 = fmaxf(fmaf(-2.f, acc[rt][j], xr[rt][j] + ln), 0.f);
          o[j] = __builtin_amdgcn_exp2f(d2 * scale);
        }
        if (vec && rb + 3 < N) {
          store4(dst + rb, make_float4(o[0], o[1], o[2], o[3]));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (rb + j < N) dst[rb + j] = o[j];
        }
      }
    }
  }
}

template <typename T, int D>
static hipError_t gauss_t(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                          float* We, hipStream_t st) {
  const long tilesN = (static_cast<long>(s.N) + 63) / 64;
  const long rowblocks = static_cast<long>(s.G) * 2 * tilesN;
  const long npairs = static_cast<long>(s.G) * s.m * s.m;
  const long blocks = rowblocks + (npairs + 255) / 256;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  hipLaunchKernelGGL((k_gauss<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), L, CQ, CK, We, s.N, s.m,
                     static_cast<int>(tilesN), static_cast<int>(tilesN), static_cast<int>(rowblocks), npairs, scale,
                     s.eps);
  return hipGetLastError();
}

template <typename T>
static hipError_t gauss_d(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                          float* We, hipStream_t st) {
  switch (s.d) {
    case 16: return gauss_t<T, 16>(s, Q, K, L, CQ, CK, We, st);
    case 32: return gauss_t<T, 32>(s, Q, K, L, CQ, CK, We, st);
    case 64: return gauss_t<T, 64>(s, Q, K, L, CQ, CK, We, st);
    default: return gauss_t<T, 128>(s, Q, K, L, CQ, CK, We, st);
  }
}

hipError_t launch_gauss(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                        float* We, hipStream_t st) {
  return s.dtype == 1 ? gauss_d<bf16_t>(s, Q, K, L, CQ, CK, We, st) : gauss_d<float>(s, Q, K, L, CQ, CK, We, st);
}

}  // namespace lf
