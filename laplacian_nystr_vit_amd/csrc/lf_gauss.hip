// Gaussian-kernel variant of the similarity step: C[i][l] = exp(-||x_i - L_l||_2^2 / lambda) for the rows x of
// Q and K, and W_eps = k(L, L) + eps I. The papernotes.org LaplacianFormer note sets this kernel against the
// Laplacian one: its motivation section says the Gaussian kernel of earlier linear attentions decays with the
// squared l2 distance, and its key findings open with swapping that kernel for the Laplacian one. Everything
// after the kernel (landmarks, eps shift, Newton-Schulz, whitening, products, DWC) is shared with the Laplacian
// path.
//
// Unlike the l1 distance, the squared l2 distance is a dense contraction plus two norms:
//   ||x - l||^2 = ||x||^2 + ||l||^2 - 2 x.l,
// so the cross-kernels run on MFMA. x.l is formed from split fp16 operands, x = x_hi + x_lo with
// x_hi = fp16(x) and x_lo = fp16(x - x_hi), as x_hi.l_hi + x_hi.l_lo + x_lo.l_hi on v_mfma_f32_16x16x32_f16 with
// fp32 accumulation: about 22 bits of each operand, three fp16 MFMAs at a fifth of the issue time of the fp32 MFMA
// product. Rows and landmarks are scaled by powers of two (largest entry near 2^12) so that the halves stay clear
// of fp16 overflow and subnormals; the scales come back out exactly in the epilogue. The landmark kernel W is
// computed from the differences themselves on the VALU:
// it is tiny (m^2 d per slice), and (a - b)^2 == (b - a)^2 in float32 makes W bitwise symmetric with an exact
// zero distance on its diagonal, which Newton-Schulz relies on.
#include <hip/hip_runtime.h>

#include <climits>

#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

typedef _Float16 gh8 __attribute__((ext_vector_type(8)));
typedef float gf8 __attribute__((ext_vector_type(8)));

// Exponent e of |v| = f 2^e, f in [1, 2), for v != 0 (subnormals count as 2^-126); the scale exponent of a row or
// landmark whose largest entry is mx puts that entry in [2^12, 2^13).
__device__ __forceinline__ int scale_exp(float mx) {
  if (!(mx > 0.f)) return 0;
  const int bexp = static_cast<int>((__float_as_uint(mx) >> 23) & 0xffu);
  return (bexp == 0 ? 1 : bexp) - 127 - 12;
}

// v 2^-e split into fp16 halves, eight values.
__device__ __forceinline__ void split8(gf8 v, int e, gh8& h, gh8& l) {
  gf8 sv;
#pragma unroll
  for (int t = 0; t < 8; ++t) sv[t] = ldexpf(v[t], -e);
  h = __builtin_convertvector(sv, gh8);
  l = __builtin_convertvector(sv - __builtin_convertvector(h, gf8), gh8);
}

// Grid: pairblocks blocks of 256 landmark pairs, then G * (tilesQ + tilesK) row blocks of 64 rows.
// Row block (4 waves): the block stages its 64 rows of one source (Q or K) of one slice in LDS with coalesced
// 16-byte loads, together with their squared norms and scale exponents. Wave w then takes the 16-landmark tiles
// w, w + 4, ... and, for each, all four 16-row tiles: four independent MFMA accumulation chains that share one
// landmark operand. In the 16x16x32 fp16 MFMA, lane (r16, q) = (lane % 16, lane / 16) supplies channels
// 32c + 8q .. 32c + 8q + 7 of chunk c, of row r16 of a row tile (A, from LDS) and of landmark r16 of the landmark
// tile (B, read straight from L2: one slice's landmarks are m*D*4 bytes). The accumulator of lane (r16, q) holds
// x.l for rows 4q + {0..3} of the row tile and landmark r16: rescaling, adding the two norms and one v_exp_f32
// give four consecutive tokens of one landmark column, stored as one 16-byte write into the landmark-major C.
template <typename T, int D>
__global__ __launch_bounds__(256, D <= 64 ? 4 : 2) void k_gauss(const T* __restrict__ Q, const T* __restrict__ K,
                                               const float* __restrict__ L, float* __restrict__ CQ,
                                               float* __restrict__ CK, float* __restrict__ We, int N, int m,
                                               int tilesQ, int tilesK, int rowblocks, int pairblocks, long npairs,
                                               float scale, float eps) {
  constexpr int CPL = D / 4;             // channels per thread in the norm pass
  constexpr int KC = (D + 31) / 32;      // 32-channel MFMA chunks (D = 16 pads its chunk with zeros)
  constexpr int LDX = D + 4;             // LDS row stride: 16 rows at one column offset hit distinct banks
  __shared__ float sX[64 * LDX];
  __shared__ float sN[64];
  __shared__ int sE[64];
  // Blocks [0, pairblocks) (a multiple of 8) form W, spread over all XCDs; the row blocks follow, remapped so that
  // consecutive row blocks run on one XCD (blocks are dealt to the 8 XCDs round-robin) and a slice's row blocks
  // share its landmarks through one L2.
  const int hw = static_cast<int>(blockIdx.x);
  if (hw < pairblocks) {
    // Landmark pairs: W[g][l][l2] = exp(-sum_c (L_lc - L_l2c)^2 / lambda) + eps [l == l2].
    const long e = static_cast<long>(hw) * 256 + threadIdx.x;
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
  int b = hw - pairblocks;
  {
    const int full = (rowblocks / 8) * 8;
    if (b < full) b = (b % 8) * (full / 8) + b / 8;
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
    // Squared norm and largest |x| of row tid / 4 from its four channel quarters, summed in a fixed order.
    const float* src = sX + (tid >> 2) * LDX + (tid & 3) * CPL;
    float p = 0.f, mx = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + c);
      p = fmaf(v.x, v.x, p);
      p = fmaf(v.y, v.y, p);
      p = fmaf(v.z, v.z, p);
      p = fmaf(v.w, v.w, p);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    p += __shfl_xor(p, 1);
    p += __shfl_xor(p, 2);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    if ((tid & 3) == 0) {
      sN[tid >> 2] = p;
      sE[tid >> 2] = scale_exp(mx);
    }
  }
  __syncthreads();

  const int ntiles = (m + 15) >> 4;
  if (w >= ntiles) return;
  // A operands: the lane's channels of row rt*16 + r16 in each chunk, scaled by the row's exponent and split.
  gh8 ah[4][KC], al[4][KC];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = rt * 16 + r16;
    const int er = sE[row];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k0 = c * 32 + 8 * q;
      gf8 v;
      if (k0 < D) {
        const float4 u0 = *reinterpret_cast<const float4*>(sX + row * LDX + k0);
        const float4 u1 = *reinterpret_cast<const float4*>(sX + row * LDX + k0 + 4);
        v = gf8{u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      } else {
        v = gf8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      }
      split8(v, er, ah[rt][c], al[rt][c]);
    }
  }
  const bool vec = (N & 3) == 0;
  const float* __restrict__ Lg = L + static_cast<size_t>(g) * m * D;
  float* __restrict__ Cg = (isq ? CQ : CK) + static_cast<size_t>(g) * m * N;

  for (int lt = w; lt < ntiles; lt += 4) {
    gf8 lv[KC];
    {
      const float* __restrict__ src = Lg + static_cast<size_t>(min(lt * 16 + r16, m - 1)) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int k0 = c * 32 + 8 * q;
        if (k0 < D) {
          const float4 u0 = load4(src + k0), u1 = load4(src + k0 + 4);
          lv[c] = gf8{u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        } else {
          lv[c] = gf8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    float ln = 0.f, lm = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        ln = fmaf(lv[c][t], lv[c][t], ln);
        lm = fmaxf(lm, fabsf(lv[c][t]));
      }
    ln += __shfl_xor(ln, 16);
    ln += __shfl_xor(ln, 32);  // ||L_{lt*16 + r16}||^2, identical bits in the four lanes of landmark r16
    lm = fmaxf(lm, __shfl_xor(lm, 16));
    lm = fmaxf(lm, __shfl_xor(lm, 32));
    const int el = scale_exp(lm);
    gh8 bh[KC], bl[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) split8(lv[c], el, bh[c], bl[c]);

    f32x4 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][c], bh[c], acc[rt], 0, 0, 0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][c], bl[c], acc[rt], 0, 0, 0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rt][c], bh[c], acc[rt], 0, 0, 0);
    }

    const int l = lt * 16 + r16;
    if (l < m) {
      float* __restrict__ dst = Cg + static_cast<size_t>(l) * N;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int rb = i0 + rt * 16 + 4 * q;  // first of this lane's four rows in this row tile
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // norm and scale exponent of row rt*16 + 4q + j, the row this accumulator element belongs to
          const int row = rt * 16 + 4 * q + j;
          const float dot = ldexpf(acc[rt][j], sE[row] + el);
          const float d2 = fmaxf(fmaf(-2.f, dot, sN[row] + ln), 0.f);
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
  const long pairblocks = ((npairs + 255) / 256 + 7) / 8 * 8;  // a multiple of 8 keeps the row blocks' XCD order
  const long blocks = rowblocks + pairblocks;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  hipLaunchKernelGGL((k_gauss<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), L, CQ, CK, We, s.N, s.m,
                     static_cast<int>(tilesN), static_cast<int>(tilesN), static_cast<int>(rowblocks),
                     static_cast<int>(pairblocks), npairs, scale, s.eps);
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
