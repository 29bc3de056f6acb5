// Forward-pass kernels of the LaplacianFormer attention block for gfx950 (CDNA4).
//
// Citations: papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力"
// ([note] below), sections motivation ("core idea"), framework (flowchart), Design 1, Design 2 and Design 3.
#include <algorithm>
#include <cmath>

#include "lf_device.h"
#include "lf_laplace.h"
#include "lf_internal.h"
#include "lf_split.h"

namespace lf {

// =====================================================================================================
// landmark_pool: L[g][l][c] = (1/r^2) sum_{a,b<r} Q[g][(Y r + a) W + X r + b][c]      ([note] Design 2)
// Thread = (landmark, window row slot, 4 channels): it sums its window rows with independent 16-byte (fp32) or
// 8-byte (bf16) loads that are all in flight at once, and the window-row partials are added through LDS in a
// fixed order. `tpl` threads serve one landmark (d/4 channel quads x `slots` row slots), `lpb` landmarks a block.
// =====================================================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_landmark_pool(const T* __restrict__ Q, float* __restrict__ L, int G, int H,
                                                       int W, int d, int r, int m, int tpl, int lpb) {
  __shared__ float4 part[256];
  const int c4n = d >> 2;
  const int slots = tpl / c4n;
  const int t = threadIdx.x;
  const int ll = t / tpl, rem = t % tpl;
  const int slot = rem / c4n, c4 = rem % c4n;
  const size_t lin = static_cast<size_t>(blockIdx.x) * lpb + ll;
  const bool valid = ll < lpb && lin < static_cast<size_t>(G) * m;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  size_t g = 0;
  if (valid) {
    g = lin / m;
    const int l = static_cast<int>(lin % m);
    const int wr = W / r;
    const int Yb = l / wr, Xb = l % wr;
    const T* base = Q + g * static_cast<size_t>(H) * W * d + 4 * c4;
    for (int a = slot; a < r; a += slots) {
      const T* row = base + (static_cast<size_t>(Yb * r + a) * W + static_cast<size_t>(Xb) * r) * d;
#pragma unroll 8
      for (int b = 0; b < r; ++b) {
        const float4 v = load4(row + static_cast<size_t>(b) * d);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
  }
  part[t] = acc;
  __syncthreads();
  if (valid && slot == 0) {
    float4 s = part[t];
    for (int k = 1; k < slots; ++k) {
      const float4 v = part[t + k * c4n];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    const float inv = static_cast<float>(r * r);
    store4(L + lin * d + 4 * c4, make_float4(s.x / inv, s.y / inv, s.z / inv, s.w / inv));
  }
}

// laplace_l1_exp: the distance kernel (lf_laplace.h).
template <typename T, int D>
__global__ __launch_bounds__(512) void k_laplace(const T* __restrict__ Q, const T* __restrict__ K,
                                                 const float* __restrict__ L, float* __restrict__ CQ,
                                                 float* __restrict__ CK, float* __restrict__ We, int N, int m,
                                                 int tilesQ, int tilesK, int tilesL, int nsc, int lc, float scale,
                                                 float eps) {
  __shared__ __attribute__((aligned(16))) float sX[kLaplaceLds<D> / 4];
  laplace_block<T, D>(sX, static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x),
                      static_cast<int>(blockDim.x) >> 6, Q, K, L, CQ, CK, We, N, m, tilesQ, tilesK, tilesL, nsc, lc,
                      scale, eps);
}

// =====================================================================================================
// whiten_stats: per landmark column of C_Q, mean and 1/sqrt(biased variance + eps_w) over the N tokens
//   ([note] Design 1, diagonal whitening). One block per (landmark, slice): the column is one contiguous row of the
//   landmark-major C_Q. Two passes in float64, fixed reduction order.
// =====================================================================================================
__device__ __forceinline__ double block_sum256(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_whiten_stats(const float* __restrict__ CQ, float* __restrict__ mu,
                                                      float* __restrict__ rstd, int N, int m, float weps) {
  __shared__ double red[4];
  const int l = blockIdx.x, g = blockIdx.y;
  const float* c = CQ + (static_cast<size_t>(g) * m + l) * N;
  double s = 0.0;
  for (int i = threadIdx.x; i < N; i += 256) s += static_cast<double>(c[i]);
  const double mean = block_sum256(s, red) / static_cast<double>(N);
  double v = 0.0;
  for (int i = threadIdx.x; i < N; i += 256) {
    const double dd = static_cast<double>(c[i]) - mean;
    v += dd * dd;
  }
  const double var = block_sum256(v, red) / static_cast<double>(N);
  if (threadIdx.x == 0) {
    mu[static_cast<size_t>(g) * m + l] = static_cast<float>(mean);
    rstd[static_cast<size_t>(g) * m + l] = static_cast<float>(1.0 / sqrt(var + static_cast<double>(weps)));
  }
}

// LDS leading dimension that is 16 mod 32 floats: rows k and k+1 of an MFMA B-style read (lanes 0-15 on row k,
// lanes 16-31 on row k+1) land in disjoint bank halves.
__host__ __device__ inline int ld_b(int cols) { return ((cols + 31) / 32) * 32 + 16; }

// =====================================================================================================
// ckv_reduce: S[g][l][c] = sum_i C_K[g][i][l] V[g][i][c], deterministic split-N reduction
//   ([note] motivation: linear attention forms K^T V first; Design 2).
// Stage 1: each block reduces `rows_per_split` token rows of one slice into a partial [mout][D] on the fp16 MFMA
// in split form (M = landmarks, N = channels, K = tokens), staging 64-row chunks of C and V through LDS as fp16
// halves, each chunk of each operand scaled by a power of two from its largest entry (undone exactly per chunk). With more than 64
// landmarks the landmarks are split over blocks too (64 per block), so that each split covers more rows and the
// partials stay small next to the C_K bytes they summarise.
// Stage 2: the partials are summed in split order.
// `ones` appends a column of ones to C (mout = mrow + 1), so row mrow of the result is sum_i V[i][c]; the
// backward pass uses this to get the column sums of dY in the same sweep as C_Q^T dY.
// =====================================================================================================
template <typename T, int D, int MT>
__global__ __launch_bounds__(256) void k_ckv_partial(const float* __restrict__ C, const T* __restrict__ V,
                                                     float* __restrict__ part, int N, int mrow, int ones,
                                                     int nsplit, int rows_per_split, int lsplit) {
  // LDS, as fp16 halves (hi, lo): the C chunk as [landmark][64 tokens] (A rows, K contiguous) and the V chunk as
  // [64 tokens][D] (B, read by transposing reads); row strides of 16 bytes mod 128.
  // Landmark rows >= mout are never written; they only feed output rows that are not stored.
  constexpr int LDC = 64 + 8;
  constexpr int LDV = D + 8;
  constexpr int DT = D / 16;
  constexpr int CTW = (DT + 3) / 4;  // column tiles per wave
  constexpr int NQC = MT;            // float4 loads of C per thread: MT*16 landmarks x 16 float4
  constexpr int NQV = D / 16;        // 4-element loads of V per thread for a full chunk
  __shared__ __align__(16) _Float16 sCh[MT * 16 * LDC];
  __shared__ __align__(16) _Float16 sCl[MT * 16 * LDC];
  __shared__ __align__(16) _Float16 sVh[64 * LDV];
  __shared__ __align__(16) _Float16 sVl[64 * LDV];
  __shared__ float sMax[8];
  const int mout = mrow + ones;
  // Block = (slice, token split, landmark block of MT*16 landmarks), landmark block fastest. Consecutive blocks run on
  // one XCD (blocks are dealt to the 8 XCDs round-robin), so the landmark blocks of one split read its V rows
  // through one L2.
  int b = static_cast<int>(blockIdx.x);
  {
    const int full = (static_cast<int>(gridDim.x) / 8) * 8;
    if (lsplit > 1 && b < full) b = (b % 8) * (full / 8) + b / 8;
  }
  const int lsb = b % lsplit;
  b /= lsplit;
  const int g = b / nsplit, s = b % nsplit;
  const int lbase = lsb * MT * 16;  // first landmark of this block
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const bool vec = (N & 3) == 0;  // landmark rows start 16-byte aligned
  const int t16 = ln & 15, gq = ln >> 4;

  f32x4 acc[MT][CTW];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < CTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r0 = s * rows_per_split, r1 = min(N, r0 + rows_per_split);
  const float* cg = C + static_cast<size_t>(g) * mrow * N;
  const T* vg = V + static_cast<size_t>(g) * N * D;
  for (int c0 = r0; c0 < r1; c0 += 64) {
    const int nr = min(64, r1 - c0);
    const T* vsrc = vg + static_cast<size_t>(c0) * D;
    float4 cbuf[NQC];
    float4 vbuf[NQV];
#pragma unroll
    for (int q = 0; q < NQC; ++q) {
      const int e = tid + 256 * q;
      const int l = lbase + (e >> 4), i = 4 * (e & 15);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (l < mrow) {
        const float* src = cg + static_cast<size_t>(l) * N + c0 + i;
        if (vec && i + 3 < nr) {
          v = load4(src);
        } else {
          v.x = i + 0 < nr ? src[0] : 0.f;
          v.y = i + 1 < nr ? src[1] : 0.f;
          v.z = i + 2 < nr ? src[2] : 0.f;
          v.w = i + 3 < nr ? src[3] : 0.f;
        }
      } else if (ones && l == mrow) {  // the appended column of ones (tokens of this chunk only)
        v = make_float4(i + 0 < nr ? 1.f : 0.f, i + 1 < nr ? 1.f : 0.f, i + 2 < nr ? 1.f : 0.f,
                        i + 3 < nr ? 1.f : 0.f);
      }
      cbuf[q] = v;
    }
    float cmax = 0.f, vmax = 0.f;
#pragma unroll
    for (int q = 0; q < NQC; ++q)
      cmax = fmaxf(cmax, fmaxf(fmaxf(fabsf(cbuf[q].x), fabsf(cbuf[q].y)), fmaxf(fabsf(cbuf[q].z), fabsf(cbuf[q].w))));
#pragma unroll
    for (int q = 0; q < NQV; ++q) {
      const int e = 4 * (tid + 256 * q);
      vbuf[q] = (e < nr * D) ? load4(vsrc + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(vbuf[q].x), fabsf(vbuf[q].y)), fmaxf(fabsf(vbuf[q].z), fabsf(vbuf[q].w))));
    }
    cmax = wave_max_nonneg(cmax);
    vmax = wave_max_nonneg(vmax);
    if (ln == 0) {
      sMax[wv] = cmax;
      sMax[4 + wv] = vmax;
    }
    __syncthreads();  // the previous chunk's MFMA reads are done; the chunk's maxima are in
    // each operand chunk's scale puts its largest entry in [2^12, 2^13) (clamped to keep the factors finite)
    const int ec = max(-100, min(100, store_exp(fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3])))));
    const int ev = max(-100, min(100, store_exp(fmaxf(fmaxf(sMax[4], sMax[5]), fmaxf(sMax[6], sMax[7])))));
    const float sc = ldexpf(1.f, -ec), sv = ldexpf(1.f, -ev);
#pragma unroll
    for (int q = 0; q < NQC; ++q) {
      const int e = tid + 256 * q;
      half4 h, l;
      split_scaled4(f32x4{cbuf[q].x, cbuf[q].y, cbuf[q].z, cbuf[q].w}, sc, h, l);
      const int o = (e >> 4) * LDC + 4 * (e & 15);
      *reinterpret_cast<half4*>(&sCh[o]) = h;
      *reinterpret_cast<half4*>(&sCl[o]) = l;
    }
#pragma unroll
    for (int q = 0; q < NQV; ++q) {
      const int e = 4 * (tid + 256 * q);
      half4 h, l;
      split_scaled4(f32x4{vbuf[q].x, vbuf[q].y, vbuf[q].z, vbuf[q].w}, sv, h, l);
      const int o = (e / D) * LDV + (e % D);
      *reinterpret_cast<half4*>(&sVh[o]) = h;
      *reinterpret_cast<half4*>(&sVl[o]) = l;
    }
    __syncthreads();
    if (wv * CTW < DT) {
      // K = the chunk's 64 tokens in two halves of 32; the lane supplies row t16 of A (landmark) and column t16 of
      // B (channel) at tokens 8 gq .. 8 gq + 7 of the half. Each chunk sums into a fresh accumulator that is added
      // to the block's sum with the chunk's scale undone.
      f32x4 p[MT][CTW];
#pragma unroll
      for (int lt = 0; lt < MT; ++lt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) p[lt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        half8 bh[CTW], bl[CTW];
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const int k0 = kh * 32 + 8 * gq + (t16 >> 2), i = (wv * CTW + ct) * 16 + 4 * (t16 & 3);
          const half4 h0 = __builtin_bit_cast(half4, lds_read_tr(&sVh[k0 * LDV + i]));
          const half4 h1 = __builtin_bit_cast(half4, lds_read_tr(&sVh[(k0 + 4) * LDV + i]));
          const half4 l0 = __builtin_bit_cast(half4, lds_read_tr(&sVl[k0 * LDV + i]));
          const half4 l1 = __builtin_bit_cast(half4, lds_read_tr(&sVl[(k0 + 4) * LDV + i]));
          bh[ct] = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          bl[ct] = half8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        }
#pragma unroll
        for (int lt = 0; lt < MT; ++lt) {
          const int oa = (lt * 16 + t16) * LDC + kh * 32 + 8 * gq;
          const half8 ah = *reinterpret_cast<const half8*>(&sCh[oa]);
          const half8 al = *reinterpret_cast<const half8*>(&sCl[oa]);
#pragma unroll
          for (int ct = 0; ct < CTW; ++ct) {
            p[lt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[ct], p[lt][ct], 0, 0, 0);
            p[lt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[ct], p[lt][ct], 0, 0, 0);
            p[lt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh[ct], p[lt][ct], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int lt = 0; lt < MT; ++lt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[lt][ct][rr] += ldexpf(p[lt][ct][rr], ec + ev);
    }
  }
  if (wv * CTW < DT) {
    float* pg = part + (static_cast<size_t>(g) * nsplit + s) * mout * D;
#pragma unroll
    for (int lt = 0; lt < MT; ++lt)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int c = (wv * CTW + ct) * 16 + (ln & 15);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int l = lbase + lt * 16 + 4 * (ln >> 4) + rr;
          if (l < mout && c < D) pg[static_cast<size_t>(l) * D + c] = acc[lt][ct][rr];
        }
      }
  }
}

__global__ __launch_bounds__(256) void k_ckv_finalize(const float* __restrict__ part, float* __restrict__ S, int G,
                                                      int nsplit, int md) {
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= static_cast<size_t>(G) * md) return;
  const size_t g = t / md, e = t % md;
  const float* p = part + g * nsplit * md + e;
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) acc += p[static_cast<size_t>(s) * md];
  S[t] = acc;
}

// =====================================================================================================
// landmark_mix: P[g][l][c] = rstd[l] * sum_k X[g][l][k] S[g][k][c]   (X = Newton-Schulz pseudo-inverse,
//   [note] Designs 2 and 3; rstd from the diagonal whitening of Design 1). m x m times m x D per slice.
// Block: 256 / D landmark rows x D channels of one slice, one output per thread; X rows and 64-row chunks of S are
// staged in LDS, and each output sums its landmarks in order.
// With wst the block first finishes the whitening statistics of its landmark rows from the per-tile partials of
// C_Q (tile sum and sum of squared deviations from the tile mean, 64 rows per tile): wave w takes rows w, w + 4, ..;
// lane t merges tiles t, t + 64, .. in order, then the lanes are merged in a fixed butterfly, each merge the
// pairwise update of Chan, Golub and LeVeque in float64 (counts add, sums add, and the squared-deviation sums add
// plus delta^2 n_a n_b / (n_a + n_b) for the difference delta of the two means). mu = sum / N and
// rstd = 1 / sqrt(M2 / N + weps) (the population variance) are written for the output kernel and the backward.
// =====================================================================================================
__device__ __forceinline__ void chan_merge(double& na, double& sa, double& qa, double nb, double sb, double qb) {
  if (nb == 0.0) return;
  if (na == 0.0) {
    na = nb;
    sa = sb;
    qa = qb;
    return;
  }
  const double d = sb / nb - sa / na;
  qa = (qa + qb) + d * d * (na * nb / (na + nb));
  sa += sb;
  na += nb;
}

template <int D>
__global__ __launch_bounds__(256) void k_mix(const float* __restrict__ X, const float* __restrict__ S,
                                             const float* __restrict__ rstd, float* __restrict__ P,
                                             float* __restrict__ Praw, int m, const float* __restrict__ wst,
                                             float* __restrict__ mu_out, float* __restrict__ rstd_out, int N,
                                             float weps) {
  constexpr int RB = 256 / D;  // landmark rows per block: one output (row, channel) per thread
  __shared__ float sX[RB * 65];
  __shared__ float sS[64 * D];
  __shared__ float s_rstd[RB];
  const int g = blockIdx.y, l0 = blockIdx.x * RB, tid = threadIdx.x;
  const float* xg = X + static_cast<size_t>(g) * m * m;
  const float* sg = S + static_cast<size_t>(g) * m * D;
  // chunk k0 of S (64 landmark rows) and of the block's X rows into registers; the first chunk's loads go out
  // before the whitening merge so that the two memory round trips overlap
  constexpr int NQ = (64 * D / 4 + 255) / 256;
  constexpr int NXV = (RB * 64 + 255) / 256;
  float4 buf[NQ];
  float xv[NXV];
  auto load_chunk = [&](int k0) {
    const int nk = min(64, m - k0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      buf[q] = (e < nk * D) ? load4(sg + static_cast<size_t>(k0) * D + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int e = tid + 256 * q;
      const int xr = e >> 6, kk = e & 63;
      xv[q] = (xr < RB && l0 + xr < m && kk < nk) ? xg[static_cast<size_t>(l0 + xr) * m + k0 + kk] : 0.f;
    }
  };
  load_chunk(0);
  if (wst) {
    const int tiles = (N + 63) / 64, wv = tid >> 6, ln = tid & 63;
    for (int r2 = wv; r2 < RB; r2 += 4) {
      const int l = l0 + r2;
      if (l >= m) break;
      double n = 0.0, sum = 0.0, q = 0.0;
      for (int t = ln; t < tiles; t += 64) {
        const float* w = wst + 2 * ((static_cast<size_t>(g) * m + l) * tiles + t);
        chan_merge(n, sum, q, static_cast<double>(min(64, N - 64 * t)), static_cast<double>(w[0]),
                   static_cast<double>(w[1]));
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double n2 = __shfl_xor(n, off), s2 = __shfl_xor(sum, off), q2 = __shfl_xor(q, off);
        chan_merge(n, sum, q, n2, s2, q2);
      }
      if (ln == 0) {
        const double mean = sum / n, var = q / n;
        const float r = static_cast<float>(1.0 / sqrt(var + static_cast<double>(weps)));
        mu_out[static_cast<size_t>(g) * m + l] = static_cast<float>(mean);
        rstd_out[static_cast<size_t>(g) * m + l] = r;
        s_rstd[r2] = r;
      }
    }
    __syncthreads();
  }
  const int rr = tid / D, c = tid % D;
  float acc = 0.f;
  for (int k0 = 0; k0 < m; k0 += 64) {
    const int nk = min(64, m - k0);
    if (k0 > 0) load_chunk(k0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int e = tid + 256 * q;
      if ((e >> 6) < RB) sX[(e >> 6) * 65 + (e & 63)] = xv[q];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = 4 * (tid + 256 * q);
      if (e < 64 * D) store4(sS + e, buf[q]);
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < nk; ++kk) acc += sX[rr * 65 + kk] * sS[kk * D + c];
  }
  const int l = l0 + rr;
  if (l < m) {
    const float sc = wst ? s_rstd[rr] : (rstd ? rstd[static_cast<size_t>(g) * m + l] : 1.f);
    P[(static_cast<size_t>(g) * m + l) * D + c] = acc * sc;
    if (Praw) Praw[(static_cast<size_t>(g) * m + l) * D + c] = acc;
  }
}

// =====================================================================================================
// out_gemm_dwc: Y[g][i][c] = sum_l C_Q[g][l][i] P[g][l][c] - sum_l mu[g][l] P[g][l][c] + DWC(V)[g][i][c]
//   ([note] Design 1: output = ZV + DWC(V); flowchart nodes G, H, I). The whitening bias is the folded form of
//   (C_Q - mu) rstd P with rstd already applied to P. With flip = 1 the 3x3 filter is rotated by 180 degrees,
//   which makes the stencil the adjoint of DWC (the backward pass uses that for dV = C_K dS + DWC^T(dY)).
// Block: an 8 x 8 patch of the token grid of one slice (64 tokens) and all D channels.
//   1. The 10 x 10 halo of V around the patch is staged once in LDS (zero outside the grid).
//   2. The product runs transposed, Y^T[c][u] = sum_l P[l][c] C[l][u], on the fp16 MFMA with both operands split
//      into fp16 halves (hi + lo; three MFMAs per product: hi hi, hi lo, lo hi, fp32 accumulation), which tracks
//      the fp32 product to a few units of 1e-7 at a fifth of the fp32 MFMA's cost. 64-landmark chunks of C and P
//      are staged in LDS as split halves in their natural [landmark][...] layouts; both operands are read with
//      gfx950's transposing LDS read (each lane gets 8 consecutive landmarks of its channel or token). Both carry
//      power-of-two scales that put their largest entries near 2^12, far from fp16's limits: P one per chunk,
//      C one per token and chunk (a token far from every landmark has all its entries of C many decades below 1,
//      which unscaled fp16 halves would flush to zero); each chunk's product is accumulated apart and added to
//      the token's total with both scales undone. Each lane's accumulator holds 4 consecutive channels of one
//      token.
//   3. The epilogue adds the bias and the 3x3 stencil per float4 and stores Y per (token, 4 channels).
// =====================================================================================================
template <int D>
struct OutLds {  // byte offsets
  static constexpr int NHC = 72;     // C (and X) rows: 64 tokens (or landmarks) + 8 halves
  static constexpr int NHP = D + 8;  // P^T (and S) rows: D channels + 8 halves
  static constexpr int LDV = D + 4;  // V halo row stride in floats (float4 aligned)
  static constexpr int SPLIT_C = 2 * 64 * NHC * 2;
  static constexpr int SPLIT_P = 2 * 64 * NHP * 2;
  static constexpr int HALO = 100 * LDV * 4;
  static constexpr int CA = 0;                 // C tile (MIX: X first)
  static constexpr int PA = CA + SPLIT_C;      // P^T
  static constexpr int VA = PA + SPLIT_P;      // V halo (MIX: S first)
  static constexpr int MU = VA + (HALO > SPLIT_P ? HALO : SPLIT_P);
  static constexpr int WT = MU + 64 * 4;
  static constexpr int BIAS = WT + 9 * D * 4;
  static constexpr int RED = BIAS + D * 4;     // 16 floats of block reductions
  static constexpr int CMAX = RED + 16 * 4;    // [8 waves][64 tokens]: largest C of each token per wave
  static constexpr int TOTAL = CMAX + 8 * 64 * 4;
};

// Fragment of a split matrix stored with element (k, x) at k * stride + x (x contiguous): lane t of 16-lane group
// g receives x = 16 strip + t at K = 32 c + 8 g .. + 7 (two transposing 8-byte reads per half). With x a row this
// is an A operand, with x a column a B operand.
__device__ __forceinline__ void frag_tr(const _Float16* hi, const _Float16* lo, int stride, int strip, int ln, int c,
                                        half8& h, half8& l) {
  const int g = ln >> 4, t = ln & 15;
  const int x = strip * 16 + 4 * (t & 3);
  const int k0 = c * 32 + 8 * g + (t >> 2);
  const short4v h0 = lds_read_tr(hi + k0 * stride + x), h1 = lds_read_tr(hi + (k0 + 4) * stride + x);
  const short4v l0 = lds_read_tr(lo + k0 * stride + x), l1 = lds_read_tr(lo + (k0 + 4) * stride + x);
  const half4 hh0 = __builtin_bit_cast(half4, h0), hh1 = __builtin_bit_cast(half4, h1);
  const half4 ll0 = __builtin_bit_cast(half4, l0), ll1 = __builtin_bit_cast(half4, l1);
  h = half8{hh0[0], hh0[1], hh0[2], hh0[3], hh1[0], hh1[1], hh1[2], hh1[3]};
  l = half8{ll0[0], ll0[1], ll0[2], ll0[3], ll1[0], ll1[1], ll1[2], ll1[3]};
}

// Fragment of a split matrix stored with element (x, k) at x * stride + k (k contiguous): one 16-byte read per half.
__device__ __forceinline__ void frag_rows(const _Float16* hi, const _Float16* lo, int stride, int strip, int ln,
                                          int c, half8& h, half8& l) {
  const int x = strip * 16 + (ln & 15), k0 = c * 32 + 8 * (ln >> 4);
  h = *reinterpret_cast<const half8*>(hi + x * stride + k0);
  l = *reinterpret_cast<const half8*>(lo + x * stride + k0);
}

// acc += A B for one 32-wide K chunk of split operands.
__device__ __forceinline__ f32x4 mma_split(half8 ah, half8 al, half8 bh, half8 bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc, 0, 0, 0);
  return acc;
}

// 2^-e for a storage exponent, kept inside float's normal range.
__device__ __forceinline__ float pow2_neg(int e) {
  e = max(-100, min(100, e));
  return __int_as_float((127 - e) << 23);
}

// Largest of the block's non-negative values a and b (8 waves), through red[0..15]; every thread gets both.
// The caller keeps red untouched until all threads have passed the next barrier.
__device__ __forceinline__ void block_max2(float a, float b, float* red, int wv, float& ma, float& mb) {
  a = wave_max_nonneg(a);
  b = wave_max_nonneg(b);
  if ((threadIdx.x & 63) == 0) {
    red[wv] = a;
    red[8 + wv] = b;
  }
  __syncthreads();
  ma = red[0];
  mb = red[8];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    ma = fmaxf(ma, red[i]);
    mb = fmaxf(mb, red[8 + i]);
  }
}

// MIX (m <= 64, no whitening): P = X S is formed in the block's prologue from the Newton-Schulz result X and
// S = C_K^T V (P then stands for S, and Xm for X), instead of being read from memory: this replaces the separate
// landmark-mix launch. It runs as P^T = S^T X^T on the same split MFMA, with S and X staged in the halo and C areas
// (each with its own power-of-two scale) before either is needed, and the halo's and the C tile's global loads
// already in flight meanwhile.
template <typename T, int D, bool FUSED, bool MIX>
__global__ __launch_bounds__(512) void k_out(const float* __restrict__ CQ, const float* __restrict__ P,
                                             const float* __restrict__ mu, const T* __restrict__ V,
                                             const float* __restrict__ w, T* __restrict__ Y, int N, int m, int H,
                                             int W, int heads, int flip, int tiles_x, const T* __restrict__ Q,
                                             const float* __restrict__ L, float scale, const float* __restrict__ Xm) {
  using Lay = OutLds<D>;
  constexpr int NWV = 8, NT = 64 * NWV;  // 8 waves: two blocks per CU (LDS) give 4 waves per SIMD
  constexpr int NHC = Lay::NHC, NHP = Lay::NHP;
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* sChi = reinterpret_cast<_Float16*>(smem + Lay::CA);
  _Float16* sClo = sChi + 64 * NHC;
  _Float16* sPhi = reinterpret_cast<_Float16*>(smem + Lay::PA);
  _Float16* sPlo = sPhi + 64 * NHP;
  float* sVh = reinterpret_cast<float*>(smem + Lay::VA);
  float* sMu = reinterpret_cast<float*>(smem + Lay::MU);
  float* sWt = reinterpret_cast<float*>(smem + Lay::WT);
  float* sBias = reinterpret_cast<float*>(smem + Lay::BIAS);
  float* sRed = reinterpret_cast<float*>(smem + Lay::RED);
  float* sCmax = reinterpret_cast<float*>(smem + Lay::CMAX);
  constexpr int CS = D / 16;                     // channel strips of 16
  constexpr int NP = CS * 4;                     // output tiles: (channel strip, 16-token tile) pairs
  constexpr int PPW = (NP + NWV - 1) / NWV;      // tiles per wave
  static_assert(NP % PPW == 0, "tiles per wave must divide the tile count");
  constexpr int C4 = D / 4;
  constexpr int LQM = 64 / NWV;                  // FUSED: most landmarks of a chunk per wave
  // Block order: the hardware deals workgroups to the 8 XCDs round-robin by linear index (x fastest), and each XCD
  // has its own L2. The linear index is remapped so that consecutive patches run on one XCD: the patches of one
  // patch row read their C_Q runs (32 bytes per landmark row) from shared 128-byte lines and overlap in their V
  // halos, so those lines leave HBM once instead of once per XCD.
  long lin = static_cast<long>(blockIdx.y) * gridDim.x + blockIdx.x;
  {
    const long total = static_cast<long>(gridDim.x) * gridDim.y, full = (total / 8) * 8;
    if (lin < full) lin = (lin % 8) * (full / 8) + lin / 8;
  }
  const int g = static_cast<int>(lin / gridDim.x);
  const int pt = static_cast<int>(lin % gridDim.x);
  const int ty0 = (pt / tiles_x) * 8, tx0 = (pt % tiles_x) * 8;
  const int h = g % heads;
  // the wave index through readfirstlane: the compiler then knows it is uniform and keeps the per-wave tile
  // guards below as scalar branches outside the MFMA sequences
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const float* cg = CQ + static_cast<size_t>(g) * m * N;
  const float* pg = P + static_cast<size_t>(g) * m * D;
  const T* vg = V + static_cast<size_t>(g) * N * D;
  const bool has_w = w != nullptr;

  // MIX: X and S are loaded before anything else. Vector loads complete in issue order, so the prologue's product
  // then waits only for these two small matrices while the V halo and the C_Q tile below are still in flight. The
  // loads up to that point are branch-free (clamped address; out-of-range values are zeroed where they are
  // staged), which lets the compiler wait for a count of outstanding loads instead of draining them all.
  constexpr int NXQ = MIX ? 4096 / NT : 1;              // MIX: X elements per thread, [64][64] zero-padded
  constexpr int NSQ = MIX ? (16 * D + NT - 1) / NT : 1;  // MIX: S float4 per thread, [64][D / 4]
  float xr[NXQ];
  float4 sr[NSQ];
  if constexpr (MIX) {
    const float* xg = Xm + static_cast<size_t>(g) * m * m;
#pragma unroll
    for (int q = 0; q < NXQ; ++q) {
      const int e = tid + NT * q;
      const int l = e >> 6, k = e & 63;
      xr[q] = xg[(l < m && k < m) ? l * m + k : 0];
    }
#pragma unroll
    for (int q = 0; q < NSQ; ++q) {
      const int e = tid + NT * q;  // float4 index over [64][D / 4]
      const int k = e / C4, c4 = e % C4;
      sr[q] = load4(pg + ((e < 16 * D && k < m) ? static_cast<size_t>(k) * D + 4 * c4 : 0));
    }
  }

  // 1. V halo and filter taps (both loaded here, stored to LDS after the prologue)
  constexpr int NQ = (100 * C4 + NT - 1) / NT;
  constexpr int NWT = (9 * D + NT - 1) / NT;
  float4 vb[NQ];
  float wt[NWT];
  if (has_w) {
#pragma unroll
    for (int q = 0; q < NWT; ++q) {
      const int e = min(tid + NT * q, 9 * D - 1), tap = e / D, c = e % D;
      wt[q] = w[(static_cast<size_t>(h) * D + c) * 9 + (flip ? 8 - tap : tap)];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + NT * q;
      const int tok = e / C4, c4 = e % C4;
      const int y = ty0 - 1 + tok / 10, x = tx0 - 1 + tok % 10;
      const bool in = e < 100 * C4 && y >= 0 && y < H && x >= 0 && x < W;
      vb[q] = load4(vg + (in ? static_cast<size_t>(y * W + x) * D + 4 * c4 : 0));  // zeroed when staged
    }
  }
  // MIX: m <= 64 is a single landmark chunk; its C_Q tile is loaded up front so that its latency overlaps the
  // prologue's product.
  constexpr int NCV0 = MIX ? 4096 / NT : 1;
  float cv0[NCV0];
  if constexpr (MIX) {
#pragma unroll
    for (int q = 0; q < NCV0; ++q) {
      const int e = tid + NT * q;
      const int l = e >> 6, u = e & 63;
      const int y = ty0 + (u >> 3), x = tx0 + (u & 7);
      cv0[q] = cg[(l < m && y < H && x < W) ? static_cast<size_t>(l) * N + y * W + x : 0];  // zeroed when staged
    }
  }
  int pexp = 0;  // MIX: P^T is stored times 2^-pexp
  if constexpr (MIX) {
    // P^T = S^T X^T, S^T by transposing reads of S ([k][c], the halo area) and X^T by plain reads of X ([l][k],
    // the C area), each scaled so that its largest entry lands near 2^12.
    float mx = 0.f, ms = 0.f;
#pragma unroll
    for (int q = 0; q < NXQ; ++q) {
      const int e = tid + NT * q;
      if ((e >> 6) < m && (e & 63) < m) mx = fmaxf(mx, fabsf(xr[q]));
    }
#pragma unroll
    for (int q = 0; q < NSQ; ++q) {
      const int e = tid + NT * q;
      if (e < 16 * D && e / C4 < m)
        ms = fmaxf(ms, fmaxf(fmaxf(fabsf(sr[q].x), fabsf(sr[q].y)), fmaxf(fabsf(sr[q].z), fabsf(sr[q].w))));
    }
    float bmx, bms;
    block_max2(mx, ms, sRed, wv, bmx, bms);
    const int ex = store_exp(bmx), es = store_exp(bms);
    const float fx = pow2_neg(ex), fs = pow2_neg(es);
    _Float16* sXhi = sChi;
    _Float16* sXlo = sClo;
    _Float16* sShi = reinterpret_cast<_Float16*>(sVh);
    _Float16* sSlo = sShi + 64 * NHP;
    static_assert(Lay::SPLIT_P <= Lay::MU - Lay::VA, "S must fit the halo area");
#pragma unroll
    for (int q = 0; q < NXQ; ++q) {
      const int e = tid + NT * q;
      const int l = e >> 6, k = e & 63;
      _Float16 hh, ll;
      split_f16((l < m && k < m) ? xr[q] * fx : 0.f, hh, ll);
      sXhi[l * NHC + k] = hh;
      sXlo[l * NHC + k] = ll;
    }
#pragma unroll
    for (int q = 0; q < NSQ; ++q) {
      const int e = tid + NT * q;
      if (e < 16 * D) {
        const int k = e / C4, c4 = e % C4;
        half4 hh, ll;
        const float4 v = k < m ? sr[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        split_scaled4(f32x4{v.x, v.y, v.z, v.w}, fs, hh, ll);
        *reinterpret_cast<half4*>(sShi + k * NHP + 4 * c4) = hh;
        *reinterpret_cast<half4*>(sSlo + k * NHP + 4 * c4) = ll;
      }
    }
    __syncthreads();
    // A wave owns PPM whole tiles or none (NPM is a multiple of PPM), so one uniform test covers them all. Tile
    // (channel strip cs, landmark tile lt).
    constexpr int NPM = 4 * CS, PPM = (NPM + NWV - 1) / NWV;
    static_assert(NPM % PPM == 0, "tiles per wave must divide the tile count");
    f32x4 a4[PPM];
#pragma unroll
    for (int jj = 0; jj < PPM; ++jj) a4[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float pm = 0.f;
    if (wv * PPM < NPM) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int jj = 0; jj < PPM; ++jj) {
          const int cs = (wv * PPM + jj) / 4, lt = (wv * PPM + jj) % 4;
          half8 ah, al, bh, bl;
          frag_tr(sShi, sSlo, NHP, cs, ln, c, ah, al);
          frag_rows(sXhi, sXlo, NHC, lt, ln, c, bh, bl);
          a4[jj] = mma_split(ah, al, bh, bl, a4[jj]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < PPM; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm = fmaxf(pm, fabsf(a4[jj][r]));
    }
    // the barrier inside also retires every read of X and S
    float bpm, unused;
    block_max2(pm, 0.f, sRed, wv, bpm, unused);
    const int e1 = store_exp(bpm);
    pexp = ex + es + e1;
    const float f1 = pow2_neg(e1);
    if (wv * PPM < NPM) {
#pragma unroll
      for (int jj = 0; jj < PPM; ++jj) {
        const int cs = (wv * PPM + jj) / 4, lt = (wv * PPM + jj) % 4;
        const int c0 = cs * 16 + 4 * (ln >> 4), l = lt * 16 + (ln & 15);
        half4 hh, ll;
        split_scaled4(a4[jj], f1, hh, ll);
        *reinterpret_cast<half4*>(sPhi + l * NHP + c0) = hh;
        *reinterpret_cast<half4*>(sPlo + l * NHP + c0) = ll;
      }
    }
  }
  if (has_w) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + NT * q;
      const int tok = e / C4;
      const int y = ty0 - 1 + tok / 10, x = tx0 - 1 + tok % 10;
      const bool in = y >= 0 && y < H && x >= 0 && x < W;
      if (e < 100 * C4) store4(sVh + tok * Lay::LDV + 4 * (e % C4), in ? vb[q] : make_float4(0.f, 0.f, 0.f, 0.f));
    }
#pragma unroll
    for (int q = 0; q < NWT; ++q)
      if (tid + NT * q < 9 * D) sWt[tid + NT * q] = wt[q];
  }
  if constexpr (FUSED) {
    // chunk rows a wave does not write keep finite values: zero them once (their P^T columns are staged as zero)
    for (int e = tid; e < 64 * NHC; e += NT) {
      sChi[e] = static_cast<_Float16>(0.f);
      sClo[e] = static_cast<_Float16>(0.f);
    }
  }
  float bias_acc = 0.f;  // the whitening bias of channel tid, in true units

  // FUSED: C_Q is not read from memory but computed here. Every wave holds the Q rows of the patch's 64 tokens
  // (lane = token) and computes its share of each landmark chunk, landmark coordinates arriving through scalar
  // loads (the landmark index is wave-uniform).
  float xq[FUSED ? D : 1];
  bool tok_ok = false;
  const float* Lg = nullptr;
  int wq = 0;
  if constexpr (FUSED) {
    const int y = ty0 + (ln >> 3), x = tx0 + (ln & 7);
    tok_ok = y < H && x < W;
    const T* qp = Q + (static_cast<size_t>(g) * N + (tok_ok ? y * W + x : 0)) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const float4 v = tok_ok ? load4(qp + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      xq[c] = v.x;
      xq[c + 1] = v.y;
      xq[c + 2] = v.z;
      xq[c + 3] = v.w;
    }
    Lg = L + static_cast<size_t>(g) * m * D;
    wq = __builtin_amdgcn_readfirstlane(wv);
  }

  // 2. Y^T = P^T C over 64-landmark chunks
  f32x4 acc[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int lc0 = 0; lc0 < m; lc0 += 64) {
    const int nl = min(64, m - lc0);
    // FUSED: landmarks per wave
    const int lq = (nl + NWV - 1) / NWV;
    constexpr int NCV = FUSED ? LQM : 4096 / NT;
    float cv[NCV];
    if constexpr (FUSED) {
#pragma unroll
      for (int q = 0; q < LQM; ++q) {
        const int l = wq * lq + q;
        float v = 0.f;
        if (q < lq && l < nl) {
          const float* __restrict__ lp = Lg + static_cast<size_t>(lc0 + l) * D;
          float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
          for (int c = 0; c < D; c += 4) {
            a0 += fabsf(xq[c + 0] - lp[c + 0]);
            a1 += fabsf(xq[c + 1] - lp[c + 1]);
            a2 += fabsf(xq[c + 2] - lp[c + 2]);
            a3 += fabsf(xq[c + 3] - lp[c + 3]);
          }
          v = tok_ok ? __builtin_amdgcn_exp2f(((a0 + a1) + (a2 + a3)) * scale) : 0.f;
        }
        cv[q] = v;
      }
    } else if constexpr (MIX) {
#pragma unroll
      for (int q = 0; q < NCV; ++q) {
        const int e = tid + NT * q;
        const int l = e >> 6, u = e & 63;
        cv[q] = (l < m && ty0 + (u >> 3) < H && tx0 + (u & 7) < W) ? cv0[q] : 0.f;
      }
    } else {
#pragma unroll
      for (int q = 0; q < NCV; ++q) {
        const int e = tid + NT * q;
        const int l = e >> 6, u = e & 63;
        const int y = ty0 + (u >> 3), x = tx0 + (u & 7);
        cv[q] = (l < nl && y < H && x < W) ? cg[static_cast<size_t>(lc0 + l) * N + y * W + x] : 0.f;
      }
    }
    constexpr int NQB = (16 * D + NT - 1) / NT;
    float4 bv[NQB];
    if constexpr (!MIX) {
#pragma unroll
      for (int q = 0; q < NQB; ++q) {
        const int e = tid + NT * q;
        const int rr = e / C4, c4 = e % C4;
        bv[q] = (e < 16 * D && rr < nl) ? load4(pg + static_cast<size_t>(lc0 + rr) * D + 4 * c4)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    const float muv = (mu && tid < 64 && tid < nl) ? mu[static_cast<size_t>(g) * m + lc0 + tid] : 0.f;
    // Scales of the chunk: every value of C this thread holds belongs to token ln (NT is a multiple of 64;
    // FUSED: lane = token), and P's largest entry. P's per-wave maxima go to LDS before the barrier below (the
    // previous chunk read them before its second barrier); C's per-token maxima only after it, because the
    // previous chunk reads them until its MFMAs are done, and every thread passes the barrier below only after
    // those reads.
    float cm = 0.f;
#pragma unroll
    for (int q = 0; q < NCV; ++q) cm = fmaxf(cm, cv[q]);
    if constexpr (!MIX) {
      float pm = 0.f;
#pragma unroll
      for (int q = 0; q < NQB; ++q)
        pm = fmaxf(pm, fmaxf(fmaxf(fabsf(bv[q].x), fabsf(bv[q].y)), fmaxf(fabsf(bv[q].z), fabsf(bv[q].w))));
      pm = wave_max_nonneg(pm);
      if (ln == 0) sRed[wv] = pm;
    }
    __syncthreads();  // previous chunk's reads are done
    sCmax[wv * 64 + ln] = cm;
    int eP = pexp;    // P of this chunk is stored times 2^-eP
    if constexpr (!MIX) {
      float bpm = sRed[0];
#pragma unroll
      for (int i = 1; i < NWV; ++i) bpm = fmaxf(bpm, sRed[i]);
      eP = store_exp(bpm);
      const float fp = pow2_neg(eP);
#pragma unroll
      for (int q = 0; q < NQB; ++q) {
        const int e = tid + NT * q;
        if (e < 16 * D) {
          half4 hh, ll;
          split_scaled4(f32x4{bv[q].x, bv[q].y, bv[q].z, bv[q].w}, fp, hh, ll);
          *reinterpret_cast<half4*>(sPhi + (e / C4) * NHP + 4 * (e % C4)) = hh;
          *reinterpret_cast<half4*>(sPlo + (e / C4) * NHP + 4 * (e % C4)) = ll;
        }
      }
    }
    if (tid < 64) sMu[tid] = muv;
    __syncthreads();
    {
      // C of token ln scaled by 2^-e, its largest entry in the chunk near 2^12
      float tm = sCmax[ln];
#pragma unroll
      for (int i = 1; i < NWV; ++i) tm = fmaxf(tm, sCmax[i * 64 + ln]);
      const float fc = pow2_neg(store_exp(tm));
      if constexpr (FUSED) {
#pragma unroll
        for (int q = 0; q < LQM; ++q)
          if (q < lq) {
            _Float16 hh, ll;
            split_f16(cv[q] * fc, hh, ll);
            sChi[(wq * lq + q) * NHC + ln] = hh;
            sClo[(wq * lq + q) * NHC + ln] = ll;
          }
      } else {
#pragma unroll
        for (int q = 0; q < NCV; ++q) {
          const int e = tid + NT * q;
          _Float16 hh, ll;
          split_f16(cv[q] * fc, hh, ll);
          sChi[(e >> 6) * NHC + (e & 63)] = hh;
          sClo[(e >> 6) * NHC + (e & 63)] = ll;
        }
      }
    }
    __syncthreads();
    if (mu && tid < D) {
      // the chunk's share of the bias, from the two halves of P
      float b = 0.f;
      for (int kk = 0; kk < nl; ++kk)
        b += sMu[kk] * (static_cast<float>(sPhi[kk * NHP + tid]) + static_cast<float>(sPlo[kk * NHP + tid]));
      bias_acc += ldexpf(b, eP);
    }
    // a wave owns PPW whole tiles or none (NP is a multiple of PPW): one uniform test outside the MFMA sequence
    if (wv * PPW < NP) {
      const int strip = (wv * PPW) >> 2;  // the wave's tiles share their channel strip
      f32x4 ac[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) ac[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        half8 ah, al;
        frag_tr(sPhi, sPlo, NHP, strip, ln, c, ah, al);
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
          half8 bh, bl;
          frag_tr(sChi, sClo, NHC, (wv * PPW + j) & 3, ln, c, bh, bl);
          ac[j] = mma_split(ah, al, bh, bl, ac[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        // undo the scales of P and of this lane's token u (tile column ln % 16)
        const int u = ((wv * PPW + j) & 3) * 16 + (ln & 15);
        float tm = sCmax[u];
#pragma unroll
        for (int i = 1; i < NWV; ++i) tm = fmaxf(tm, sCmax[i * 64 + u]);
        const int eu = max(-100, min(100, store_exp(tm))) + eP;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] += ldexpf(ac[j][r], eu);
      }
    }
  }
  if (tid < D) sBias[tid] = bias_acc;
  __syncthreads();

  // 3. epilogue: for tile (strip, t) the lane holds Y[token 16 t + ln%16][channels 16 strip + 4 (ln/16) .. +3]
  T* yg = Y + static_cast<size_t>(g) * N * D;
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int pr = wv * PPW + j;
    if (pr >= NP) continue;
    const int strip = pr >> 2, t = pr & 3;
    const int c0 = strip * 16 + 4 * (ln >> 4);
    const int u = t * 16 + (ln & 15);
    const int ty = u >> 3, tx = u & 7;
    const int y = ty0 + ty, x = tx0 + tx;
    if (y >= H || x >= W) continue;
    const float4 b = *reinterpret_cast<const float4*>(sBias + c0);
    float4 o = make_float4(acc[j][0] - b.x, acc[j][1] - b.y, acc[j][2] - b.z, acc[j][3] - b.w);
    if (has_w) {
#pragma unroll
      for (int aa = 0; aa < 3; ++aa)
#pragma unroll
        for (int bb = 0; bb < 3; ++bb) {
          const float4 v = *reinterpret_cast<const float4*>(sVh + ((ty + aa) * 10 + tx + bb) * Lay::LDV + c0);
          const float4 k4 = *reinterpret_cast<const float4*>(sWt + (aa * 3 + bb) * D + c0);
          o.x += k4.x * v.x;
          o.y += k4.y * v.y;
          o.z += k4.z * v.z;
          o.w += k4.w * v.w;
        }
    }
    store4(yg + static_cast<size_t>(y * W + x) * D + c0, o);
  }
}

// =====================================================================================================
// Launchers
// =====================================================================================================
static inline int cdiv(long a, long b) { return static_cast<int>((a + b - 1) / b); }

hipError_t launch_landmark_pool(const Shape& s, const void* Q, float* L, hipStream_t st) {
  const int c4n = s.d / 4;
  int slots = s.r < 256 / c4n ? s.r : 256 / c4n;
  if (slots < 1) slots = 1;
  const int tpl = c4n * slots;
  const int lpb = 256 / tpl;
  const long total = static_cast<long>(s.G) * s.m;
  const dim3 grid(cdiv(total, lpb));
  if (s.dtype == 1)
    hipLaunchKernelGGL(k_landmark_pool<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(Q), L, s.G, s.H,
                       s.W, s.d, s.r, s.m, tpl, lpb);
  else
    hipLaunchKernelGGL(k_landmark_pool<float>, grid, dim3(256), 0, st, static_cast<const float*>(Q), L, s.G, s.H,
                       s.W, s.d, s.r, s.m, tpl, lpb);
  return hipGetLastError();
}

// Launch shape of the distance kernel for T row tiles: nsc landmark super-chunks per tile, nw waves per block,
// lc landmarks per wave. A small model of the chip picks it: blocks are dealt in rounds of what fits on the 256 CUs
// at once (waves per SIMD from the register use, blocks per CU from LDS); a round costs the work of its busiest
// SIMD (its waves times lc + 2 landmarks, the 2 standing for a wave's fixed start-up cost), divided by how well w
// waves per SIMD hide the memory and scalar-load latency, w / (w + 2); each super-chunk adds 1% for reloading the
// rows. The constants were fitted to a sweep of all plans on the stage-1, stage-3 and high-resolution shapes, where
// this picks the fastest plan of each.
struct LaplacePlan {
  int nsc, nw, lc;
};

static LaplacePlan laplace_plan(long tiles, int m, int d) {
  const int resident = d <= 32 ? 8 : (d <= 64 ? 6 : 3);  // waves per SIMD that fit the kernel's registers
  const int lds_blocks = (160 * 1024) / (64 * (d + 4) * 4);
  auto eff = [](double w) { return w / (w + 2.0); };
  LaplacePlan best{1, 1, m};
  double best_t = 1e300;
  for (int nw = 1; nw <= 8; ++nw) {
    for (int nsc = 1; nsc <= 16; ++nsc) {
      const int chunks = nsc * nw;
      const int lc = cdiv(m, chunks);
      if (chunks > 1 && lc < 4) continue;        // too little work per wave
      if (static_cast<long>(chunks) * lc - m >= lc) continue;  // a wave with no landmarks
      const int rb = std::min(4 * resident / nw, lds_blocks);
      if (rb < 1) continue;
      const long nb = tiles * nsc, per_round = 256L * rb;
      auto round = [&](long bpc) {
        const double w = static_cast<double>(bpc * nw) / 4.0;
        return std::ceil(w) * (lc + 2) / eff(w);
      };
      double t = static_cast<double>(nb / per_round) * round(rb);
      if (nb % per_round) t += round(cdiv(nb % per_round, 256));
      t *= 1.0 + 0.01 * nsc;
      if (t < best_t - 1e-9) {
        best_t = t;
        best = {nsc, nw, lc};
      }
    }
  }
  return best;
}

template <typename T, int D>
static void laplace_t(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK, float* We,
                      int srcmask, hipStream_t st) {
  const int tilesN = cdiv(s.N, 64), tilesM = cdiv(s.m, 64);
  const int tq = (srcmask & 1) ? tilesN : 0, tk = (srcmask & 2) ? tilesN : 0, tl = (srcmask & 4) ? tilesM : 0;
  const long tiles = static_cast<long>(s.G) * (tq + tk + tl);
  if (tiles == 0) return;
  const LaplacePlan pl = laplace_plan(tiles, s.m, D);
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  hipLaunchKernelGGL((k_laplace<T, D>), dim3(static_cast<unsigned>(tiles * pl.nsc)), dim3(64 * pl.nw), 0, st,
                     static_cast<const T*>(Q), static_cast<const T*>(K), L, CQ, CK, We, s.N, s.m, tq, tk, tl, pl.nsc,
                     pl.lc, scale, s.eps);
}

template <typename T>
static void laplace_d(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK, float* We,
                      int srcmask, hipStream_t st) {
  switch (s.d) {
    case 16: laplace_t<T, 16>(s, Q, K, L, CQ, CK, We, srcmask, st); break;
    case 32: laplace_t<T, 32>(s, Q, K, L, CQ, CK, We, srcmask, st); break;
    case 64: laplace_t<T, 64>(s, Q, K, L, CQ, CK, We, srcmask, st); break;
    default: laplace_t<T, 128>(s, Q, K, L, CQ, CK, We, srcmask, st); break;
  }
}

hipError_t launch_laplace(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                          float* We, hipStream_t st, int srcmask) {
  if (s.dtype == 1)
    laplace_d<bf16_t>(s, Q, K, L, CQ, CK, We, srcmask, st);
  else
    laplace_d<float>(s, Q, K, L, CQ, CK, We, srcmask, st);
  return hipGetLastError();
}

hipError_t launch_whiten_stats(const Shape& s, const float* CQ, float* mu, float* rstd, hipStream_t st) {
  hipLaunchKernelGGL(k_whiten_stats, dim3(s.m, s.G), dim3(256), 0, st, CQ, mu, rstd, s.N, s.m, s.whiten_eps);
  return hipGetLastError();
}

int ckv_lsplit(const Shape& s) { return s.m > 64 ? cdiv(s.m, 64) : 1; }

void ckv_split(const Shape& s, int* nsplit, int* rows_per_split) {
  // At most ~512 blocks in all (splits times landmark blocks); each split covers whole 64-row chunks.
  const int chunks = cdiv(s.N, 64);
  int want = 512 / (s.G * ckv_lsplit(s));
  if (want > chunks) want = chunks;
  if (want < 1) want = 1;
  const int cps = cdiv(chunks, want);
  *rows_per_split = 64 * cps;
  *nsplit = cdiv(chunks, cps);
}

template <typename T, int D, int MT>
static void ckv_launch(const Shape& s, const float* C, int ones, const void* V, float* part, int nsplit, int rps,
                       int lsplit, hipStream_t st) {
  hipLaunchKernelGGL((k_ckv_partial<T, D, MT>), dim3(s.G * nsplit * lsplit), dim3(256), 0, st, C,
                     static_cast<const T*>(V), part, s.N, s.m, ones, nsplit, rps, lsplit);
}

template <typename T, int D>
static void ckv_mt(const Shape& s, const float* C, int ones, const void* V, float* part, int nsplit, int rps,
                   hipStream_t st) {
  // landmark blocks of 64 when m > 64 (the ones column is only used with m <= 64)
  const int lsplit = ones ? 1 : ckv_lsplit(s);
  if (lsplit > 1) {
    ckv_launch<T, D, 4>(s, C, ones, V, part, nsplit, rps, lsplit, st);
    return;
  }
  const int mt = cdiv(s.m + ones, 16);
  if (mt <= 1) ckv_launch<T, D, 1>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 2) ckv_launch<T, D, 2>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 3) ckv_launch<T, D, 3>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 4) ckv_launch<T, D, 4>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 5) ckv_launch<T, D, 5>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 8) ckv_launch<T, D, 8>(s, C, ones, V, part, nsplit, rps, 1, st);
  else if (mt <= 12) ckv_launch<T, D, 12>(s, C, ones, V, part, nsplit, rps, 1, st);
  else ckv_launch<T, D, 16>(s, C, ones, V, part, nsplit, rps, 1, st);
}

template <typename T>
static void ckv_d(const Shape& s, const float* C, int ones, const void* V, float* part, int nsplit, int rps,
                  hipStream_t st) {
  switch (s.d) {
    case 16: ckv_mt<T, 16>(s, C, ones, V, part, nsplit, rps, st); break;
    case 32: ckv_mt<T, 32>(s, C, ones, V, part, nsplit, rps, st); break;
    case 64: ckv_mt<T, 64>(s, C, ones, V, part, nsplit, rps, st); break;
    default: ckv_mt<T, 128>(s, C, ones, V, part, nsplit, rps, st); break;
  }
}

hipError_t launch_ckv_general(const Shape& s, const float* C, int ones, const void* V, float* partial, float* S,
                              hipStream_t st) {
  int nsplit, rps;
  ckv_split(s, &nsplit, &rps);
  const int mout = s.m + ones;
  float* dst = (nsplit == 1) ? S : partial;
  if (s.dtype == 1)
    ckv_d<bf16_t>(s, C, ones, V, dst, nsplit, rps, st);
  else
    ckv_d<float>(s, C, ones, V, dst, nsplit, rps, st);
  if (nsplit > 1) {
    const int md = mout * s.d;
    hipLaunchKernelGGL(k_ckv_finalize, dim3(cdiv(static_cast<long>(s.G) * md, 256)), dim3(256), 0, st, partial, S,
                       s.G, nsplit, md);
  }
  return hipGetLastError();
}

hipError_t launch_ckv(const Shape& s, const float* CK, const void* V, float* partial, float* S, hipStream_t st) {
  return launch_ckv_general(s, CK, 0, V, partial, S, st);
}

hipError_t launch_mix(const Shape& s, const float* X, const float* S, const float* rstd, float* P, float* Praw,
                      hipStream_t st) {
  // P = rstd * (X S) (rstd == nullptr means 1); Praw, when given, receives the unscaled X S.
  return launch_mix_whiten(s, X, S, nullptr, nullptr, const_cast<float*>(rstd), P, Praw, st);
}

hipError_t launch_mix_whiten(const Shape& s, const float* X, const float* S, const float* wst, float* mu, float* rstd,
                             float* P, float* Praw, hipStream_t st) {
  // wst null: P = rstd * (X S) with the given rstd (null means 1). Otherwise mu and rstd are outputs.
  const dim3 grid(cdiv(s.m, 256 / s.d), s.G);  // 256 / d landmark rows per block (k_mix)
  const float* rin = wst ? nullptr : rstd;
  float* rout = wst ? rstd : nullptr;
#define LF_MIX(D_)                                                                                                \
  hipLaunchKernelGGL(k_mix<D_>, grid, dim3(256), 0, st, X, S, rin, P, Praw, s.m, wst, mu, rout, s.N, s.whiten_eps)
  switch (s.d) {
    case 16: LF_MIX(16); break;
    case 32: LF_MIX(32); break;
    case 64: LF_MIX(64); break;
    default: LF_MIX(128); break;
  }
#undef LF_MIX
  return hipGetLastError();
}

template <typename T, int D, bool FUSED, bool MIX>
static void out_launch(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V,
                       const float* w, void* Y, int flip, const void* Q, const float* L, const float* X,
                       hipStream_t st) {
  const int tiles_x = cdiv(s.W, 8), tiles_y = cdiv(s.H, 8);
  const size_t lds = OutLds<D>::TOTAL;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_out<T, D, FUSED, MIX>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  hipLaunchKernelGGL((k_out<T, D, FUSED, MIX>), dim3(tiles_x * tiles_y, s.G), dim3(512), lds, st, CQ, P, mu,
                     static_cast<const T*>(V), w, static_cast<T*>(Y), s.N, s.m, s.H, s.W, s.heads, flip, tiles_x,
                     static_cast<const T*>(Q), L, scale, X);
}

template <typename T, bool FUSED, bool MIX>
static void out_d(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V, const float* w,
                  void* Y, int flip, const void* Q, const float* L, const float* X, hipStream_t st) {
  switch (s.d) {
    case 16: out_launch<T, 16, FUSED, MIX>(s, CQ, P, mu, V, w, Y, flip, Q, L, X, st); break;
    case 32: out_launch<T, 32, FUSED, MIX>(s, CQ, P, mu, V, w, Y, flip, Q, L, X, st); break;
    case 64: out_launch<T, 64, FUSED, MIX>(s, CQ, P, mu, V, w, Y, flip, Q, L, X, st); break;
    default: out_launch<T, 128, FUSED, MIX>(s, CQ, P, mu, V, w, Y, flip, Q, L, X, st); break;
  }
}

hipError_t launch_out(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V, const float* w,
                      void* Y, hipStream_t st) {
  if (s.dtype == 1)
    out_d<bf16_t, false, false>(s, CQ, P, mu, V, w, Y, 0, nullptr, nullptr, nullptr, st);
  else
    out_d<float, false, false>(s, CQ, P, mu, V, w, Y, 0, nullptr, nullptr, nullptr, st);
  return hipGetLastError();
}

bool out_mix_supported(const Shape& s) { return s.m <= 64 && s.d >= 32; }

// Recomputing C_Q inside the output kernel saves writing and reading C_Q (2 G m N 4 bytes: 9.8 MB at the stage-1
// shape, about 1.3 us of HBM time) but moves the G N m d distance terms into a kernel that runs them slower than
// the distance kernel does. Measured end to end (forward, inference, both paths green against the oracle):
// stage-1 56x56 m=49 fp32 49.6 us stored / 52.6 us recomputed; stage-3 14x14 m=49 121.2 / 140.5; 128x128 m=256
// bf16 225.0 / 239.5; 8x8 d=16 27.7 / 27.6 (within noise). The stored path is kept on every shape.
bool out_fused_pays(const Shape&) { return false; }

template <typename T>
static void out_mix_d(const Shape& s, const float* CQ, const float* X, const float* S, const void* V, const float* w,
                      void* Y, hipStream_t st) {
  switch (s.d) {
    case 32: out_launch<T, 32, false, true>(s, CQ, S, nullptr, V, w, Y, 0, nullptr, nullptr, X, st); break;
    case 64: out_launch<T, 64, false, true>(s, CQ, S, nullptr, V, w, Y, 0, nullptr, nullptr, X, st); break;
    default: out_launch<T, 128, false, true>(s, CQ, S, nullptr, V, w, Y, 0, nullptr, nullptr, X, st); break;
  }
}

hipError_t launch_out_mix(const Shape& s, const float* CQ, const float* X, const float* S, const void* V,
                          const float* w, void* Y, hipStream_t st) {
  if (!out_mix_supported(s)) return hipErrorInvalidValue;
  if (s.dtype == 1)
    out_mix_d<bf16_t>(s, CQ, X, S, V, w, Y, st);
  else
    out_mix_d<float>(s, CQ, X, S, V, w, Y, st);
  return hipGetLastError();
}

hipError_t launch_out_fused(const Shape& s, const void* Q, const float* L, const float* P, const void* V,
                            const float* w, void* Y, hipStream_t st) {
  if (s.dtype == 1)
    out_d<bf16_t, true, false>(s, nullptr, P, nullptr, V, w, Y, 0, Q, L, nullptr, st);
  else
    out_d<float, true, false>(s, nullptr, P, nullptr, V, w, Y, 0, Q, L, nullptr, st);
  return hipGetLastError();
}

hipError_t launch_out_adjoint(const Shape& s, const float* C, const float* P, const void* U, const float* w, void* out,
                              hipStream_t st) {
  if (s.dtype == 1)
    out_d<bf16_t, false, false>(s, C, P, nullptr, U, w, out, 1, nullptr, nullptr, nullptr, st);
  else
    out_d<float, false, false>(s, C, P, nullptr, U, w, out, 1, nullptr, nullptr, nullptr, st);
  return hipGetLastError();
}

}  // namespace lf
