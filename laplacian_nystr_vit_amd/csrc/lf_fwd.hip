// Forward-pass kernels of the LaplacianFormer attention block for gfx950 (CDNA4).
//
// Citations: papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力"
// ([note] below), sections motivation ("core idea"), framework (flowchart), Design 1, Design 2 and Design 3.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

// =====================================================================================================
// landmark_pool: L[g][l][c] = (1/r^2) sum_{a,b<r} Q[g][(Y r + a) W + X r + b][c]      ([note] Design 2)
// One thread per output element, channel fastest, so each wave reads whole token rows (coalesced).
// =====================================================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_landmark_pool(const T* __restrict__ Q, float* __restrict__ L, int G, int H,
                                                       int W, int d, int r, int m) {
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = static_cast<size_t>(G) * m * d;
  if (t >= total) return;
  const int c = static_cast<int>(t % d);
  const size_t gl = t / d;
  const int l = static_cast<int>(gl % m);
  const size_t g = gl / m;
  const int wr = W / r;
  const int Yb = l / wr, Xb = l % wr;
  const T* q = Q + g * static_cast<size_t>(H) * W * d + c;
  float acc = 0.f;
  for (int a = 0; a < r; ++a) {
    const T* row = q + (static_cast<size_t>(Yb * r + a) * W + static_cast<size_t>(Xb) * r) * d;
    for (int b = 0; b < r; ++b) acc += to_f32(row[static_cast<size_t>(b) * d]);
  }
  L[t] = acc / static_cast<float>(r * r);
}

// =====================================================================================================
// laplace_l1_exp: C[i][l] = exp(-sum_c |x_ic - L_lc| / lambda) for the rows x of Q, K and L
//   ([note] motivation "core idea" and Design 2; W + eps I from Design 3).
//
// This is a reduction of |x - l| and not a dot product, so it runs on the VALU, not on MFMA. One thread owns
// one row of Q, K or L and keeps it in VGPRs. The landmark index is wave-uniform, so the landmark values come
// through the scalar data cache into SGPRs and feed the VALU as free scalar operands: per (row, landmark,
// channel) the inner loop issues one v_sub_f32 and one v_add_f32 with an |.| source modifier, and no LDS or
// vector-memory traffic. exp(-s/lambda) becomes one v_exp_f32 of s * (-log2(e)/lambda).
//
// Grid: one 64-thread block (one wave) per (slice, source, 64-row tile, landmark chunk). The landmark chunks
// give each wave fewer landmarks so that the chip sees several waves per SIMD even at B*heads = 8.
// =====================================================================================================
template <typename T, int D>
__global__ __launch_bounds__(64) void k_laplace(const T* __restrict__ Q, const T* __restrict__ K,
                                                const float* __restrict__ L, float* __restrict__ CQ,
                                                float* __restrict__ CK, float* __restrict__ We, int N, int m,
                                                int tilesN, int tilesM, int nlc, int lc, float scale, float eps) {
  int b = blockIdx.x;
  const int lchunk = b % nlc;
  b /= nlc;
  const int per_slice = 2 * tilesN + tilesM;
  const int local = b % per_slice;
  const int g = b / per_slice;
  int src, tile;
  if (local < tilesN) {
    src = 0;
    tile = local;
  } else if (local < 2 * tilesN) {
    src = 1;
    tile = local - tilesN;
  } else {
    src = 2;
    tile = local - 2 * tilesN;
  }
  const int rows = (src == 2) ? m : N;
  const int row = tile * 64 + static_cast<int>(threadIdx.x);
  const int l0 = lchunk * lc;
  const int l1 = min(l0 + lc, m);
  const float* __restrict__ Lg = L + static_cast<size_t>(g) * m * D;
  if (row >= rows) return;

  float x[D];
  float* out;
  if (src == 2) {
    const float* p = Lg + static_cast<size_t>(row) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) x[c] = p[c];
    out = We + (static_cast<size_t>(g) * m + row) * m;
  } else {
    const T* p = (src == 0 ? Q : K) + (static_cast<size_t>(g) * N + row) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) x[c] = to_f32(p[c]);
    out = (src == 0 ? CQ : CK) + (static_cast<size_t>(g) * N + row) * m;
  }

  for (int l = l0; l < l1; ++l) {
    const float* __restrict__ lp = Lg + static_cast<size_t>(l) * D;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      a0 += fabsf(x[c + 0] - lp[c + 0]);
      a1 += fabsf(x[c + 1] - lp[c + 1]);
      a2 += fabsf(x[c + 2] - lp[c + 2]);
      a3 += fabsf(x[c + 3] - lp[c + 3]);
    }
    float v = __builtin_amdgcn_exp2f(((a0 + a1) + (a2 + a3)) * scale);
    if (src == 2 && l == row) v += eps;
    out[l] = v;
  }
}

// =====================================================================================================
// whiten_stats: per landmark column of C_Q, mean and 1/sqrt(biased variance + eps_w) over the N tokens
//   ([note] Design 1, diagonal whitening). Two passes in float64, fixed reduction order.
// =====================================================================================================
__global__ __launch_bounds__(256) void k_whiten_stats(const float* __restrict__ CQ, float* __restrict__ mu,
                                                      float* __restrict__ rstd, int N, int m, float weps) {
  __shared__ double red[4][64];
  const int g = blockIdx.y;
  const int ln = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int l = blockIdx.x * 64 + ln;
  const float* c = CQ + static_cast<size_t>(g) * N * m;
  double s = 0.0;
  if (l < m)
    for (int i = rg; i < N; i += 4) s += static_cast<double>(c[static_cast<size_t>(i) * m + l]);
  red[rg][ln] = s;
  __syncthreads();
  const double mean = (red[0][ln] + red[1][ln] + red[2][ln] + red[3][ln]) / static_cast<double>(N);
  __syncthreads();
  double v = 0.0;
  if (l < m)
    for (int i = rg; i < N; i += 4) {
      const double dd = static_cast<double>(c[static_cast<size_t>(i) * m + l]) - mean;
      v += dd * dd;
    }
  red[rg][ln] = v;
  __syncthreads();
  if (rg == 0 && l < m) {
    const double var = (red[0][ln] + red[1][ln] + red[2][ln] + red[3][ln]) / static_cast<double>(N);
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
// Stage 1: each block reduces `rows_per_split` token rows of one slice into a partial [mout][D] on fp32 MFMA
// (M = landmarks, N = channels, K = tokens), staging 64-row chunks of C and V through LDS.
// Stage 2: the partials are summed in split order.
// `ones` appends a column of ones to C (mout = mrow + 1), so row mrow of the result is sum_i V[i][c]; the
// backward pass uses this to get the column sums of dY in the same sweep as C_Q^T dY.
// =====================================================================================================
template <typename T, int D, int TPW>
__global__ __launch_bounds__(256) void k_ckv_partial(const float* __restrict__ CK, const T* __restrict__ V,
                                                     float* __restrict__ part, int N, int mrow, int mout, int nsplit,
                                                     int rows_per_split) {
  extern __shared__ float smem[];
  const int g = blockIdx.x / nsplit, s = blockIdx.x % nsplit;
  const int mt = (mout + 15) / 16;
  constexpr int DT = D / 16;
  const int ntiles = mt * DT;
  const int mp = mt * 16;
  const int LDC = ld_b(mp), LDV = ld_b(D);
  float* sC = smem;
  float* sV = smem + 64 * LDC;
  const int wv = wave_id(), ln = lane_id();
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r0 = s * rows_per_split, r1 = min(N, r0 + rows_per_split);
  const float* ckg = CK + static_cast<size_t>(g) * N * mrow;
  const T* vg = V + static_cast<size_t>(g) * N * D;
  for (int c0 = r0; c0 < r1; c0 += 64) {
    const int nr = min(64, r1 - c0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * mp; idx += 256) {
      const int rr = idx / mp, cc = idx % mp;
      float v = 0.f;
      if (rr < nr) v = (cc < mrow) ? ckg[static_cast<size_t>(c0 + rr) * mrow + cc] : (cc < mout ? 1.f : 0.f);
      sC[rr * LDC + cc] = v;
    }
    for (int idx = threadIdx.x; idx < 64 * D; idx += 256) {
      const int rr = idx / D, cc = idx % D;
      sV[rr * LDV + cc] = (rr < nr) ? to_f32(vg[static_cast<size_t>(c0 + rr) * D + cc]) : 0.f;
    }
    __syncthreads();
    const int ksteps = (nr + 3) / 4;
    for (int ks = 0; ks < ksteps; ++ks) {
      const int kr = ks * 4 + (ln >> 4);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tile = wv + 4 * t;
        if (tile < ntiles) {
          const int lt = tile / DT, ct = tile % DT;
          const float a = sC[kr * LDC + lt * 16 + (ln & 15)];
          const float b = sV[kr * LDV + ct * 16 + (ln & 15)];
          acc[t] = mfma16x16x4(a, b, acc[t]);
        }
      }
    }
  }
  float* pg = part + (static_cast<size_t>(g) * nsplit + s) * mout * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wv + 4 * t;
    if (tile < ntiles) {
      const int lt = tile / DT, ct = tile % DT;
      const int c = ct * 16 + (ln & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int l = lt * 16 + 4 * (ln >> 4) + rr;
        if (l < mout) pg[static_cast<size_t>(l) * D + c] = acc[t][rr];
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
  for (int s = 0; s < nsplit; ++s) acc += p[static_cast<size_t>(s) * md];
  S[t] = acc;
}

// =====================================================================================================
// landmark_mix: P[g][l][c] = rstd[l] * sum_k X[g][l][k] S[g][k][c]   (X = Newton-Schulz pseudo-inverse,
//   [note] Design 2 and 3; rstd from the diagonal whitening of Design 1). Small: m x m times m x D per slice.
// Block: 16 landmark rows x D channels of one slice; thread (row, 16-column group).
// =====================================================================================================
template <int D>
__global__ __launch_bounds__(256) void k_mix(const float* __restrict__ X, const float* __restrict__ S,
                                             const float* __restrict__ rstd, float* __restrict__ P,
                                             float* __restrict__ Praw, int m) {
  const int g = blockIdx.y;
  const int lr = threadIdx.x >> 4, cg = threadIdx.x & 15;
  const int l = blockIdx.x * 16 + lr;
  if (l >= m) return;
  constexpr int NC = (D + 15) / 16;
  float acc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) acc[j] = 0.f;
  const float* xr = X + (static_cast<size_t>(g) * m + l) * m;
  const float* sg = S + static_cast<size_t>(g) * m * D;
  for (int k = 0; k < m; ++k) {
    const float xv = xr[k];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = cg + 16 * j;
      if (c < D) acc[j] += xv * sg[static_cast<size_t>(k) * D + c];
    }
  }
  const float sc = rstd ? rstd[static_cast<size_t>(g) * m + l] : 1.f;
  float* pr = P + (static_cast<size_t>(g) * m + l) * D;
  float* prr = Praw ? Praw + (static_cast<size_t>(g) * m + l) * D : nullptr;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = cg + 16 * j;
    if (c < D) {
      pr[c] = acc[j] * sc;
      if (prr) prr[c] = acc[j];
    }
  }
}

// =====================================================================================================
// out_gemm_dwc: Y[g][i][c] = sum_l C_Q[g][i][l] P[g][l][c] - sum_l mu[g][l] P[g][l][c] + DWC(V)[g][i][c]
//   With flip = 1 the 3x3 filter is rotated by 180 degrees, which makes the stencil the adjoint of DWC; the
//   backward pass uses that for dV = C_K dS + DWC^T(dY).
//   ([note] Design 1: output = ZV + DWC(V); flowchart nodes G, H, I). The whitening bias is the folded form of
//   (C_Q - mu) rstd P with rstd already applied to P.
// Block: 64 tokens x D channels of one slice, 4 waves of 16 tokens each. The K = m reduction runs on fp32
// MFMA with 64-landmark chunks of C_Q and P staged in LDS; the depthwise 3x3 stencil and the bias are added
// in the epilogue before the single store of Y.
// =====================================================================================================
constexpr int OUT_LDA = 66;  // 2 mod 32: A-style reads (row = lane % 16, k = lane / 16) are conflict free

template <typename T, int D>
__global__ __launch_bounds__(256) void k_out(const float* __restrict__ CQ, const float* __restrict__ P,
                                             const float* __restrict__ mu, const T* __restrict__ V,
                                             const float* __restrict__ w, T* __restrict__ Y, int N, int m, int H,
                                             int W, int heads, int flip) {
  constexpr int LDB = ((D + 31) / 32) * 32 + 16;
  constexpr int DT = D / 16;
  __shared__ float sA[64 * OUT_LDA];
  __shared__ float sB[64 * LDB];
  __shared__ float sBias[D];
  const int g = blockIdx.y;
  const int i0 = blockIdx.x * 64;
  const int h = g % heads;
  const int wv = wave_id(), ln = lane_id();
  const float* cq = CQ + static_cast<size_t>(g) * N * m;
  const float* pg = P + static_cast<size_t>(g) * m * D;

  if (threadIdx.x < D) {
    float b = 0.f;
    if (mu) {
      const float* mg = mu + static_cast<size_t>(g) * m;
      for (int l = 0; l < m; ++l) b += mg[l] * pg[static_cast<size_t>(l) * D + threadIdx.x];
    }
    sBias[threadIdx.x] = b;
  }

  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int lc0 = 0; lc0 < m; lc0 += 64) {
    const int nl = min(64, m - lc0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
      const int rr = idx >> 6, cc = idx & 63;
      const int i = i0 + rr;
      sA[rr * OUT_LDA + cc] = (i < N && cc < nl) ? cq[static_cast<size_t>(i) * m + lc0 + cc] : 0.f;
    }
    for (int idx = threadIdx.x; idx < 64 * D; idx += 256) {
      const int rr = idx / D, cc = idx % D;
      sB[rr * LDB + cc] = (rr < nl) ? pg[static_cast<size_t>(lc0 + rr) * D + cc] : 0.f;
    }
    __syncthreads();
    const int ksteps = (nl + 3) / 4;
    for (int ks = 0; ks < ksteps; ++ks) {
      const int k = ks * 4 + (ln >> 4);
      const float a = sA[(wv * 16 + (ln & 15)) * OUT_LDA + k];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const float bb = sB[k * LDB + t * 16 + (ln & 15)];
        acc[t] = mfma16x16x4(a, bb, acc[t]);
      }
    }
  }
  __syncthreads();

  const T* vg = V + static_cast<size_t>(g) * N * D;
  T* yg = Y + static_cast<size_t>(g) * N * D;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int c = t * 16 + (ln & 15);
    float wk[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) wk[q] = w ? w[(static_cast<size_t>(h) * D + c) * 9 + (flip ? 8 - q : q)] : 0.f;
    const float bias = sBias[c];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = i0 + wv * 16 + 4 * (ln >> 4) + rr;
      if (i >= N) continue;
      float y = acc[t][rr] - bias;
      if (w) {
        const int yy = i / W, xx = i % W;
        float dsum = 0.f;
#pragma unroll
        for (int a = -1; a <= 1; ++a) {
#pragma unroll
          for (int bb = -1; bb <= 1; ++bb) {
            const int y2 = yy + a, x2 = xx + bb;
            if (y2 >= 0 && y2 < H && x2 >= 0 && x2 < W)
              dsum += wk[(a + 1) * 3 + (bb + 1)] * to_f32(vg[static_cast<size_t>(y2 * W + x2) * D + c]);
          }
        }
        y += dsum;
      }
      yg[static_cast<size_t>(i) * D + c] = from_f32<T>(y);
    }
  }
}

// =====================================================================================================
// Launchers
// =====================================================================================================
static inline int cdiv(long a, long b) { return static_cast<int>((a + b - 1) / b); }

hipError_t launch_landmark_pool(const Shape& s, const void* Q, float* L, hipStream_t st) {
  const size_t total = static_cast<size_t>(s.G) * s.m * s.d;
  const dim3 grid(cdiv(static_cast<long>(total), 256));
  if (s.dtype == 1)
    hipLaunchKernelGGL(k_landmark_pool<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(Q), L, s.G, s.H,
                       s.W, s.d, s.r, s.m);
  else
    hipLaunchKernelGGL(k_landmark_pool<float>, grid, dim3(256), 0, st, static_cast<const float*>(Q), L, s.G, s.H,
                       s.W, s.d, s.r, s.m);
  return hipGetLastError();
}

template <typename T, int D>
static void laplace_t(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK, float* We,
                      hipStream_t st) {
  const int tilesN = cdiv(s.N, 64), tilesM = cdiv(s.m, 64);
  const long waves = static_cast<long>(s.G) * (2 * tilesN + tilesM);
  // Split the landmark loop until the chip holds about 12 waves per CU, keeping >= 8 landmarks per wave.
  int nlc = 1;
  while (waves * nlc < 3072 && cdiv(s.m, nlc * 2) >= 8) nlc *= 2;
  const int lc = cdiv(s.m, nlc);
  nlc = cdiv(s.m, lc);
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  const dim3 grid(static_cast<unsigned>(waves * nlc));
  hipLaunchKernelGGL((k_laplace<T, D>), grid, dim3(64), 0, st, static_cast<const T*>(Q), static_cast<const T*>(K), L,
                     CQ, CK, We, s.N, s.m, tilesN, tilesM, nlc, lc, scale, s.eps);
}

template <typename T>
static void laplace_d(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK, float* We,
                      hipStream_t st) {
  switch (s.d) {
    case 16: laplace_t<T, 16>(s, Q, K, L, CQ, CK, We, st); break;
    case 32: laplace_t<T, 32>(s, Q, K, L, CQ, CK, We, st); break;
    case 64: laplace_t<T, 64>(s, Q, K, L, CQ, CK, We, st); break;
    default: laplace_t<T, 128>(s, Q, K, L, CQ, CK, We, st); break;
  }
}

hipError_t launch_laplace(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                          float* We, hipStream_t st) {
  if (s.dtype == 1)
    laplace_d<bf16_t>(s, Q, K, L, CQ, CK, We, st);
  else
    laplace_d<float>(s, Q, K, L, CQ, CK, We, st);
  return hipGetLastError();
}

hipError_t launch_whiten_stats(const Shape& s, const float* CQ, float* mu, float* rstd, hipStream_t st) {
  hipLaunchKernelGGL(k_whiten_stats, dim3(cdiv(s.m, 64), s.G), dim3(256), 0, st, CQ, mu, rstd, s.N, s.m,
                     s.whiten_eps);
  return hipGetLastError();
}

void ckv_split(const Shape& s, int* nsplit, int* rows_per_split) {
  // Aim for ~256 blocks; each split covers a multiple of 64 rows.
  int want = cdiv(256, s.G);
  const int maxsplit = cdiv(s.N, 64);
  if (want > maxsplit) want = maxsplit;
  if (want < 1) want = 1;
  int rps = cdiv(cdiv(s.N, want), 64) * 64;
  *rows_per_split = rps;
  *nsplit = cdiv(s.N, rps);
}

template <typename T, int D, int TPW>
static void ckv_launch(const Shape& s, const float* C, int mrow, int mout, const void* V, float* part, int nsplit,
                       int rps, hipStream_t st) {
  const int mp = cdiv(mout, 16) * 16;
  const size_t lds = sizeof(float) * 64 * (ld_b(mp) + ld_b(D));
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ckv_partial<T, D, TPW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL((k_ckv_partial<T, D, TPW>), dim3(s.G * nsplit), dim3(256), lds, st, C, static_cast<const T*>(V),
                     part, s.N, mrow, mout, nsplit, rps);
}

template <typename T, int D>
static void ckv_tpw(const Shape& s, const float* C, int mrow, int mout, const void* V, float* part, int nsplit,
                    int rps, hipStream_t st) {
  const int ntiles = cdiv(mout, 16) * (D / 16);
  const int tpw = cdiv(ntiles, 4);
  if (tpw <= 1)
    ckv_launch<T, D, 1>(s, C, mrow, mout, V, part, nsplit, rps, st);
  else if (tpw <= 2)
    ckv_launch<T, D, 2>(s, C, mrow, mout, V, part, nsplit, rps, st);
  else if (tpw <= 4)
    ckv_launch<T, D, 4>(s, C, mrow, mout, V, part, nsplit, rps, st);
  else if (tpw <= 8)
    ckv_launch<T, D, 8>(s, C, mrow, mout, V, part, nsplit, rps, st);
  else if (tpw <= 16)
    ckv_launch<T, D, 16>(s, C, mrow, mout, V, part, nsplit, rps, st);
  else
    ckv_launch<T, D, 32>(s, C, mrow, mout, V, part, nsplit, rps, st);
}

template <typename T>
static void ckv_d(const Shape& s, const float* C, int mrow, int mout, const void* V, float* part, int nsplit, int rps,
                  hipStream_t st) {
  switch (s.d) {
    case 16: ckv_tpw<T, 16>(s, C, mrow, mout, V, part, nsplit, rps, st); break;
    case 32: ckv_tpw<T, 32>(s, C, mrow, mout, V, part, nsplit, rps, st); break;
    case 64: ckv_tpw<T, 64>(s, C, mrow, mout, V, part, nsplit, rps, st); break;
    default: ckv_tpw<T, 128>(s, C, mrow, mout, V, part, nsplit, rps, st); break;
  }
}

hipError_t launch_ckv_general(const Shape& s, const float* C, int ones, const void* V, float* partial, float* S,
                              hipStream_t st) {
  int nsplit, rps;
  ckv_split(s, &nsplit, &rps);
  const int mout = s.m + ones;
  float* dst = (nsplit == 1) ? S : partial;
  if (s.dtype == 1)
    ckv_d<bf16_t>(s, C, s.m, mout, V, dst, nsplit, rps, st);
  else
    ckv_d<float>(s, C, s.m, mout, V, dst, nsplit, rps, st);
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
  const dim3 grid(cdiv(s.m, 16), s.G);
  switch (s.d) {
    case 16: hipLaunchKernelGGL(k_mix<16>, grid, dim3(256), 0, st, X, S, rstd, P, Praw, s.m); break;
    case 32: hipLaunchKernelGGL(k_mix<32>, grid, dim3(256), 0, st, X, S, rstd, P, Praw, s.m); break;
    case 64: hipLaunchKernelGGL(k_mix<64>, grid, dim3(256), 0, st, X, S, rstd, P, Praw, s.m); break;
    default: hipLaunchKernelGGL(k_mix<128>, grid, dim3(256), 0, st, X, S, rstd, P, Praw, s.m); break;
  }
  return hipGetLastError();
}

template <typename T>
static void out_d(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V, const float* w,
                  void* Y, int flip, hipStream_t st) {
  const dim3 grid(cdiv(s.N, 64), s.G);
  const T* v = static_cast<const T*>(V);
  T* y = static_cast<T*>(Y);
  switch (s.d) {
    case 16: hipLaunchKernelGGL((k_out<T, 16>), grid, dim3(256), 0, st, CQ, P, mu, v, w, y, s.N, s.m, s.H, s.W, s.heads, flip); break;
    case 32: hipLaunchKernelGGL((k_out<T, 32>), grid, dim3(256), 0, st, CQ, P, mu, v, w, y, s.N, s.m, s.H, s.W, s.heads, flip); break;
    case 64: hipLaunchKernelGGL((k_out<T, 64>), grid, dim3(256), 0, st, CQ, P, mu, v, w, y, s.N, s.m, s.H, s.W, s.heads, flip); break;
    default: hipLaunchKernelGGL((k_out<T, 128>), grid, dim3(256), 0, st, CQ, P, mu, v, w, y, s.N, s.m, s.H, s.W, s.heads, flip); break;
  }
}

hipError_t launch_out(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V, const float* w,
                      void* Y, hipStream_t st) {
  if (s.dtype == 1)
    out_d<bf16_t>(s, CQ, P, mu, V, w, Y, 0, st);
  else
    out_d<float>(s, CQ, P, mu, V, w, Y, 0, st);
  return hipGetLastError();
}

hipError_t launch_out_adjoint(const Shape& s, const float* C, const float* P, const void* U, const float* w, void* out,
                              hipStream_t st) {
  if (s.dtype == 1)
    out_d<bf16_t>(s, C, P, nullptr, U, w, out, 1, st);
  else
    out_d<float>(s, C, P, nullptr, U, w, out, 1, st);
  return hipGetLastError();
}

}  // namespace lf
