// Newton-Schulz pseudo-inverse of the landmark kernel on fp32 MFMA (gfx950).
//
// [note] = papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力", Design 3:
// W is shifted by eps I, X_0 = alpha W^T and X_{k+1} = X_k (2I - W X_k): only matrix products and additions,
// no inverse or SVD. alpha = 1/(||W||_1 ||W||_inf) (max column abs sum times max row abs sum) is the reading that
// keeps every eigenvalue of alpha W W^T in (0, 1]; the page's 2/||W||_2 would diverge for a unit-diagonal W.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

// =====================================================================================================
// m <= 64: one 256-thread block per slice runs every iteration out of LDS.
// Matrices are padded to 64 x 64 with zeros. Each product is 16 tiles of 16 x 16; wave w owns row strip w and
// the four column tiles, so one A fragment feeds four MFMAs per k step. X is kept both row-major (A operand
// of X U) and transposed (B operand of W X); U = 2I - W X is written transposed (B operand of X U), so every
// operand read has the lane pattern the LDS banks like (leading dimension 66 = 2 mod 32).
// =====================================================================================================
constexpr int NS_LD = 66;

__device__ __forceinline__ void ns_product(const float* __restrict__ sA, const float* __restrict__ sBt, int ksteps,
                                           int wv, int ln, int ntile, f32x4 acc[4]) {
  // acc[t] = A[16 wv .. 16 wv + 15][:] * B[:][16 t .. 16 t + 15], with B read from its transpose sBt.
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < ksteps; ++ks) {
    const int k = ks * 4 + (ln >> 4);
    const float a = sA[(wv * 16 + (ln & 15)) * NS_LD + k];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < ntile) {
        const float b = sBt[(t * 16 + (ln & 15)) * NS_LD + k];
        acc[t] = mfma16x16x4(a, b, acc[t]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_ns_small(const float* __restrict__ We, float* __restrict__ Xout,
                                                  float* __restrict__ xs, float* __restrict__ alpha_out,
                                                  float* __restrict__ resid, int m, int iters) {
  __shared__ float sW[64 * NS_LD];
  __shared__ float sX[2][64 * NS_LD];
  __shared__ float sXt[2][64 * NS_LD];
  __shared__ float sUt[64 * NS_LD];
  __shared__ double red[2][256];
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;

  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    sW[i * NS_LD + j] = (i < m && j < m) ? wg[i * m + j] : 0.f;
  }
  __syncthreads();

  // alpha = 1 / (max_j sum_i |W_ij| * max_i sum_j |W_ij|), accumulated in float64.
  double colsum = 0.0, rowsum = 0.0;
  if (tid < m) {
    for (int i = 0; i < m; ++i) {
      colsum += fabs(static_cast<double>(sW[i * NS_LD + tid]));
      rowsum += fabs(static_cast<double>(sW[tid * NS_LD + i]));
    }
  }
  red[0][tid] = colsum;
  red[1][tid] = rowsum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] = fmax(red[0][tid], red[0][tid + s]);
      red[1][tid] = fmax(red[1][tid], red[1][tid + s]);
    }
    __syncthreads();
  }
  const float alpha = static_cast<float>(1.0 / (red[0][0] * red[1][0]));
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;

  // X_0 = alpha W^T  (row-major), and its transpose alpha W.
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    const float wij = sW[i * NS_LD + j];
    sXt[0][i * NS_LD + j] = alpha * wij;  // Xt[i][j] = X[j][i] = alpha W[i][j]
    sX[0][j * NS_LD + i] = alpha * wij;   // X[j][i] = alpha W[i][j]
    if (xs && i < m && j < m) xs[(static_cast<size_t>(g) * (iters + 1)) * mm + j * m + i] = alpha * wij;
  }
  __syncthreads();

  const int ksteps = (m + 3) / 4;
  const int ntile = (m + 15) / 16;
  const bool active = wv < ntile;
  int cur = 0;
  f32x4 acc[4];
  for (int it = 0; it < iters; ++it) {
    // T = W X_cur ; Ut = (2I - T)^T restricted to the m x m block
    if (active) {
      ns_product(sW, sXt[cur], ksteps, wv, ln, ntile, acc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < ntile) {
          const int j = t * 16 + (ln & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = wv * 16 + 4 * (ln >> 4) + r;
            const float u = (i < m && j < m) ? ((i == j ? 2.f : 0.f) - acc[t][r]) : 0.f;
            sUt[j * NS_LD + i] = u;
          }
        }
      }
    }
    __syncthreads();
    // X_next = X_cur U
    const int nxt = cur ^ 1;
    if (active) {
      ns_product(sX[cur], sUt, ksteps, wv, ln, ntile, acc);
      float* xg = xs ? xs + (static_cast<size_t>(g) * (iters + 1) + it + 1) * mm : nullptr;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < ntile) {
          const int j = t * 16 + (ln & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = wv * 16 + 4 * (ln >> 4) + r;
            const float v = (i < m && j < m) ? acc[t][r] : 0.f;
            sX[nxt][i * NS_LD + j] = v;
            sXt[nxt][j * NS_LD + i] = v;
            if (xg && i < m && j < m) xg[i * m + j] = v;
          }
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }

  float* xo = Xout + g * mm;
  for (int idx = tid; idx < m * m; idx += 256) {
    const int i = idx / m, j = idx % m;
    xo[idx] = sX[cur][i * NS_LD + j];
  }

  if (resid) {
    // ||W X - I||_F
    double ss = 0.0;
    if (active) {
      ns_product(sW, sXt[cur], ksteps, wv, ln, ntile, acc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < ntile) {
          const int j = t * 16 + (ln & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = wv * 16 + 4 * (ln >> 4) + r;
            if (i < m && j < m) {
              const double e = static_cast<double>(acc[t][r]) - (i == j ? 1.0 : 0.0);
              ss += e * e;
            }
          }
        }
      }
    }
    __syncthreads();
    red[0][tid] = ss;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) red[0][tid] += red[0][tid + s];
      __syncthreads();
    }
    if (tid == 0) resid[g] = static_cast<float>(sqrt(red[0][0]));
  }
}

// =====================================================================================================
// m > 64: the m x m matrices do not fit one CU's LDS, so each product is its own launch of a batched
// 32 x 32-tile fp32 MFMA GEMM (4 waves of 16 x 16), with K staged through LDS in chunks of 32.
//   EPI 0: C = 2I - A B   (U = 2I - W X)
//   EPI 1: C = A B        (X_next = X U), optionally also written to C2
//   EPI 2: C = A B - I    (residual W X - I)
// =====================================================================================================
__global__ __launch_bounds__(256) void k_ns_init(const float* __restrict__ We, float* __restrict__ X0,
                                                 float* __restrict__ X0b, size_t strideX0b,
                                                 float* __restrict__ alpha_out, int m) {
  __shared__ double red[2][256];
  const int g = blockIdx.x, tid = threadIdx.x;
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  double cmax = 0.0, rmax = 0.0;
  for (int j = tid; j < m; j += 256) {
    double cs = 0.0, rs = 0.0;
    for (int i = 0; i < m; ++i) {
      cs += fabs(static_cast<double>(wg[static_cast<size_t>(i) * m + j]));
      rs += fabs(static_cast<double>(wg[static_cast<size_t>(j) * m + i]));
    }
    cmax = fmax(cmax, cs);
    rmax = fmax(rmax, rs);
  }
  red[0][tid] = cmax;
  red[1][tid] = rmax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] = fmax(red[0][tid], red[0][tid + s]);
      red[1][tid] = fmax(red[1][tid], red[1][tid + s]);
    }
    __syncthreads();
  }
  const float alpha = static_cast<float>(1.0 / (red[0][0] * red[1][0]));
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;
  float* x0 = X0 + g * mm;
  float* x0b = X0b ? X0b + g * strideX0b : nullptr;
  for (size_t idx = tid; idx < mm; idx += 256) {
    const size_t i = idx / m, j = idx % m;
    const float v = alpha * wg[j * m + i];
    x0[idx] = v;
    if (x0b) x0b[idx] = v;
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void k_ns_gemm(const float* __restrict__ A, size_t strideA,
                                                 const float* __restrict__ B, size_t strideB, float* __restrict__ C,
                                                 size_t strideC, float* __restrict__ C2, size_t strideC2, int m) {
  constexpr int LDA = 34;  // 2 mod 32
  constexpr int LDB = 48;  // 16 mod 32
  __shared__ float sA[32 * LDA];
  __shared__ float sB[32 * LDB];
  const int g = blockIdx.z;
  const int tm = blockIdx.y * 32, tn = blockIdx.x * 32;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const float* ag = A + g * strideA;
  const float* bg = B + g * strideB;
  const int wr = (wv >> 1) * 16, wc = (wv & 1) * 16;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < m; kc += 32) {
    __syncthreads();
    for (int idx = tid; idx < 32 * 32; idx += 256) {
      const int rr = idx >> 5, cc = idx & 31;
      const int ai = tm + rr, ak = kc + cc;
      sA[rr * LDA + cc] = (ai < m && ak < m) ? ag[static_cast<size_t>(ai) * m + ak] : 0.f;
      const int bk = kc + rr, bj = tn + cc;
      sB[rr * LDB + cc] = (bk < m && bj < m) ? bg[static_cast<size_t>(bk) * m + bj] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int k = ks * 4 + (ln >> 4);
      acc = mfma16x16x4(sA[(wr + (ln & 15)) * LDA + k], sB[k * LDB + wc + (ln & 15)], acc);
    }
  }
  const int j = tn + wc + (ln & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = tm + wr + 4 * (ln >> 4) + r;
    if (i < m && j < m) {
      float v = acc[r];
      if (EPI == 0) v = (i == j ? 2.f : 0.f) - v;
      if (EPI == 2) v -= (i == j ? 1.f : 0.f);
      C[g * strideC + static_cast<size_t>(i) * m + j] = v;
      if (EPI == 1 && C2) C2[g * strideC2 + static_cast<size_t>(i) * m + j] = v;
    }
  }
}

__global__ __launch_bounds__(256) void k_frob(const float* __restrict__ E, float* __restrict__ out, int m) {
  __shared__ double red[256];
  const size_t mm = static_cast<size_t>(m) * m;
  const float* e = E + blockIdx.x * mm;
  double s = 0.0;
  for (size_t idx = threadIdx.x; idx < mm; idx += 256) {
    const double v = e[idx];
    s += v * v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = static_cast<float>(sqrt(red[0]));
}

size_t ns_tmp_floats(const Shape& s) {
  return s.m > 64 ? 2 * static_cast<size_t>(s.G) * s.m * s.m : 0;
}

hipError_t launch_ns(const Shape& s, const float* We, float* X, float* xs, float* alpha, float* resid, float* tmp,
                     hipStream_t st) {
  const int m = s.m, K = s.ns_iters;
  if (m <= 64) {
    hipLaunchKernelGGL(k_ns_small, dim3(s.G), dim3(256), 0, st, We, X, xs, alpha, resid, m, K);
    return hipGetLastError();
  }
  const size_t mm = static_cast<size_t>(m) * m;
  float* U = tmp;
  float* Xalt = tmp + static_cast<size_t>(s.G) * mm;
  // Iterate X_k into buffers that alternate so that X_K lands in X. With xs, X_k also goes to slot k.
  float* bufs[2] = {X, Xalt};
  int cur = (K % 2 == 0) ? 0 : 1;
  const size_t xs_stride = static_cast<size_t>(K + 1) * mm;
  hipLaunchKernelGGL(k_ns_init, dim3(s.G), dim3(256), 0, st, We, bufs[cur], xs, xs_stride, alpha, m);
  const int tiles = (m + 31) / 32;
  const dim3 grid(tiles, tiles, s.G);
  for (int it = 0; it < K; ++it) {
    hipLaunchKernelGGL(k_ns_gemm<0>, grid, dim3(256), 0, st, We, mm, bufs[cur], mm, U, mm, nullptr, 0, m);
    const int nxt = cur ^ 1;
    float* xslot = xs ? xs + static_cast<size_t>(it + 1) * mm : nullptr;
    hipLaunchKernelGGL(k_ns_gemm<1>, grid, dim3(256), 0, st, bufs[cur], mm, U, mm, bufs[nxt], mm, xslot, xs_stride, m);
    cur = nxt;
  }
  if (resid) {
    hipLaunchKernelGGL(k_ns_gemm<2>, grid, dim3(256), 0, st, We, mm, X, mm, U, mm, nullptr, 0, m);
    hipLaunchKernelGGL(k_frob, dim3(s.G), dim3(256), 0, st, U, resid, m);
  }
  return hipGetLastError();
}

}  // namespace lf
