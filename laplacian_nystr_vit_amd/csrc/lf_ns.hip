// Newton-Schulz pseudo-inverse of the landmark kernel on MFMA (gfx950).
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
//
// Products run on the fp16 MFMA (v_mfma_f32_16x16x32_f16, 16x the fp32 MFMA rate on gfx950) with every fp32
// operand split as x = hi + lo (two fp16 values, about 22 significant bits) and
//   A B ~= A_hi B_hi + (A_hi B_lo + A_lo B_hi),
// accumulated in fp32. Three fp16 MFMAs cost less than a fifth of one fp32 MFMA product, and the result tracks an
// fp32 product to a few units of 1e-7.
// X carries a power-of-two scale so that its fp16 halves stay in range whatever the conditioning of W; W and
// U = 2I - W X need none (W's entries are at most 1 + eps and the eigenvalues of W X stay in (0, 1]).
//
// Matrices are zero-padded to 64 x 64 and kept K-contiguous in LDS, so each lane's 8-element fragment is one
// 16-byte read: W by rows (A operand of W X), U = 2I - W X by columns (B operand of X U), and X twice, by rows
// (A operand of X U) and by columns (B operand of W X). Wave w owns output row strip w; tile and K-chunk counts
// are template parameters, so the inner loop has no branches. (X_k is symmetric in exact arithmetic, but feeding
// its transpose to the update doubles the antisymmetric part of the rounding error every step, so both layouts
// are kept.)
// =====================================================================================================
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

constexpr int NH = 72;  // fp16 elements per LDS row: 64 + 8 (144-byte stride, 16-byte aligned)

struct alignas(16) SplitMat {
  _Float16 hi[64 * NH];
  _Float16 lo[64 * NH];
};

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// acc = A[16 wv .. +15][0 .. 32 KC) * B[0 .. 32 KC)[16 t .. +15] for t < NT, B given transposed (Bt[j][k]).
// All fragments are read first.
template <int NT, int KC>
__device__ __forceinline__ void prod_split(const SplitMat& A, const SplitMat& Bt, int wv, int ln, f32x4 acc[NT]) {
  const int i = wv * 16 + (ln & 15);
  const int kg = 8 * (ln >> 4);
  half8 ah[KC], al[KC], bh[KC][NT], bl[KC][NT];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int k0 = c * 32 + kg;
    ah[c] = *reinterpret_cast<const half8*>(&A.hi[i * NH + k0]);
    al[c] = *reinterpret_cast<const half8*>(&A.lo[i * NH + k0]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int j = t * 16 + (ln & 15);
      bh[c][t] = *reinterpret_cast<const half8*>(&Bt.hi[j * NH + k0]);
      bl[c][t] = *reinterpret_cast<const half8*>(&Bt.lo[j * NH + k0]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // One fp32 accumulator per tile takes hi*hi and both cross terms: each MFMA step rounds at fp32 relative to
  // the running sum, which keeps the product at fp32 accuracy.
#pragma unroll
  for (int c = 0; c < KC; ++c) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[c], bh[c][t], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[c], bl[c][t], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[c], bh[c][t], acc[t], 0, 0, 0);
  }
}

// Stores v (the 4 rows i0 .. i0+3 of column j) as the transposed split: Mt[j][i0 .. i0+3].
__device__ __forceinline__ void store_t4(SplitMat& Mt, int j, int i0, const float v[4]) {
  half4 h, l;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    _Float16 a, b;
    split_f16(v[r], a, b);
    h[r] = a;
    l[r] = b;
  }
  *reinterpret_cast<half4*>(&Mt.hi[j * NH + i0]) = h;
  *reinterpret_cast<half4*>(&Mt.lo[j * NH + i0]) = l;
}

__device__ __forceinline__ void store_rowmajor(SplitMat& M, int i, int j, float v) {
  _Float16 a, b;
  split_f16(v, a, b);
  M.hi[i * NH + j] = a;
  M.lo[i * NH + j] = b;
}

// Entries of X are kept below 2^14 in magnitude in the fp16 halves; X is stored as X * 2^-e.
constexpr float kScaleLimit = 16384.f;

template <int NT, int KC>
__global__ __launch_bounds__(256) void k_ns_small(const float* __restrict__ We, float* __restrict__ Xout,
                                                  float* __restrict__ xs, float* __restrict__ alpha_out,
                                                  float* __restrict__ resid, int m, int iters) {
  __shared__ SplitMat sW, sX, sXt, sUt;
  __shared__ double red[2][4][64];
  __shared__ float s_alpha;
  __shared__ unsigned int s_big;  // max |X| bits, written only when some entry exceeds the scale limit
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  float* wf = reinterpret_cast<float*>(&sUt);  // fp32 W (64 x 65) in the not yet used Ut area

  float wv16[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = tid + 256 * q;
    const int i = idx >> 6, j = idx & 63;
    wv16[q] = (i < m && j < m) ? wg[i * m + j] : 0.f;
  }
  {
    // zero the three split matrices that will be read before being fully written (16-byte stores)
    uint4* z0 = reinterpret_cast<uint4*>(&sW);
    uint4* z1 = reinterpret_cast<uint4*>(&sX);
    uint4* z2 = reinterpret_cast<uint4*>(&sXt);
    constexpr int NZ = static_cast<int>(sizeof(SplitMat) / sizeof(uint4));
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int q = tid; q < NZ; q += 256) {
      z0[q] = zero;
      z1[q] = zero;
      z2[q] = zero;
    }
  }
  if (tid == 0) s_big = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = tid + 256 * q;
    const int i = idx >> 6, j = idx & 63;
    wf[i * 65 + j] = wv16[q];
    store_rowmajor(sW, i, j, wv16[q]);
  }
  __syncthreads();

  // alpha = 1 / (max_j sum_i |W_ij| * max_i sum_j |W_ij|) in float64: thread (c, quarter) sums 16 entries of
  // column c and of row c, the quarters are combined, then wave 0 takes the maxima.
  {
    const int c = tid & 63, qtr = tid >> 6;
    double cs = 0.0, rs = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      cs += fabs(static_cast<double>(wf[(qtr * 16 + k) * 65 + c]));
      rs += fabs(static_cast<double>(wf[c * 65 + qtr * 16 + k]));
    }
    red[0][qtr][c] = cs;
    red[1][qtr][c] = rs;
  }
  __syncthreads();
  if (wv == 0) {
    double cs = red[0][0][ln] + red[0][1][ln] + red[0][2][ln] + red[0][3][ln];
    double rs = red[1][0][ln] + red[1][1][ln] + red[1][2][ln] + red[1][3][ln];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      cs = fmax(cs, __shfl_xor(cs, off));
      rs = fmax(rs, __shfl_xor(rs, off));
    }
    if (ln == 0) s_alpha = static_cast<float>(1.0 / (cs * rs));
  }
  __syncthreads();
  const float alpha = s_alpha;
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;

  // X_0 = alpha W^T: each wave keeps its own output tiles of the current X in fp32 registers.
  const bool active = wv < NT;
  float xcur[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = t * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = wv * 16 + 4 * (ln >> 4) + r;
      xcur[t][r] = active ? alpha * wf[j * 65 + i] : 0.f;
    }
  }
  __syncthreads();  // wf (inside sUt) is dead after this point
  int e = 0;        // sX and sXt hold X * 2^-e
  if (active) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int j = t * 16 + (ln & 15);
      const int i0 = wv * 16 + 4 * (ln >> 4);
      store_t4(sXt, j, i0, xcur[t]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        store_rowmajor(sX, i0 + r, j, xcur[t][r]);
        if (xs && i0 + r < m && j < m) xs[static_cast<size_t>(g) * (iters + 1) * mm + (i0 + r) * m + j] = xcur[t][r];
      }
    }
  }
  {
    uint4* z3 = reinterpret_cast<uint4*>(&sUt);
    constexpr int NZ = static_cast<int>(sizeof(SplitMat) / sizeof(uint4));
    for (int q = tid; q < NZ; q += 256) z3[q] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  // Constant part of U = 2I - T on the m x m block (zero outside it).
  float two_i[NT][4];
  bool inside[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = t * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = wv * 16 + 4 * (ln >> 4) + r;
      inside[t][r] = i < m && j < m;
      two_i[t][r] = (i == j && i < m) ? 2.f : 0.f;
    }
  }

  f32x4 acc[NT];
  for (int it = 0; it < iters; ++it) {
    const float unscale = ldexpf(1.f, e);
    // T = W X ; Ut = (2I - T)^T
    if (active) {
      prod_split<NT, KC>(sW, sXt, wv, ln, acc);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int j = t * 16 + (ln & 15);
        const int i0 = wv * 16 + 4 * (ln >> 4);
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = inside[t][r] ? two_i[t][r] - acc[t][r] * unscale : 0.f;
        store_t4(sUt, j, i0, u);
      }
    }
    __syncthreads();
    // X_next = X U
    if (active) {
      prod_split<NT, KC>(sX, sUt, wv, ln, acc);
      float lmax = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xcur[t][r] = acc[t][r] * unscale;
          lmax = fmaxf(lmax, fabsf(xcur[t][r]));
        }
      if (lmax > ldexpf(kScaleLimit, e)) atomicMax(&s_big, __float_as_uint(lmax));  // rare
    }
    __syncthreads();  // all reads of sX / sXt are done; s_big is final
    const unsigned int big = s_big;
    if (big != 0u) {
      const float mx = __uint_as_float(big);
      while (ldexpf(kScaleLimit, e) < mx) ++e;
    }
    const float scale = ldexpf(1.f, -e);
    if (active) {
      float* xg = xs ? xs + (static_cast<size_t>(g) * (iters + 1) + it + 1) * mm : nullptr;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int j = t * 16 + (ln & 15);
        const int i0 = wv * 16 + 4 * (ln >> 4);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = xcur[t][r] * scale;
          store_rowmajor(sX, i0 + r, j, v[r]);
          if (xg && inside[t][r]) xg[(i0 + r) * m + j] = xcur[t][r];
        }
        store_t4(sXt, j, i0, v);
      }
    }
    __syncthreads();
    if (tid == 0) s_big = 0u;
  }

  float* xo = Xout + g * mm;
  if (active) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int j = t * 16 + (ln & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wv * 16 + 4 * (ln >> 4) + r;
        if (inside[t][r]) xo[i * m + j] = xcur[t][r];
      }
    }
  }

  if (resid) {
    // ||W X - I||_F with the same split products
    double ss = 0.0;
    if (active) {
      prod_split<NT, KC>(sW, sXt, wv, ln, acc);
      const float unscale = ldexpf(1.f, e);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inside[t][r]) {
            const double e2 = static_cast<double>(acc[t][r] * unscale) - 0.5 * two_i[t][r];
            ss += e2 * e2;
          }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    __syncthreads();
    if (ln == 0) red[0][0][wv] = ss;
    __syncthreads();
    if (tid == 0) resid[g] = static_cast<float>(sqrt(red[0][0][0] + red[0][0][1] + red[0][0][2] + red[0][0][3]));
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
    const int nt = (m + 15) / 16;
    const dim3 grid(s.G), block(256);
    if (nt == 1)
      hipLaunchKernelGGL((k_ns_small<1, 1>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else if (nt == 2)
      hipLaunchKernelGGL((k_ns_small<2, 1>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else if (nt == 3)
      hipLaunchKernelGGL((k_ns_small<3, 2>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else
      hipLaunchKernelGGL((k_ns_small<4, 2>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
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
