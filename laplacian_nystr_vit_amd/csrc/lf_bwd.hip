// Backward pass of the LaplacianFormer attention block for gfx950 (m <= 64, d <= 64).
//
// [note] = papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力";
// [abs]  = the arXiv 2604.20368 abstract, which states that the kernel and the solver have forward and backward
//          implementations.
// The gradient of k(x, l) = exp(-||x - l||_1 / lambda) is -(1/lambda) sign(x - l) k in x and +(1/lambda)
// sign(x - l) k in l ([note] motivation, "core idea", with the minus sign the page drops restored; sign(0) = 0).
// alpha of the Newton-Schulz start is held constant.
//
// Per slice, with A_hat = C_Q (or its whitened form), S = C_K^T V, P = X_K S, Y = A_hat P + DWC(V):
//   dP = A_hat^T dY          dA_hat = dY P^T        dX_K = dP S^T      dS = X_K^T dP
//   dV = C_K dS + DWC^T(dY)  dC_K = V dS^T
//   whitening: dC_Q = rstd (dA_hat - mean_i dA_hat - A_hat mean_i(dA_hat A_hat))
//   Newton-Schulz reverse (X_{k+1} = 2 X_k - X_k W X_k):  dW -= X_k^T G X_k^T ; G <- 2G - G (W X_k)^T - (X_k W)^T G
//   and finally dW += alpha G^T (X_0 = alpha W^T).
//   Gq = dC_Q C_Q / lambda, Gk = dC_K C_K / lambda, Gw = dW W / lambda (off the diagonal)
//   dQ = -sum_l Gq sign(Q - L) ; dK = -sum_l Gk sign(K - L)
//   dL = sum_i Gq sign(Q - L) + sum_j Gk sign(K - L) - sum_l' (Gw + Gw^T) sign(L - L')
//   dQ_i += dL_{owner(i)} / r^2 (landmarks are r x r block means of Q).
// Both column means of the whitening backward come from m x d products: mean_i dA_hat[:, l] = (1/N) P_l . (1^T dY)
// and mean_i (dA_hat A_hat)[:, l] = (1/N) P_l . dP_l, so no extra pass over the N x m matrices is needed.
#include <type_traits>

#include "../../include/lf_attn.h"
#include "lf_bwd_internal.h"
#include "lf_device.h"
#include "lf_split.h"

namespace lf {

static inline int cdiv(long a, long b) { return static_cast<int>((a + b - 1) / b); }

constexpr int kFragUnits = 2048;
constexpr int kDwcThreads = 256;  // DWC weight gradient: threads per block
constexpr int kDwcRun = 8;        // DWC weight gradient: tokens per work item (a run along a grid row)  // 16-byte units of the backward Newton-Schulz chain's fragments per (slice, step)
__device__ __forceinline__ float sgnf(float x) { return x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f); }

// sign(x - l) from xs = x 2^100 (exact): fmaf(l, -2^100, xs) is (x - l) 2^100 rounded once, and its median with -1
// and 1 is the sign whenever x == l or |x - l| >= 2^-100 (for |l| < 2^28; a larger difference may round to +-inf,
// which keeps its sign). Two VALU operations where the three-way sign takes two compares and two selects; an fp32
// difference of values of order one is 0 or at least 2^-24 in magnitude.
constexpr float kSgnScale = 0x1p100f;
__device__ __forceinline__ float sgn_of_scaled(float xs, float l) {
  return __builtin_amdgcn_fmed3f(fmaf(l, -kSgnScale, xs), -1.f, 1.f);
}

// Sign reductions (k_bwd_sign): row sub-tiles per block (the block has kSignSub * D threads) and token rows per
// thread.
constexpr int kSignSub = 8;
constexpr int kSignRt = 8;

namespace {

struct BwdWs {
  size_t T1, part, dX, dS, stats, dWe, dLW, Gq, Gk, dLpart, dQp, lampart, dwcpart, nsA1, nsA2, nsG, nsD, nsGf, total;
  int nsplitS;
  int lamchunks, dwcseg, dwcblocks;
};

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

BwdWs plan(const Shape& s) {
  const size_t G = s.G, N = s.N, m = s.m, d = s.d;
  int nsplit, rps;
  ckv_split(s, &nsplit, &rps);
  BwdWs w;
  // Sign reductions (k_bwd_sign): blocks of kSignSub * kSignRt token rows per slice.
  w.nsplitS = cdiv(s.N, kSignSub * kSignRt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al(off + bytes);
    return o;
  };
  w.T1 = take(4 * G * (m + 1) * d);
  w.part = take(nsplit > 1 ? 4 * G * nsplit * (m + 1) * d : 0);
  w.dX = take(4 * G * m * m);
  w.dS = take(4 * G * m * d);
  w.stats = take(4 * G * 2 * m);
  w.dWe = take(4 * G * m * m);
  w.dLW = take(4 * G * m * d);
  w.Gq = take(4 * G * N * m);
  w.Gk = take(4 * G * N * m);
  w.dLpart = take(4 * G * static_cast<size_t>(w.nsplitS) * m * d);
  w.dQp = take(4 * G * N * d);
  // lambda gradient: per slice, chunks of 64 landmarks' worth of kernel entries; DWC weight gradient: per slice,
  // one [9][d] partial per block of runs of kDwcRun tokens (dwcseg runs per grid row)
  // lambda-gradient partials: one per row-gradient block (2 sides x 64-token tiles) and one per landmark row of W
  w.lamchunks = 2 * cdiv(N, 64) + m;
  w.lampart = take(4 * G * static_cast<size_t>(w.lamchunks));
  w.dwcseg = cdiv(s.W, kDwcRun);
  w.dwcblocks = cdiv(static_cast<long>(s.H) * w.dwcseg, kDwcThreads / (s.d / 4));
  w.dwcpart = take(4 * G * static_cast<size_t>(w.dwcblocks) * 9 * d);
  // Newton-Schulz reverse chain: A1_k, A2_k, G_k and D_k for every step, and the final adjoint, each m x m
  const size_t nsk = 4 * G * static_cast<size_t>(s.ns_iters) * m * m;
  w.nsA1 = take(G * static_cast<size_t>(s.ns_iters) * kFragUnits * 16);  // split fragments of A1_k and A2_k^T
  w.nsA2 = take(8 * G * static_cast<size_t>(s.ns_iters));                 // per-step scale exponent and bound
  w.nsG = take(4 * G * static_cast<size_t>(s.ns_iters) * 4096);  // G_k as zero-padded 64 x 64 tiles
  w.nsD = take(nsk);
  w.nsGf = take(4 * G * m * m);
  w.total = off;
  return w;
}

}  // namespace

// ---------------------------------------------------------------------------------------------------------
// Small per-slice products: dP from T1 = [C_Q | 1]^T dY, then dX = dP S^T, dS = X_K^T dP and the two whitening
// column means. m x m x d work per slice, on the VALU. The slice's output rows are spread over gridDim.y blocks
// (rows l = blockIdx.y, blockIdx.y + gridDim.y, ...); each block forms the whole dP, which every dS row needs.
// ---------------------------------------------------------------------------------------------------------
// Up to MAXN floats of a flat array, spread over the NT threads of a block (element it * NT + threadIdx.x in v[it]).
// Loads go to clamped addresses (n >= 1), so a block can issue the loads of several arrays before the first LDS
// store and wait for one memory round trip instead of one per array.
template <int NT, int MAXN>
struct FlatRegs {
  static constexpr int IT = (MAXN + NT - 1) / NT;
  float v[IT];
  __device__ __forceinline__ void load(const float* __restrict__ src, int n) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = static_cast<int>(threadIdx.x) + it * NT;
      v[it] = src[idx < n ? idx : 0];
    }
  }
  __device__ __forceinline__ void store(float* __restrict__ dst, int n) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = static_cast<int>(threadIdx.x) + it * NT;
      if (idx < n) dst[idx] = v[it];
    }
  }
};

template <int D>
__global__ __launch_bounds__(256) void k_bwd_small1(const float* __restrict__ T1, const float* __restrict__ S,
                                                    const float* __restrict__ P, const float* __restrict__ xs,
                                                    const float* __restrict__ mu, const float* __restrict__ rstd,
                                                    float* __restrict__ dX, float* __restrict__ dS,
                                                    float* __restrict__ stats, int m, int K, int N, int whiten) {
  __shared__ float sT1[65 * D];
  __shared__ float sS[64 * D];
  __shared__ float sP[64 * D];
  __shared__ float sdP[64 * D];
  __shared__ float sX[64 * 64];
  __shared__ float sMu[64], sRs[64];
  const int g = blockIdx.x, part = blockIdx.y, nparts = gridDim.y, tid = threadIdx.x;
  const size_t md = static_cast<size_t>(m) * D, mm = static_cast<size_t>(m) * m;
  const float* t1 = T1 + static_cast<size_t>(g) * (m + 1) * D;
  // every load (T1, S, P, X_K and the whitening mean and scale) in flight before the first LDS store
  FlatRegs<256, 65 * D> rT;
  FlatRegs<256, 64 * D> rS, rP;
  FlatRegs<256, 64 * 64> rX;
  rT.load(t1, (m + 1) * D);
  rS.load(S + g * md, m * D);
  rP.load(P + g * md, m * D);
  rX.load(xs + (static_cast<size_t>(g) * (K + 1) + K) * mm, m * m);
  float mu_v = 0.f, rs_v = 1.f;
  if (whiten && tid < m) {
    mu_v = mu[g * m + tid];
    rs_v = rstd[g * m + tid];
  }
  rT.store(sT1, (m + 1) * D);
  rS.store(sS, m * D);
  rP.store(sP, m * D);
  rX.store(sX, m * m);
  if (tid < m) {
    sMu[tid] = mu_v;
    sRs[tid] = rs_v;
  }
  __syncthreads();
  for (int idx = tid; idx < m * D; idx += 256) {
    const int l = idx / D, c = idx % D;
    float v = sT1[idx];
    if (whiten) v = sRs[l] * (v - sMu[l] * sT1[m * D + c]);
    sdP[idx] = v;
  }
  __syncthreads();
  const int rows = (m - part + nparts - 1) / nparts;  // this block's rows: l = part + nparts q, q < rows
  for (int idx = tid; idx < rows * m; idx += 256) {
    const int l = part + nparts * (idx / m), k = idx % m;
    float acc = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) acc += sdP[l * D + c] * sS[k * D + c];
    dX[g * mm + static_cast<size_t>(l) * m + k] = acc;
  }
  for (int idx = tid; idx < rows * D; idx += 256) {
    const int l = part + nparts * (idx / D), c = idx % D;
    float acc = 0.f;
#pragma unroll 7
    for (int k = 0; k < m; ++k) acc += sX[k * m + l] * sdP[k * D + c];
    dS[g * md + static_cast<size_t>(l) * D + c] = acc;
  }
  if (whiten) {
    for (int q = tid; q < rows; q += 256) {
      const int l = part + nparts * q;
      float a = 0.f, b = 0.f;
      for (int c = 0; c < D; ++c) {
        a += sT1[m * D + c] * sP[l * D + c];
        b += sP[l * D + c] * sdP[l * D + c];
      }
      stats[static_cast<size_t>(g) * 2 * m + l] = a / static_cast<float>(N);
      stats[static_cast<size_t>(g) * 2 * m + m + l] = b / static_cast<float>(N);
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// Newton-Schulz reverse chain. With X_{k+1} = 2 X_k - X_k W X_k and G the adjoint of X_{k+1}, step k (from K - 1
// down to 0) gives
//   dW -= X_k^T G X_k^T,    G <- 2G - G (W X_k)^T - (X_k W)^T G.
// Only the second line is a chain: A1_k = W X_k and A2_k = X_k W depend on the saved iterates alone, and the dW
// terms feed nothing back. So the work runs as four launches (64 x 64 zero-padded tiles in LDS):
//   k_bwd_ns_pre   A1_k and A2_k for every (slice, step), all in parallel (fp32 MFMA), written as scaled
//                  split-fp16 operand fragments;
//   k_bwd_ns_chain one block (16 waves) per slice: per step one phase of two split-fp16 products,
//                  G <- 2G - (G A1_k^T + A2_k^T G), storing each step's G_k;
//   k_bwd_ns_dk    D_k = X_k^T G_k X_k^T for every (slice, step), all in parallel;
//   k_bwd_ns_final dW = -sum_k D_k (k from K - 1 down to 0) + alpha G_0^T (X_0 = alpha W^T), plus the path through
//                  alpha when asked; blocks of 256 entries.
// G_k is [G][K][64][64] float32 (zero-padded) and D_k [G][K][m][m] float32 in the workspace.
// ---------------------------------------------------------------------------------------------------------
constexpr int BL = 66;

// acc[t] += op(A)[strip rows][:] op(B)[:][tile t0 + t] over k = 0..63, with op = transpose when TA / TB.
template <bool TA, bool TB, int NT>
__device__ __forceinline__ void mm64u(const float* __restrict__ sA, const float* __restrict__ sB, int strip, int t0,
                                      int ln, f32x4 acc[NT]) {
  const int i = strip * 16 + (ln & 15);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int k = ks * 4 + (ln >> 4);
    const float a = TA ? sA[k * BL + i] : sA[i * BL + k];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int j = (t0 + t) * 16 + (ln & 15);
      const float b = TB ? sB[j * BL + k] : sB[k * BL + j];
      acc[t] = mfma16x16x4(a, b, acc[t]);
    }
  }
}

template <int NT>
__device__ __forceinline__ void zero_n(f32x4 acc[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Row strip `strip`, tiles t0 .. t0 + NT - 1 of a 64 x 64 LDS matrix from accumulator tiles.
template <int NT>
__device__ __forceinline__ void store_tiles(float* __restrict__ sC, const f32x4 acc[NT], int strip, int t0, int ln) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = (t0 + t) * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) sC[(strip * 16 + 4 * (ln >> 4) + r) * BL + j] = acc[t][r];
  }
}

// Zero-padded 64 x 64 copy (row stride BL) of an m x m matrix from global memory, by the NT threads of the block,
// every load issued before the first store.
template <int NT>
__device__ __forceinline__ void stage_mm(float* __restrict__ sM, const float* __restrict__ src, int m) {
  constexpr int IT = 64 * 64 / NT;
  float v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = static_cast<int>(threadIdx.x) + it * NT;
    const int i = idx >> 6, j = idx & 63;
    v[it] = (i < m && j < m) ? src[i * m + j] : 0.f;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = static_cast<int>(threadIdx.x) + it * NT;
    sM[(idx >> 6) * BL + (idx & 63)] = v[it];
  }
}

// Accumulator tiles of row strip `strip`, tiles t0 .. t0 + NT - 1, to an m x m matrix in global memory.
template <int NT>
__device__ __forceinline__ void store_tiles_mm(float* __restrict__ dst, const f32x4 acc[NT], int strip, int t0, int ln,
                                               int m) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = (t0 + t) * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = strip * 16 + 4 * (ln >> 4) + r;
      if (i < m && j < m) dst[i * m + j] = acc[t][r];
    }
  }
}

constexpr int NSB_THREADS = 512;  // 8 waves

// The per-(slice, step) launches deal their blocks so that every block of slice g runs on the XCD that runs the
// chain block of slice g (blocks go to the 8 XCDs round-robin by linear index): what they write for the chain, and
// what they read of its output, stays in that XCD's L2. False for the padding blocks when G is not a multiple of 8.
__device__ __forceinline__ bool slice_step_of(int b, int K, int G, int& g, int& k) {
  const int q = b >> 3;
  const int grp = q / K;
  g = grp * 8 + (b & 7);
  k = q - grp * K;
  return g < G;
}

typedef _Float16 bh8 __attribute__((ext_vector_type(8)));
typedef _Float16 bh4 __attribute__((ext_vector_type(4)));
typedef float bf8 __attribute__((ext_vector_type(8)));

// Exponent e with mx 2^-e in [2^12, 2^13) (0 for mx = 0; subnormals count as 2^-126).
__device__ __forceinline__ int ns_scale_exp(float mx) {
  if (!(mx > 0.f)) return 0;
  const int bexp = static_cast<int>((__float_as_uint(mx) >> 23) & 0xffu);
  return (bexp == 0 ? 1 : bexp) - 127 - 12;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Largest v over the wave, in every lane: max within quads (quad_perm [1,0,3,2], [2,3,0,1]), across the quads of a
// 16-lane row (row_ror 4, 8), then over the four rows through scalar reads of lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// Split-fp16 operand fragments of the chain, per (slice, step) kFragUnits units of 16 bytes. Unit
// (((mat * 4 + strip) * 2 + c) * 2 + h) * 64 + lane holds half h (0: hi = round_f16(v), 1: lo = round_f16(v - hi))
// of entries 32 c + 8 (lane / 16) .. + 7 of row strip * 16 + lane % 16 of A1_k 2^-f (mat 0) or A2_k^T 2^-f
// (mat 1): the operand a lane supplies to v_mfma_f32_16x16x32_f16 as B of G A1_k^T and as A of A2_k^T G.

// Block (slice, step) as dealt by slice_step_of: A1_k = W X_k (waves 0-3, one row strip each) and A2_k = X_k W
// (waves 4-7), both scaled by 2^-f so that the largest entry of either sits in [2^12, 2^13), written as chain
// fragments. sc[2 (g K + k)] = f and sc[2 (g K + k) + 1] = gamma_k = 2 + m (max|A1_k| + max|A2_k|), a bound on
// max|G_new| / max|G| over one chain step (each entry of G A1^T is a sum of m terms |G| |A1|, and likewise A2^T G).
__global__ __launch_bounds__(NSB_THREADS) void k_bwd_ns_pre(const float* __restrict__ We, const float* __restrict__ xs,
                                                             bh8* __restrict__ frag, float* __restrict__ sc, int m,
                                                             int K, int G) {
  __shared__ float sW[64 * BL];
  __shared__ float sX[64 * BL];
  __shared__ float s_red[8];
  int g, k;
  if (!slice_step_of(static_cast<int>(blockIdx.x), K, G, g, k)) return;
  const int tid = threadIdx.x, ln = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const size_t mm = static_cast<size_t>(m) * m;
  stage_mm<NSB_THREADS>(sW, We + g * mm, m);
  stage_mm<NSB_THREADS>(sX, xs + (static_cast<size_t>(g) * (K + 1) + k) * mm, m);
  __syncthreads();
  f32x4 acc[4];
  zero_n<4>(acc);
  if (wv < 4)
    mm64u<false, false, 4>(sW, sX, wv, 0, ln, acc);  // W X_k
  else
    mm64u<false, false, 4>(sX, sW, wv - 4, 0, ln, acc);  // X_k W
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[t][r]));
  mx = wave_max(mx);
  if (ln == 0) s_red[wv] = mx;
  __syncthreads();  // also: every wave is done reading sW and sX
  const float m1 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float m2 = fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7]));
  const int f = ns_scale_exp(fmaxf(m1, m2));
  const int strip = wv & 3;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = t * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = strip * 16 + 4 * (ln >> 4) + r;
      const float v = ldexpf(acc[t][r], -f);
      if (wv < 4)
        sW[i * BL + j] = v;  // A1 2^-f
      else
        sX[j * BL + i] = v;  // A2^T 2^-f
    }
  }
  __syncthreads();
  bh8* out = frag + (static_cast<size_t>(g) * K + k) * kFragUnits;
  for (int u = tid; u < kFragUnits / 2; u += NSB_THREADS) {
    const int L = u & 63, c = (u >> 6) & 1, s = (u >> 7) & 3, mat = u >> 9;
    const float* row = (mat ? sX : sW) + (s * 16 + (L & 15)) * BL + 32 * c + 8 * (L >> 4);
    bf8 v;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = row[t];
    const bh8 h = __builtin_convertvector(v, bh8);
    const bh8 l = __builtin_convertvector(v - __builtin_convertvector(h, bf8), bh8);
    const int base = ((mat * 4 + s) * 2 + c) * 2;
    out[base * 64 + L] = h;
    out[(base + 1) * 64 + L] = l;
  }
  if (tid == 0) {
    sc[2 * (static_cast<size_t>(g) * K + k)] = static_cast<float>(f);
    sc[2 * (static_cast<size_t>(g) * K + k) + 1] = 2.f + static_cast<float>(m) * (m1 + m2);
  }
}

constexpr int NHB = 72;  // fp16 per LDS row of the split adjoint: 144-byte stride, conflict-free 16-byte reads

// The 4 entries G[i0 .. i0+3][j] of a lane's tile, scaled by 2^-e and split into fp16 halves, into the row-major
// (rh, rl) and transposed (ch, cl) copies of the split adjoint.
__device__ __forceinline__ void put_split(_Float16* __restrict__ rh, _Float16* __restrict__ rl,
                                          _Float16* __restrict__ ch, _Float16* __restrict__ cl, const float Gr[4],
                                          int e, int i0, int j) {
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ldexpf(Gr[r], -e);
  const bh4 h = __builtin_convertvector(v, bh4);
  const bh4 l = __builtin_convertvector(v - __builtin_convertvector(h, f32x4), bh4);
  *reinterpret_cast<bh4*>(&ch[j * NHB + i0]) = h;
  *reinterpret_cast<bh4*>(&cl[j * NHB + i0]) = l;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rh[(i0 + r) * NHB + j] = h[r];
    rl[(i0 + r) * NHB + j] = l[r];
  }
}

// One block per slice: the adjoint chain G <- 2G - (G A1_k^T + A2_k^T G), k = K-1 .. 0, one barrier per step.
// Sixteen waves; wave w owns tile (row strip w & 3, column strip w >> 2) of G and keeps it in fp32 registers (the
// 2G term, the stored G_k and the final G are exact fp32). The products run on v_mfma_f32_16x16x32_f16 with split
// operands (hi hi + hi lo + lo hi, fp32 accumulation): G is kept in LDS as G 2^-e in fp16 halves, row-major (A of
// G A1^T) and transposed (B of A2^T G), double-buffered; the step's A1 / A2 fragments come from the precompute,
// loaded into registers four steps ahead and copied into LDS (double-buffered) one step ahead. The exponent of
// the next G follows from max|G_k| (a DPP wave maximum, combined through LDS in the previous step) and the bound
// gamma_k, so the new G is split before the barrier with its bound below 2^14: no fp16 overflow, and the fp16
// subnormal range starts 2^-38 below that bound.
constexpr int NSC_THREADS = 1024;
__global__ __launch_bounds__(NSC_THREADS) void k_bwd_ns_chain(const bh8* __restrict__ frag,
                                                               const float* __restrict__ sc,
                                                               const float* __restrict__ dX, float* __restrict__ Gs,
                                                               float* __restrict__ Gfin, int m, int K) {
  __shared__ __attribute__((aligned(16))) _Float16 sGr[2][2][64 * NHB];
  __shared__ __attribute__((aligned(16))) _Float16 sGc[2][2][64 * NHB];
  __shared__ bh8 sA[2][kFragUnits];
  __shared__ float s_max[2][16];
  __shared__ float s_sc[2 * LF_NS_ITERS_MAX];
  const int g = blockIdx.x, tid = threadIdx.x, ln = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int si = wv & 3, sj = wv >> 2;
  const int i0 = si * 16 + 4 * (ln >> 4), jj = sj * 16 + (ln & 15);
  const size_t mm = static_cast<size_t>(m) * m;
  for (int q = tid; q < 2 * K; q += NSC_THREADS) s_sc[q] = sc[2 * static_cast<size_t>(g) * K + q];
  float Gr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) Gr[r] = (i0 + r < m && jj < m) ? dX[g * mm + (i0 + r) * m + jj] : 0.f;
  const bh8* fg = frag + static_cast<size_t>(g) * K * kFragUnits;
  // Fragments of later steps in flight in three register slots: step j (the t-th step run, t = K - 1 - j) uses
  // slot t % 3, loaded four steps ahead of its use and copied to LDS one step ahead.
  bh8 pr[3][2];
  auto issue = [&](bh8 (&slot)[2], int j) {
    slot[0] = fg[static_cast<size_t>(j) * kFragUnits + tid];
    slot[1] = fg[static_cast<size_t>(j) * kFragUnits + tid + NSC_THREADS];
  };
  if (K > 0) {
    sA[0][tid] = fg[static_cast<size_t>(K - 1) * kFragUnits + tid];
    sA[0][tid + NSC_THREADS] = fg[static_cast<size_t>(K - 1) * kFragUnits + tid + NSC_THREADS];
  }
  if (K > 1) issue(pr[1], K - 2);
  if (K > 2) issue(pr[2], K - 3);
  if (K > 3) issue(pr[0], K - 4);
  float lm = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) lm = fmaxf(lm, fabsf(Gr[r]));
  lm = wave_max(lm);
  if (ln == 0) s_max[0][wv] = lm;
  lds_barrier();
  float M = s_max[0][0];
#pragma unroll
  for (int q = 1; q < 16; ++q) M = fmaxf(M, s_max[0][q]);
  int e = ns_scale_exp(M);
  put_split(sGr[0][0], sGr[0][1], sGc[0][0], sGc[0][1], Gr, e, i0, jj);
  int cur = 0;
  // G_k goes out as a 64 x 64 tile (zero padding included) with unconditional stores, so the count of memory
  // operations in flight is the same on every path and the waits for the fragment slots stay partial.
  float* gs_base = Gs + static_cast<size_t>(g) * K * 4096 + i0 * 64 + jj;
  auto step = [&](auto tc, int k) __attribute__((always_inline)) {
    constexpr int sw = (decltype(tc)::value + 1) % 3;  // slot of step k - 1
    lds_barrier();  // split G_k, the step's fragments and max|G_k| are complete; step k + 1's reads are done
    const int nxt = cur ^ 1;
    M = s_max[cur][0];
#pragma unroll
    for (int q = 1; q < 16; ++q) M = fmaxf(M, s_max[cur][q]);
    if (k > 0) {
      sA[nxt][tid] = pr[sw][0];
      sA[nxt][tid + NSC_THREADS] = pr[sw][1];
      if (k > 3) issue(pr[sw], k - 4);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) gs_base[static_cast<size_t>(k) * 4096 + r * 64] = Gr[r];
    f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int k0 = 32 * c + 8 * (ln >> 4);
      const bh8 gh = *reinterpret_cast<const bh8*>(&sGr[cur][0][(si * 16 + (ln & 15)) * NHB + k0]);
      const bh8 gl = *reinterpret_cast<const bh8*>(&sGr[cur][1][(si * 16 + (ln & 15)) * NHB + k0]);
      const bh8 th = *reinterpret_cast<const bh8*>(&sGc[cur][0][(sj * 16 + (ln & 15)) * NHB + k0]);
      const bh8 tl = *reinterpret_cast<const bh8*>(&sGc[cur][1][(sj * 16 + (ln & 15)) * NHB + k0]);
      const int u1 = ((sj * 2 + c) * 2) * 64 + ln;       // mat 0, strip sj
      const int u2 = (((4 + si) * 2 + c) * 2) * 64 + ln;  // mat 1, strip si
      const bh8 b1h = sA[cur][u1], b1l = sA[cur][u1 + 64];
      const bh8 a2h = sA[cur][u2], a2l = sA[cur][u2 + 64];
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(gh, b1h, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, th, a2, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(gh, b1l, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2h, tl, a2, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(gl, b1h, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2l, th, a2, 0, 0, 0);
    }
    const int f = static_cast<int>(s_sc[2 * k]);
    const int en = M > 0.f ? ns_scale_exp(M * s_sc[2 * k + 1]) - 1 : 0;
    lm = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Gr[r] = 2.f * Gr[r] - ldexpf(a1[r] + a2[r], e + f);
      lm = fmaxf(lm, fabsf(Gr[r]));
    }
    lm = wave_max(lm);
    if (ln == 0) s_max[nxt][wv] = lm;
    put_split(sGr[nxt][0], sGr[nxt][1], sGc[nxt][0], sGc[nxt][1], Gr, en, i0, jj);
    e = en;
    cur = nxt;
  };
  using T0 = std::integral_constant<int, 0>;
  using T1 = std::integral_constant<int, 1>;
  using T2 = std::integral_constant<int, 2>;
  int k = K - 1;
  for (; k >= 2; k -= 3) {
    step(T0{}, k);
    step(T1{}, k - 1);
    step(T2{}, k - 2);
  }
  if (k >= 0) step(T0{}, k);
  if (k >= 1) step(T1{}, k - 1);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (i0 + r < m && jj < m) Gfin[g * mm + (i0 + r) * m + jj] = Gr[r];
}

// Block (slice, step) as dealt by slice_step_of: D_k = X_k^T (G_k X_k^T), each product on all 8 waves (row
// strip w & 3, tiles 2 (w >> 2) .. + 1).
__global__ __launch_bounds__(NSB_THREADS) void k_bwd_ns_dk(const float* __restrict__ xs, const float* __restrict__ Gs,
                                                            float* __restrict__ Dk, int m, int K, int G) {
  __shared__ float sX[64 * BL];
  __shared__ float sG[64 * BL];
  __shared__ float sY[64 * BL];
  int g, k;
  if (!slice_step_of(static_cast<int>(blockIdx.x), K, G, g, k)) return;
  const int ln = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const size_t mm = static_cast<size_t>(m) * m;
  stage_mm<NSB_THREADS>(sX, xs + (static_cast<size_t>(g) * (K + 1) + k) * mm, m);
  {
    const float* src = Gs + (static_cast<size_t>(g) * K + k) * 4096;  // 64 x 64 tiles, zero-padded
    constexpr int IT = 64 * 64 / NSB_THREADS;
    float v[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) v[it] = src[threadIdx.x + it * NSB_THREADS];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = static_cast<int>(threadIdx.x) + it * NSB_THREADS;
      sG[(idx >> 6) * BL + (idx & 63)] = v[it];
    }
  }
  __syncthreads();
  const int strip = wv & 3, t0 = 2 * (wv >> 2);
  f32x4 acc[2];
  zero_n<2>(acc);
  mm64u<false, true, 2>(sG, sX, strip, t0, ln, acc);  // G_k X_k^T
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = (t0 + t) * 16 + (ln & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) sY[(strip * 16 + 4 * (ln >> 4) + r) * BL + j] = acc[t][r];
  }
  __syncthreads();
  zero_n<2>(acc);
  mm64u<true, false, 2>(sX, sY, strip, t0, ln, acc);  // X_k^T (G_k X_k^T)
  store_tiles_mm<2>(Dk + (static_cast<size_t>(g) * K + k) * mm, acc, strip, t0, ln, m);
}

// Block (chunk of 256 entries, g): dW = -sum_k D_k (k from K - 1 down to 0) + alpha G_0^T, eight D_k loads in
// flight per thread. With exact_alpha also the path through alpha = 1 / (c r), c the largest column sum and r the
// largest row sum of |W|: d alpha = <G_0, W^T> and dW += d alpha * d alpha / dW, taken at the first largest column
// and row (every block of the slice forms these few reductions itself, in a fixed order).
constexpr int NSF_THREADS = 256;
__global__ __launch_bounds__(NSF_THREADS) void k_bwd_ns_final(const float* __restrict__ We,
                                                               const float* __restrict__ alpha,
                                                               const float* __restrict__ Dk,
                                                               const float* __restrict__ Gfin,
                                                               float* __restrict__ dWe, int m, int K,
                                                               int exact_alpha) {
  constexpr int NW = NSF_THREADS / 64;
  __shared__ float s_cs[64], s_rs[64], s_part[NW];
  __shared__ int s_arg[2];
  __shared__ float s_da;
  const int g = blockIdx.y, tid = threadIdx.x, ln = lane_id(), wv = wave_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  const float* gf = Gfin + g * mm;
  const float a = alpha[g];
  float da = 0.f, inv_c = 0.f, inv_r = 0.f;
  int jc = 0, ir = 0;
  if (exact_alpha) {
    if (tid < 64) {
      float cs = 0.f, rs = 0.f;
      for (int i = 0; i < m; ++i) {
        cs += fabsf(tid < m ? wg[i * m + tid] : 0.f);
        rs += fabsf(tid < m ? wg[tid * m + i] : 0.f);
      }
      s_cs[tid] = tid < m ? cs : -1.f;
      s_rs[tid] = tid < m ? rs : -1.f;
    }
    float pd = 0.f;
    for (int idx = tid; idx < 64 * 64; idx += NSF_THREADS) {
      const int i = idx >> 6, j = idx & 63;
      if (i < m && j < m) pd += gf[i * m + j] * wg[j * m + i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pd += __shfl_xor(pd, off);
    if (ln == 0) s_part[wv] = pd;
    __syncthreads();
    if (tid == 0) {
      int bc = 0, br = 0;
      for (int j = 1; j < m; ++j) {
        if (s_cs[j] > s_cs[bc]) bc = j;
        if (s_rs[j] > s_rs[br]) br = j;
      }
      s_arg[0] = bc;
      s_arg[1] = br;
      float t = 0.f;
      for (int w2 = 0; w2 < NW; ++w2) t += s_part[w2];
      s_da = t;
    }
    __syncthreads();
    jc = s_arg[0];
    ir = s_arg[1];
    inv_c = 1.f / s_cs[jc];
    inv_r = 1.f / s_rs[ir];
    da = s_da;
  }
  const int idx = blockIdx.x * NSF_THREADS + tid;
  if (idx >= m * m) return;
  const int i = idx / m, j = idx - i * m;
  const float* dk = Dk + static_cast<size_t>(g) * K * mm + idx;
  float v = 0.f;
  int k = K - 1;
  for (; k >= 7; k -= 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = dk[static_cast<size_t>(k - u) * mm];
#pragma unroll
    for (int u = 0; u < 8; ++u) v -= t[u];
  }
  for (; k >= 0; --k) v -= dk[static_cast<size_t>(k) * mm];
  v += a * gf[j * m + i];
  if (exact_alpha) {
    const float w = wg[idx];
    const float sg = w > 0.f ? 1.f : (w < 0.f ? -1.f : 0.f);
    v += da * (-a * sg) * ((j == jc ? inv_c : 0.f) + (i == ir ? inv_r : 0.f));
  }
  dWe[g * mm + idx] = v;
}

// ---------------------------------------------------------------------------------------------------------
// Landmark-kernel part of dL: dLW[l][c] = -sum_{l' != l} (Gw[l][l'] + Gw[l'][l]) sign(L[l][c] - L[l'][c]).
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_wpart(const float* __restrict__ L, const float* __restrict__ We,
                                                   const float* __restrict__ dWe, float* __restrict__ dLW,
                                                   float* __restrict__ lam_part, int lam_stride, int m, int D,
                                                   float inv_lam) {
  const int g = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= m * D) return;
  const int l = t / D, c = t % D;
  const size_t mm = static_cast<size_t>(m) * m;
  const float* Lg = L + static_cast<size_t>(g) * m * D;
  const float* wg = We + g * mm;
  const float* dw = dWe + g * mm;
  if (lam_part) {
    // row l of the lambda gradient's W term: -sum over l2 != l of (dW W / lambda) ln(W) (the eps diagonal does
    // not depend on lambda). The row's D threads (D consecutive lanes of one wave) take l2 = c, c + D, ... and
    // add their shares by a butterfly within the group.
    float a = 0.f;
    for (int l2 = c; l2 < m; l2 += D) {
      const float kv = wg[l * m + l2];
      if (l2 != l && kv > 0.f) a -= dw[l * m + l2] * kv * inv_lam * __logf(kv);
    }
    for (int o = D / 2; o > 0; o >>= 1) a += __shfl_xor(a, o);
    if (c == 0) lam_part[static_cast<size_t>(g) * lam_stride + lam_stride - m + l] = a;
  }
  const float ll = Lg[t];
  float acc = 0.f;
  // unrolled, with the diagonal term selected away instead of skipped, so that the loads of several landmarks
  // are in flight together
#pragma unroll 7
  for (int l2 = 0; l2 < m; ++l2) {
    const float gw = (dw[l * m + l2] * wg[l * m + l2] + dw[l2 * m + l] * wg[l2 * m + l]) * inv_lam;
    const float term = gw * sgnf(ll - Lg[l2 * D + c]);
    acc -= (l2 == l) ? 0.f : term;
  }
  dLW[static_cast<size_t>(g) * m * D + t] = acc;
}

// ---------------------------------------------------------------------------------------------------------
// Row gradients of the kernel matrices: dA_hat = dY P^T (side 0) and dC_K = V dS^T (side 1), 64 tokens x m
// landmarks per block, K = d. The products run on the fp16 MFMA in split form (x = hi + lo, A B ~= A_hi B_hi +
// A_hi B_lo + A_lo B_hi, fp32 accumulation): each operand tile is scaled by a power of two that puts its largest
// entry in [2^12, 2^13) and the product is scaled back exactly. The epilogue applies the whitening backward and
// the kernel derivative factor: Gq = dC_Q C_Q / lambda, Gk = dC_K C_K / lambda.
// ---------------------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_rowgrad(const T* __restrict__ dY, const T* __restrict__ V,
                                                     const float* __restrict__ P, const float* __restrict__ dS,
                                                     const float* __restrict__ CQ, const float* __restrict__ CK,
                                                     const float* __restrict__ mu, const float* __restrict__ rstd,
                                                     const float* __restrict__ stats, float* __restrict__ Gq,
                                                     float* __restrict__ Gk, float* __restrict__ lam_part, int N,
                                                     int m, float inv_lam, int whiten) {
  constexpr int KP = D < 32 ? 32 : D;  // K padded to the MFMA's 32
  constexpr int LDH = KP + 8;           // fp16 row stride: 16 bytes mod 128, conflict-free 16-byte reads
  // both operands as [row][k] fp16 halves: A rows are tokens, B rows are landmarks (rows past m are zeros)
  __shared__ __align__(16) _Float16 sAh[64 * LDH];
  __shared__ __align__(16) _Float16 sAl[64 * LDH];
  __shared__ __align__(16) _Float16 sBh[64 * LDH];
  __shared__ __align__(16) _Float16 sBl[64 * LDH];
  __shared__ float sMax[8];
  const int side = blockIdx.z, g = blockIdx.y, i0 = blockIdx.x * 64;
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const T* A = (side == 0 ? dY : V) + static_cast<size_t>(g) * N * D;
  const float* Bm = (side == 0 ? P : dS) + static_cast<size_t>(g) * m * D;
  const float* cm = (side == 0 ? CQ : CK) + static_cast<size_t>(g) * m * N;  // landmark-major [m][N]
  // The lane's 4 values of each landmark tile t are 4 consecutive tokens ib .. ib+3 of landmark t*16 + (ln & 15):
  // one 16-byte load of C and store of G each when they are all in range and N keeps them aligned.
  const int ib = i0 + wv * 16 + 4 * (ln >> 4);
  const bool vec = (N & 3) == 0 && ib + 3 < N;
  // The epilogue's inputs (C and, for whitened C_Q, the landmark's mean, scale and two column statistics) do
  // not depend on the products: loaded here, their round trip overlaps the staging and the MFMAs.
  f32x4 cv[4];
  float wmu[4], wrs[4], wma[4], wmaa[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int l = t * 16 + (ln & 15), lc = l < m ? l : 0;
    const float* crow = cm + static_cast<size_t>(lc) * N;
    if (vec) {
      const float4 c4 = *reinterpret_cast<const float4*>(crow + ib);
      cv[t] = f32x4{c4.x, c4.y, c4.z, c4.w};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) cv[t][r] = crow[ib + r < N ? ib + r : N - 1];
    }
    wmu[t] = 0.f;
    wrs[t] = 1.f;
    wma[t] = 0.f;
    wmaa[t] = 0.f;
    if (side == 0 && whiten) {
      wmu[t] = mu[static_cast<size_t>(g) * m + lc];
      wrs[t] = rstd[static_cast<size_t>(g) * m + lc];
      wma[t] = stats[static_cast<size_t>(g) * 2 * m + lc];
      wmaa[t] = stats[static_cast<size_t>(g) * 2 * m + m + lc];
    }
  }
  int esc;  // ea + eb: the two tiles' scale exponents, undone on the result
  {
    // both tiles' loads (4 channels each) in flight before the first LDS store
    constexpr int Q4 = 64 * D / 4 / 256;
    float4 va[Q4], vb[Q4];
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int idx = tid + q * 256;
      const int r = idx / (D / 4), c4 = 4 * (idx % (D / 4));  // token row of A, landmark row of B
      va[q] = (i0 + r < N) ? load4(A + static_cast<size_t>(i0 + r) * D + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      vb[q] = (r < m) ? load4(Bm + static_cast<size_t>(r) * D + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float ma = 0.f, mb = 0.f;
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      ma = fmaxf(ma, fmaxf(fmaxf(fabsf(va[q].x), fabsf(va[q].y)), fmaxf(fabsf(va[q].z), fabsf(va[q].w))));
      mb = fmaxf(mb, fmaxf(fmaxf(fabsf(vb[q].x), fabsf(vb[q].y)), fmaxf(fabsf(vb[q].z), fabsf(vb[q].w))));
    }
    ma = wave_max_nonneg(ma);
    mb = wave_max_nonneg(mb);
    if (ln == 0) {
      sMax[wv] = ma;
      sMax[4 + wv] = mb;
    }
    if constexpr (D < 32) {  // the K padding of every row is zero
      const int r = tid >> 2, c4 = D + 4 * (tid & 3);
      const half4 z = {0, 0, 0, 0};
      *reinterpret_cast<half4*>(&sAh[r * LDH + c4]) = z;
      *reinterpret_cast<half4*>(&sAl[r * LDH + c4]) = z;
      *reinterpret_cast<half4*>(&sBh[r * LDH + c4]) = z;
      *reinterpret_cast<half4*>(&sBl[r * LDH + c4]) = z;
    }
    __syncthreads();
    ma = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
    mb = fmaxf(fmaxf(sMax[4], sMax[5]), fmaxf(sMax[6], sMax[7]));
    // (clamped so that the scale factors stay finite for tiles of subnormal or zero entries)
    const int ea = max(-100, min(100, store_exp(ma))), eb = max(-100, min(100, store_exp(mb)));
    const float sa = ldexpf(1.f, -ea), sb = ldexpf(1.f, -eb);
    esc = ea + eb;
#pragma unroll
    for (int q = 0; q < Q4; ++q) {
      const int idx = tid + q * 256;
      const int r = idx / (D / 4), c4 = 4 * (idx % (D / 4));
      half4 h, l;
      split_scaled4(f32x4{va[q].x, va[q].y, va[q].z, va[q].w}, sa, h, l);
      *reinterpret_cast<half4*>(&sAh[r * LDH + c4]) = h;
      *reinterpret_cast<half4*>(&sAl[r * LDH + c4]) = l;
      split_scaled4(f32x4{vb[q].x, vb[q].y, vb[q].z, vb[q].w}, sb, h, l);
      *reinterpret_cast<half4*>(&sBh[r * LDH + c4]) = h;
      *reinterpret_cast<half4*>(&sBl[r * LDH + c4]) = l;
    }
  }
  __syncthreads();
  // all 4 landmark tiles (B rows past m are zeros), K in chunks of 32: the lane supplies row (ln & 15) of its
  // wave's 16 tokens and of the tile's 16 landmarks at k = 8 (ln >> 4) .. +7 of the chunk
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < KP / 32; ++c) {
    const int oa = (wv * 16 + (ln & 15)) * LDH + c * 32 + 8 * (ln >> 4);
    const half8 ah = *reinterpret_cast<const half8*>(&sAh[oa]);
    const half8 al = *reinterpret_cast<const half8*>(&sAl[oa]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ob = (t * 16 + (ln & 15)) * LDH + c * 32 + 8 * (ln >> 4);
      const half8 bh = *reinterpret_cast<const half8*>(&sBh[ob]);
      const half8 bl = *reinterpret_cast<const half8*>(&sBl[ob]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = ldexpf(acc[t][r], esc);
  // Gq / Gk are written landmark-major too, [m][N]: the dL reduction then reads a landmark's weights for
  // consecutive tokens as one contiguous run, and the token-row kernel reads them coalesced across its lanes.
  float* out = (side == 0 ? Gq : Gk) + static_cast<size_t>(g) * m * N;
  float lam = 0.f;  // this lane's share of -sum G ln(C) (the lambda gradient)
  auto lam_term = [](float gv, float c) { return c > 0.f ? -gv * __logf(c) : 0.f; };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int l = t * 16 + (ln & 15);
    if (l >= m) continue;
    const float mu_l = wmu[t], rs_l = wrs[t], mA = wma[t], mAA = wmaa[t];
    auto grad = [&](float v, float c) {
      if (side == 0 && whiten) {
        const float ahat = (c - mu_l) * rs_l;
        v = rs_l * (v - mA - ahat * mAA);
      }
      return v * c * inv_lam;
    };
    if (vec) {
      const f32x4 c4 = cv[t];
      const float4 o = make_float4(grad(acc[t][0], c4[0]), grad(acc[t][1], c4[1]), grad(acc[t][2], c4[2]),
                                   grad(acc[t][3], c4[3]));
      *reinterpret_cast<float4*>(out + static_cast<size_t>(l) * N + ib) = o;
      lam += lam_term(o.x, c4[0]) + lam_term(o.y, c4[1]) + lam_term(o.z, c4[2]) + lam_term(o.w, c4[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib + r;
        if (i < N) {
          const float c = cv[t][r], o = grad(acc[t][r], c);
          out[static_cast<size_t>(l) * N + i] = o;
          lam += lam_term(o, c);
        }
      }
    }
  }
  if (lam_part) {
    // the block's sum in a fixed order: butterfly within each wave, then the 4 waves in order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lam += __shfl_xor(lam, o);
    __shared__ float wsum[4];
    if (ln == 0) wsum[wv] = lam;
    __syncthreads();
    if (tid == 0)
      lam_part[static_cast<size_t>(g) * (2 * gridDim.x + m) + side * gridDim.x + blockIdx.x] =
          ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

// ---------------------------------------------------------------------------------------------------------
// The two sign reductions of the kernel gradient in one pass ([note] motivation "core idea": d/dx exp(-|x - l|_1 /
// lambda) = -(1/lambda) sign(x - l) k, with G = dC C / lambda already formed): for a token row x of Q (side 0) or K
// (side 1), landmark l and channel c, s = sign(x_c - L_lc) is evaluated once and feeds
//   dX_c  -= G[l][x] s   (summed over the landmarks: dQ before its pooling term, dK), and
//   dL_lc += G[l][x] s   (summed over the token rows of both sides).
// Block = kSignSub x RT token rows of one slice; thread = (channel c, sub-tile of RT rows). A thread runs over all
// MP landmarks (m itself, or m rounded up to 8 with zero weights) with its RT row values and dX sums in VGPRs, so
// dX leaves complete and in one piece (dK final, dQ as an fp32 partial: its pooling term comes with dL), and dL
// for every landmark accumulates in VGPRs across both sides. Per (row, landmark): s = med3(x 2^100 - l 2^100,
// -1, 1), then one fma into dL and one into dX, all register operands: the block stages Gq and Gk for its rows
// (landmark-major, as stored) and -2^100 L in LDS and reads each landmark's RT weights as 16-byte broadcasts. At
// the end the sub-tiles' dL are added through LDS in sub-tile order, 8 landmarks at a time, and the block writes
// one [m][D] partial, summed in fixed order by k_bwd_dq_final.
// ---------------------------------------------------------------------------------------------------------
template <int RT>
__device__ __forceinline__ void load_w(const float* p, float (&w)[RT]) {
#pragma unroll
  for (int q = 0; q < RT / 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(p + 4 * q);
    w[4 * q] = v.x;
    w[4 * q + 1] = v.y;
    w[4 * q + 2] = v.z;
    w[4 * q + 3] = v.w;
  }
}

// RT consecutive rows of one channel (p points at the first, rows D apart); rows past `rlast` read row `rlast`
// (the last row of the slice, finite; their weights are zero).
template <typename T, int RT, int D>
__device__ __forceinline__ void load_rows(const T* p, int rlast, float (&x)[RT]) {
  if (rlast >= RT - 1) {
#pragma unroll
    for (int r = 0; r < RT; ++r) x[r] = to_f32(p[r * D]);
  } else {
#pragma unroll
    for (int r = 0; r < RT; ++r) x[r] = to_f32(p[min(r, rlast) * D]);
  }
}

template <typename T, int D, int MP>
__global__ __launch_bounds__(kSignSub * 64) void k_bwd_sign(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const float* __restrict__ L, const float* __restrict__ Gq,
                                                           const float* __restrict__ Gk, float* __restrict__ dQp,
                                                           T* __restrict__ dK, float* __restrict__ dLpart, int N,
                                                           int m, int nsplit) {
  constexpr int RT = kSignRt, RB = kSignSub * RT, NTH = kSignSub * D;
  constexpr int kGs = 2 * MP * RB, kRed = kSignSub * 8 * D, kLs = MP * D;
  constexpr int kFirst = kGs > kRed ? kGs : kRed;
  __shared__ __align__(16) float smem[kFirst + kLs];
  float* Gs = smem;          // [2][MP][RB] weights, zero past m and past N; later [kSignSub][8][D] for dL
  float* Ls = smem + kFirst;  // [MP][D] landmark values times -2^100
  const int g = static_cast<int>(blockIdx.x) / nsplit, sp = static_cast<int>(blockIdx.x) % nsplit;
  const int r0 = sp * RB;
  const int tid = threadIdx.x, c = tid % D;
  int sub = tid / D;
  if constexpr (D == 64) sub = __builtin_amdgcn_readfirstlane(sub);  // one sub-tile per wave

  // Staging: every load is issued before the first LDS store (a fixed count per thread; NTH is a multiple of RB,
  // so a thread's row within the block is the same for all its weights). Rows past N and landmarks past m read
  // in-bounds entries and store zero.
  constexpr int KS = (kGs + NTH - 1) / NTH, KL = (kLs + NTH - 1) / NTH;
  const int rb = sub * RT;
  const int rlast = N - 1 - (r0 + rb);  // the sub-tile's rows past this one are past N
  const size_t base = (static_cast<size_t>(g) * N + r0 + rb) * D + c;
  float xn[RT];  // the next side's raw row values
  load_rows<T, RT, D>(Q + base, rlast, xn);
  {
    constexpr int KB = 16;  // loads in flight per thread
    const int rr = tid % RB, rowc = min(r0 + rr, N - 1);
    const bool rowok = r0 + rr < N;
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += KB) {
      float gv[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (k0 + k < KS) {
          const int sl = min((tid + (k0 + k) * NTH) / RB, 2 * MP - 1), side = sl / MP;
          const int lc = min(sl - side * MP, m - 1);
          gv[k] = (side ? Gk : Gq)[(static_cast<size_t>(g) * m + lc) * N + rowc];
        }
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = tid + (k0 + k) * NTH, l = (e / RB) % MP;
        if (k0 + k < KS && e < kGs) Gs[e] = rowok && l < m ? gv[k] : 0.f;
      }
    }
#pragma unroll
    for (int k0 = 0; k0 < KL; k0 += KB) {
      float lvv[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (k0 + k < KL) {
          const int lc = min((tid + (k0 + k) * NTH) / D, m - 1);
          lvv[k] = L[(static_cast<size_t>(g) * m + lc) * D + c];
        }
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = tid + (k0 + k) * NTH;
        if (k0 + k < KL && e < kLs) Ls[e] = e / D < m ? lvv[k] * -kSgnScale : 0.f;
      }
    }
  }
  __syncthreads();

  float dl[MP];
#pragma unroll
  for (int l = 0; l < MP; ++l) dl[l] = 0.f;
#pragma unroll 1
  for (int side = 0; side < 2; ++side) {
    float x[RT], xs[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      x[r] = xn[r] * kSgnScale;
      asm volatile("" : "+v"(x[r]));  // keeps x 2^100 in a VGPR: no literal-operand fma per term
      xs[r] = 0.f;
    }
    if (side == 0) load_rows<T, RT, D>(K + base, rlast, xn);  // in flight during side 0
    // Landmark l + 1's weights and value are read while landmark l is processed. After each landmark its sums are
    // pinned (an empty asm that takes and returns them) and a scheduling barrier follows, so the compiler neither
    // hoists every landmark's reads up front nor defers the dL chains (either would hold MP x RT values in VGPRs).
    const float* gw = Gs + side * MP * RB + rb;
    float w[RT], wn[RT], lv, lvn;
    load_w<RT>(gw, wn);
    lvn = Ls[c];
#pragma unroll
    for (int l = 0; l < MP; ++l) {
#pragma unroll
      for (int r = 0; r < RT; ++r) w[r] = wn[r];
      lv = lvn;
      if (l + 1 < MP) {
        load_w<RT>(gw + (l + 1) * RB, wn);
        lvn = Ls[(l + 1) * D + c];
      }
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float sg = __builtin_amdgcn_fmed3f(x[r] + lv, -1.f, 1.f);
        dl[l] = fmaf(w[r], sg, dl[l]);
        xs[r] = fmaf(w[r], sg, xs[r]);  // dX = -xs: both sums are then plain multiply-adds
      }
      asm volatile("" : "+v"(dl[l]));
#pragma unroll
      for (int r = 0; r < RT; ++r) asm volatile("" : "+v"(xs[r]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (side == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
        if (r <= rlast) dQp[base + r * D] = -xs[r];
    } else {
#pragma unroll
      for (int r = 0; r < RT; ++r)
        if (r <= rlast) dK[base + r * D] = from_f32<T>(-xs[r]);
    }
  }

  __syncthreads();  // the weights are no longer read: their space takes the dL sums
  float* red = smem;
#pragma unroll
  for (int k = 0; k < (MP + 7) / 8; ++k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[(sub * 8 + j) * D + c] = 8 * k + j < MP ? dl[8 * k + j] : 0.f;
    __syncthreads();
    for (int j = sub; j < 8; j += kSignSub) {  // output (landmark 8k + j, channel c)
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < kSignSub; ++q) v += red[(q * 8 + j) * D + c];
      if (8 * k + j < m) dLpart[((static_cast<size_t>(g) * nsplit + sp) * m + 8 * k + j) * D + c] = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------------------
// lambda gradient: every kernel entry k = exp(-D / lambda) moves by k D / lambda^2 = -k ln(k) / lambda, so
// d/dlambda = -sum G ln(k) over G = dC C / lambda (Gq, Gk, and Gw = dW W / lambda off the diagonal, where W = W_eps
// and the eps diagonal does not depend on lambda). The row-gradient kernel sums the Gq and Gk terms of each of
// its blocks (it forms those G values), k_bwd_wpart the Gw terms of each landmark row; an entry whose k
// underflowed to 0 has G = 0 and adds nothing. One extra block of k_bwd_dq_final adds the partials in a fixed
// order (after the call's stream has joined the side stream, which writes the W terms).
// ---------------------------------------------------------------------------------------------------------
// One block of 256 threads: thread t sums the partials t, t + 256, ... in order, then a fixed tree in LDS (red:
// 256 floats).
__device__ __forceinline__ void dlam_sum_block(const float* __restrict__ part, float* __restrict__ out, int n,
                                               float* red) {
  const int tid = threadIdx.x;
  float t = 0.f;
  for (int i = tid; i < n; i += 256) t += part[i];
  red[tid] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) *out = red[0];
}

// dL = sum of the sign blocks' partials (in block order) + the landmark-kernel term dLW, then the pooling term of
// dQ: every token i of landmark l's r x r block gets dQ_i = dQp_i + dL_l / r^2. Block = (landmark, slice); each
// thread takes up to kDqPer of the block's r^2 D token entries, whose dQp loads are issued before the dL sum.
// With dlam, block (m, 0) instead sums the nlam lambda-gradient partials into *dlam (blocks (m, g > 0) exit).
constexpr int kDqPer = 16;

template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_dq_final(const float* __restrict__ dLpart, const float* __restrict__ dLW,
                                                      const float* __restrict__ dQp, T* __restrict__ dQ, int N, int m,
                                                      int W, int r, int nsplit, const float* __restrict__ lampart,
                                                      float* __restrict__ dlam, int nlam) {
  constexpr int P = 256 / D;
  __shared__ float part[256];
  __shared__ float add[D];
  const int l = blockIdx.x, g = blockIdx.y, tid = threadIdx.x, c = tid % D, q = tid / D;
  if (l >= m) {
    if (g == 0 && dlam) dlam_sum_block(lampart, dlam, nlam, part);
    return;
  }
  const int wr = W / r, yb = l / wr, xb = l % wr, total = r * r * D;
  // entry e = e0 + tid + 256 u (u < kDqPer): token e / D of the block, channel e % D = c
  size_t o[kDqPer];
  float t[kDqPer];
  auto load_chunk = [&](int e0) {
#pragma unroll
    for (int u = 0; u < kDqPer; ++u) {
      const int tk = min(e0 + tid + u * 256, total - 1) / D;
      o[u] = (static_cast<size_t>(g) * N + static_cast<size_t>(yb * r + tk / r) * W + xb * r + tk % r) * D + c;
      t[u] = dQp[o[u]];
    }
  };
  load_chunk(0);
  // the landmark-kernel term of dL, loaded with everything else before the first sum
  const float dlw = tid < D ? dLW[(static_cast<size_t>(g) * m + l) * D + tid] : 0.f;
  float v = 0.f;  // partials q, q + P, q + 2P, ... in that order, loaded 16 at a time
  for (int s0 = q; s0 < nsplit; s0 += 16 * P) {
    float pv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sidx = min(s0 + u * P, nsplit - 1);
      pv[u] = dLpart[((static_cast<size_t>(g) * nsplit + sidx) * m + l) * D + c];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (s0 + u * P < nsplit) v += pv[u];
  }
  part[tid] = v;
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < P; ++u) a += part[u * D + tid];
    add[tid] = (a + dlw) * (1.f / static_cast<float>(r * r));
  }
  __syncthreads();
  const float ad = add[c];
  for (int e0 = 0;;) {
#pragma unroll
    for (int u = 0; u < kDqPer; ++u)
      if (e0 + tid + u * 256 < total) dQ[o[u]] = from_f32<T>(t[u] + ad);
    e0 += kDqPer * 256;
    if (e0 >= total) break;
    load_chunk(e0);  // r^2 D above kDqPer x 256
  }
}

// ---------------------------------------------------------------------------------------------------------
// DWC weight gradient: dw[h d + c][a][b] = sum over the batch and the grid of dY[(y, x), c] V[(y+a-1, x+b-1), c]
// (zero outside the grid). Work item = one run of kDwcRun tokens along a grid row; thread = (4-channel group,
// item): it keeps the 3 x 3 window of V in registers and slides it along the run, so each token costs one 16-byte
// load of dY and three of V, and accumulates the 9 taps of its 4 channels. A block's items are summed in LDS in
// item order into a [9][d] partial per (slice, block); the final pass gives each (head, tap, 16 channels) a block
// whose threads sum strided runs of the (batch, block) partials in order and then combine them in a fixed order.
// ---------------------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kDwcThreads) void k_dwc_wgrad_partial(const T* __restrict__ dY, const T* __restrict__ V,
                                                                   float* __restrict__ part, int H, int W, int nseg,
                                                                   int nblk) {
  constexpr int CQ = D / 4;                // channel groups of 4
  constexpr int SLOTS = kDwcThreads / CQ;  // items per block
  const int g = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const int cq = tid % CQ, slot = tid / CQ;
  const int item = blk * SLOTS + slot;
  const size_t N = static_cast<size_t>(H) * W;
  const T* dy = dY + static_cast<size_t>(g) * N * D + 4 * cq;
  const T* v = V + static_cast<size_t>(g) * N * D + 4 * cq;
  float4 acc[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (item < H * nseg) {
    const int y = item / nseg, x0 = (item - y * nseg) * kDwcRun;
    auto ldv = [&](int yy, int xx) {
      return (yy >= 0 && yy < H && xx >= 0 && xx < W) ? load4(v + static_cast<size_t>(yy * W + xx) * D)
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    float4 win[3][3];  // win[a][b] = V(y + a - 1, x + b - 1) for the current x
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      win[a][0] = ldv(y + a - 1, x0 - 1);
      win[a][1] = ldv(y + a - 1, x0);
    }
#pragma unroll
    for (int t = 0; t < kDwcRun; ++t) {
      const int x = x0 + t;
#pragma unroll
      for (int a = 0; a < 3; ++a) win[a][2] = ldv(y + a - 1, x + 1);
      const float4 gy = x < W ? load4(dy + static_cast<size_t>(y * W + x) * D) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          float4& r = acc[a * 3 + b];
          r.x += gy.x * win[a][b].x;
          r.y += gy.y * win[a][b].y;
          r.z += gy.z * win[a][b].z;
          r.w += gy.w * win[a][b].w;
        }
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        win[a][0] = win[a][1];
        win[a][1] = win[a][2];
      }
    }
  }
  __shared__ float4 red[SLOTS][9][CQ];
#pragma unroll
  for (int q = 0; q < 9; ++q) red[slot][q][cq] = acc[q];
  __syncthreads();
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0]);
  for (int e = tid; e < 9 * D; e += kDwcThreads) {  // e = q * D + c
    float t = 0.f;
    for (int s2 = 0; s2 < SLOTS; ++s2) t += rf[s2 * 9 * D + e];
    part[(static_cast<size_t>(g) * nblk + blk) * 9 * D + e] = t;
  }
}

// Block (head h, tap q; channels 16 blockIdx.y ..): thread (channel, phase) sums the partials j = phase, phase + 16,
// ... of the B * nblk (batch, block) partials of head h, then phase 0 adds the 16 phase sums in order.
template <int D>
__global__ __launch_bounds__(256) void k_dwc_wgrad_final(const float* __restrict__ part, float* __restrict__ out,
                                                         int B, int heads, int nblk) {
  const int h = blockIdx.x / 9, q = blockIdx.x % 9, tid = threadIdx.x;
  const int c = blockIdx.y * 16 + (tid & 15), ph = tid >> 4;
  const int n = B * nblk;
  float s = 0.f;
#pragma unroll 4
  for (int j = ph; j < n; j += 16) {
    const int b = j / nblk, k = j - b * nblk;
    s += part[((static_cast<size_t>(b) * heads + h) * nblk + k) * 9 * D + q * D + c];
  }
  __shared__ float red[256];
  red[tid] = s;
  __syncthreads();
  if (ph == 0) {
    float t = 0.f;
    for (int p2 = 0; p2 < 16; ++p2) t += red[p2 * 16 + (tid & 15)];
    out[(static_cast<size_t>(h) * D + c) * 9 + q] = t;
  }
}

// ---------------------------------------------------------------------------------------------------------
size_t bwd_ws_bytes(const Shape& s) {
  if (s.m > 64 || s.d > 64) return 0;
  return plan(s).total;
}

// The reverse Newton-Schulz group (k_bwd_ns_*, then k_bwd_wpart) depends only on dX and produces dW_eps and dL's
// landmark-kernel term; the row gradients, the dV adjoint, the dL partials and the DWC weight gradient depend
// only on dS and the whitening statistics. The group runs on one block per slice for most of its time, so when the
// caller lends a second stream (side) it goes there and overlaps those kernels. After the join the lambda gradient,
// which needs only Gq, Gk and dW_eps, forks to that stream once more, next to the dL finalisation and the token
// rows. Without it every launch stays on st in the same order.
template <typename T, int D>
static hipError_t bwd_t(const Shape& s, bool whiten, const void* Qv, const void* Kv, const void* Vv, const float* w,
                        const SavedPtrs& sp, const void* dYv, void* dQv, void* dKv, void* dVv, void* ws,
                        hipStream_t st, const BwdExtras& ex, const AuxStream* side) {
  const BwdWs p = plan(s);
  char* b = static_cast<char*>(ws);
  float* T1 = reinterpret_cast<float*>(b + p.T1);
  float* part = reinterpret_cast<float*>(b + p.part);
  float* dX = reinterpret_cast<float*>(b + p.dX);
  float* dS = reinterpret_cast<float*>(b + p.dS);
  float* stats = reinterpret_cast<float*>(b + p.stats);
  float* dWe = reinterpret_cast<float*>(b + p.dWe);
  float* dLW = reinterpret_cast<float*>(b + p.dLW);
  float* Gq = reinterpret_cast<float*>(b + p.Gq);
  float* Gk = reinterpret_cast<float*>(b + p.Gk);
  float* dLpart = reinterpret_cast<float*>(b + p.dLpart);
  float* dQp = reinterpret_cast<float*>(b + p.dQp);
  const T* Q = static_cast<const T*>(Qv);
  const T* K = static_cast<const T*>(Kv);
  const T* V = static_cast<const T*>(Vv);
  const T* dY = static_cast<const T*>(dYv);
  T* dQ = static_cast<T*>(dQv);
  T* dK = static_cast<T*>(dKv);
  const float inv_lam = static_cast<float>(1.0 / static_cast<double>(s.lambda));
  const int wh = whiten ? 1 : 0;

  // With a side stream: two forks and one join (an event wait costs the host about as much as four launches).
  // The side stream starts at once with the work that needs nothing from this call's other kernels (the split
  // fragments of A1_k = W X_k and A2_k = X_k W, and the DWC weight gradient), beside T1 and the small products on
  // the call's stream. After the small products it takes the reverse Newton-Schulz chain, D_k, dW and dL's
  // landmark-kernel term, while the call's stream forms the row gradients, dV and the sign reductions; the call's
  // stream then waits for it before the last two kernels. The side stream's kernels are enqueued ahead of the
  // call's stream's long ones, so that the chain's few blocks reach the GPU before those fill it. (One fork after
  // the small products, with the side stream's work enqueued after the call's stream's, left the chain waiting
  // for the sign reductions to drain: the two streams' work ran one after the other.)
  hipError_t e = hipSuccess;
  hipStream_t ns_st = side ? side->s : st;
  bool forked = false;
  // on an error after the fork the call's stream still ends after everything enqueued on the side stream
  auto bail = [&](hipError_t err) -> hipError_t {
    if (forked && hipEventRecord(side->join, side->s) == hipSuccess) (void)hipStreamWaitEvent(st, side->join, 0);
    return err;
  };
  auto fork = [&]() -> hipError_t {  // the side stream waits for everything enqueued on the call's stream so far
    if (!side) return hipSuccess;
    hipError_t f = hipEventRecord(side->fork, st);
    if (f == hipSuccess) f = hipStreamWaitEvent(side->s, side->fork, 0);
    if (f == hipSuccess) forked = true;
    return f;
  };
  float* lp = ex.d_lambda ? reinterpret_cast<float*>(b + p.lampart) : nullptr;
  bh8* frag = reinterpret_cast<bh8*>(b + p.nsA1);
  float* nsc = reinterpret_cast<float*>(b + p.nsA2);
  const int Kn = s.ns_iters;
  const int sliceblocks = 8 * cdiv(s.G, 8) * Kn;  // slice_step_of's grid
  if ((e = fork()) != hipSuccess) return bail(e);
  if (Kn > 0)
    hipLaunchKernelGGL(k_bwd_ns_pre, dim3(sliceblocks), dim3(NSB_THREADS), 0, ns_st, sp.We, sp.xs, frag, nsc, s.m,
                       Kn, s.G);
  if (ex.d_dwc_w) {
    float* dp = reinterpret_cast<float*>(b + p.dwcpart);
    hipLaunchKernelGGL((k_dwc_wgrad_partial<T, D>), dim3(p.dwcblocks, s.G), dim3(kDwcThreads), 0, ns_st, dY, V, dp,
                       s.H, s.W, p.dwcseg, p.dwcblocks);
    hipLaunchKernelGGL(k_dwc_wgrad_final<D>, dim3(s.heads * 9, D / 16), dim3(256), 0, ns_st, dp, ex.d_dwc_w,
                       s.G / s.heads, s.heads, p.dwcblocks);
  }
  if ((e = launch_ckv_general(s, sp.CQ, 1, dY, part, T1, st)) != hipSuccess) return bail(e);
  hipLaunchKernelGGL(k_bwd_small1<D>, dim3(s.G, s.m < 32 ? s.m : 32), dim3(256), 0, st, T1, sp.S, sp.P, sp.xs, sp.mu,
                     sp.rstd, dX, dS, stats, s.m, s.ns_iters, s.N, wh);
  if ((e = fork()) != hipSuccess) return bail(e);
  {
    float* Gs = reinterpret_cast<float*>(b + p.nsG);
    float* Dk = reinterpret_cast<float*>(b + p.nsD);
    float* Gf = reinterpret_cast<float*>(b + p.nsGf);
    hipLaunchKernelGGL(k_bwd_ns_chain, dim3(s.G), dim3(NSC_THREADS), 0, ns_st, frag, nsc, dX, Gs, Gf, s.m, Kn);
    if (Kn > 0)
      hipLaunchKernelGGL(k_bwd_ns_dk, dim3(sliceblocks), dim3(NSB_THREADS), 0, ns_st, sp.xs, Gs, Dk, s.m, Kn, s.G);
    hipLaunchKernelGGL(k_bwd_ns_final, dim3(cdiv(static_cast<long>(s.m) * s.m, NSF_THREADS), s.G),
                       dim3(NSF_THREADS), 0, ns_st, sp.We, sp.alpha, Dk, Gf, dWe, s.m, Kn, ex.exact_alpha ? 1 : 0);
  }
  hipLaunchKernelGGL(k_bwd_wpart, dim3(cdiv(static_cast<long>(s.m) * D, 256), s.G), dim3(256), 0, ns_st, sp.L, sp.We,
                     dWe, dLW, lp, p.lamchunks, s.m, D, inv_lam);
  hipLaunchKernelGGL((k_bwd_rowgrad<T, D>), dim3(cdiv(s.N, 64), s.G, 2), dim3(256), 0, st, dY, V, sp.P, dS, sp.CQ,
                     sp.CK, sp.mu, sp.rstd, stats, Gq, Gk, lp, s.N, s.m, inv_lam, wh);
  if ((e = launch_out_adjoint(s, sp.CK, dS, dY, w, dVv, st)) != hipSuccess) return bail(e);
  {
    const dim3 grid(s.G * p.nsplitS), block(kSignSub * D);
#define LF_SIGN(MP_)                                                                                                \
  case MP_:                                                                                                         \
    hipLaunchKernelGGL((k_bwd_sign<T, D, MP_>), grid, block, 0, st, Q, K, sp.L, Gq, Gk, dQp, dK, dLpart, s.N, s.m,  \
                       p.nsplitS);                                                                                  \
    break
    // the landmark counts of square grids run unpadded; others are padded to a multiple of 8 with zero weights
    const bool square = s.m == 4 || s.m == 9 || s.m == 25 || s.m == 36 || s.m == 49;
    switch (square ? s.m : cdiv(s.m, 8) * 8) {
      LF_SIGN(4);
      LF_SIGN(9);
      LF_SIGN(25);
      LF_SIGN(36);
      LF_SIGN(49);
      LF_SIGN(8);
      LF_SIGN(16);
      LF_SIGN(24);
      LF_SIGN(32);
      LF_SIGN(40);
      LF_SIGN(48);
      LF_SIGN(56);
      LF_SIGN(64);
      default: return bail(hipErrorInvalidValue);  // the backward takes m <= 64 (checked at the boundary)
    }
#undef LF_SIGN
  }
  if (side && (e = hipEventRecord(side->join, side->s)) != hipSuccess) return bail(e);
  if (side && (e = hipStreamWaitEvent(st, side->join, 0)) != hipSuccess) return bail(e);  // dLW, Gw's lambda terms
  hipLaunchKernelGGL((k_bwd_dq_final<T, D>), dim3(s.m + (ex.d_lambda ? 1 : 0), s.G), dim3(256), 0, st, dLpart, dLW,
                     dQp, dQ, s.N, s.m, s.W, s.r, p.nsplitS, lp, ex.d_lambda, s.G * p.lamchunks);
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_d(const Shape& s, bool whiten, const void* Q, const void* K, const void* V, const float* w,
                        const SavedPtrs& sp, const void* dY, void* dQ, void* dK, void* dV, void* ws, hipStream_t st,
                        const BwdExtras& ex, const AuxStream* aux) {
  switch (s.d) {
    case 16: return bwd_t<T, 16>(s, whiten, Q, K, V, w, sp, dY, dQ, dK, dV, ws, st, ex, aux);
    case 32: return bwd_t<T, 32>(s, whiten, Q, K, V, w, sp, dY, dQ, dK, dV, ws, st, ex, aux);
    default: return bwd_t<T, 64>(s, whiten, Q, K, V, w, sp, dY, dQ, dK, dV, ws, st, ex, aux);
  }
}

hipError_t launch_backward(const Shape& s, bool whiten, const void* Q, const void* K, const void* V, const float* w,
                           const SavedPtrs& sp, const void* dY, void* dQ, void* dK, void* dV, void* ws,
                           hipStream_t st, const BwdExtras& ex, const AuxStream* aux) {
  if (s.dtype == 1) return bwd_d<bf16_t>(s, whiten, Q, K, V, w, sp, dY, dQ, dK, dV, ws, st, ex, aux);
  return bwd_d<float>(s, whiten, Q, K, V, w, sp, dY, dQ, dK, dV, ws, st, ex, aux);
}

}  // namespace lf
