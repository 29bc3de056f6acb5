// Newton-Schulz pseudo-inverse of the landmark kernel on MFMA (gfx950).
//
// [note] = papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力", Design 3:
// W is shifted by eps I, X_0 = alpha W^T and X_{k+1} = X_k (2I - W X_k): only matrix products and additions,
// no inverse or SVD. alpha = 1/(||W||_1 ||W||_inf) (max column abs sum times max row abs sum) is the reading that
// keeps every eigenvalue of alpha W W^T in (0, 1]; the page's 2/||W||_2 would diverge for a unit-diagonal W.
#include <cmath>
#include <type_traits>

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
//
// Matrices are zero-padded to 16 ST x 16 ST (ST = 1, 2 or 4 strips of 16) and kept K-contiguous in LDS, so each
// lane's 8-element fragment is one 16-byte read: U = 2I - W X by columns (B operand of X U) and X twice, by rows
// (A operand of X U) and by columns (B operand of W X). W, the A operand of W X, never changes: each wave keeps
// its fragments in registers. (X_k is symmetric in exact arithmetic, but feeding its transpose to the update
// doubles the antisymmetric part of the rounding error every step, so both layouts are kept.)
//
// Work split: wave w owns the (w & 1, w >> 1) quadrant of every product (TQ x TQ tiles of 16 x 16), which reads
// half of each operand instead of one full operand per wave. X is double-buffered, so an iteration needs two
// barriers: after U is written and after X_next is written. The MFMA result layout (four consecutive rows of
// one column per lane) gives the by-columns copy of X_next with 8-byte stores; the by-rows copy comes from a
// second product with the operand roles swapped, (X U)^T = U^T X^T, which reuses the same fragments and yields
// four consecutive columns of one row per lane. The two copies differ only by rounding.
//
// X carries a power-of-two scale 2^-e in its fp16 halves: e follows the largest entry of the previous iterate
// so that entries sit near 2^12 (far from fp16's subnormals and its 65504 limit); an iterate that still comes
// out above 2^15 is stored again with a fresh exponent. W needs no scale (entries at most 1 + eps) and neither
// does U (the eigenvalues of W X stay in (0, 1]).
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

// Operand fragments of TQ consecutive 16-row (or 16-column) strips over KC chunks of 32 along K.
template <int TQ, int KC>
struct Frags {
  half8 h[TQ][KC], l[TQ][KC];
};

// Chunk c (K entries 32 c .. 32 c + 31) of the fragments of strips s0 .. s0+TQ-1 of a K-contiguous split
// matrix (row i holds its K entries at i*NH ...).
template <int TQ, int KC>
__device__ __forceinline__ void load_chunk(const SplitMat& M, int s0, int ln, int c, Frags<TQ, KC>& f) {
#pragma unroll
  for (int a = 0; a < TQ; ++a) {
    const int i = (s0 + a) * 16 + (ln & 15);
    const int k0 = c * 32 + 8 * (ln >> 4);
    f.h[a][c] = *reinterpret_cast<const half8*>(&M.hi[i * NH + k0]);
    f.l[a][c] = *reinterpret_cast<const half8*>(&M.lo[i * NH + k0]);
  }
}

template <int TQ>
__device__ __forceinline__ void zero_acc(f32x4 acc[TQ][TQ]) {
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc[a][b] += A-strip a times B-strip b over chunk c. One fp32 accumulator per tile takes hi*hi and both cross
// terms: each MFMA step rounds at fp32 relative to the running sum, which keeps the product at fp32 accuracy.
// Loads are issued chunk by chunk and consumed in the same order, so the MFMAs of chunk 0 can overlap the LDS
// reads of chunk 1.
template <int TQ, int KC>
__device__ __forceinline__ void mma_chunk(const Frags<TQ, KC>& A, const Frags<TQ, KC>& B, f32x4 acc[TQ][TQ],
                                          int c) {
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[a][c], B.h[b][c], acc[a][b], 0, 0, 0);
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[a][c], B.l[b][c], acc[a][b], 0, 0, 0);
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.l[a][c], B.h[b][c], acc[a][b], 0, 0, 0);
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

// The 4 rows i0 .. i0+3 of column j, stored transposed: Mt[j][i0 .. i0+3] (two 8-byte writes).
__device__ __forceinline__ void put_t4(SplitMat& Mt, int j, int i0, half4 h, half4 l) {
  *reinterpret_cast<half4*>(&Mt.hi[j * NH + i0]) = h;
  *reinterpret_cast<half4*>(&Mt.lo[j * NH + i0]) = l;
}

// The same 4 entries stored row-major: M[i0 + r][j].
__device__ __forceinline__ void put_rows4(SplitMat& M, int i0, int j, half4 h, half4 l) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    M.hi[(i0 + r) * NH + j] = h[r];
    M.lo[(i0 + r) * NH + j] = l[r];
  }
}

// Largest exponent e of an fp32 value (v = f * 2^e, f in [1, 2)) for v > 0; -126 for 0 and subnormals.
__device__ __forceinline__ int exp_of(float v) {
  const int b = static_cast<int>((__float_as_uint(v) >> 23) & 0xffu);
  return (b == 0 ? 1 : b) - 127;
}

// Storage exponent for an iterate whose largest entry is about mx: entries land in [2^12, 2^13).
__device__ __forceinline__ int store_exp(float mx) { return mx > 0.f ? exp_of(mx) - 12 : 0; }
constexpr int kRestoreExp = 15;  // an entry at or above 2^15 * 2^e triggers a re-store with a fresh exponent
// Longest run of coupled T/X steps before T is formed again as W X: 2^kPairRun times the relative rounding of
// one product must stay well below 1 (split-fp16 products: 2^-22; the fp32 products of the m > 64 path: 2^-24).
constexpr int kPairRun = 11;
constexpr int kPairRunF32 = 12;

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

template <int ST, int KC>
__device__ __forceinline__ void ns_small_block(int g, const float* __restrict__ We, float* __restrict__ Xout,
                                               float* __restrict__ xs, float* __restrict__ alpha_out,
                                               float* __restrict__ resid, int m, int iters) {
  constexpr int TQ = ST >= 2 ? ST / 2 : 1;  // tiles per side of a wave's quadrant
  constexpr int NQA = ST == 1 ? 1 : 4;      // quadrants with work
  constexpr int NTH = 512;
  // sX: X by rows. sT: T = W X by rows (and X by columns where the final exact step needs it). sU: U = 2I - T by
  // columns. Each is double-buffered by iteration parity.
  __shared__ SplitMat sX[2], sT[2], sU[2];
  __shared__ double red[3][4][64];
  __shared__ float s_alpha, s_wmax;
  // Bits of the largest |X| entry of the iterate written in step k, in slot k % 3: slot k + 1 is cleared during
  // step k (its last readers finished before the barrier of step k - 1), so the one barrier per step suffices.
  __shared__ unsigned int s_max[3];
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  float* wf = reinterpret_cast<float*>(&sU[1]);  // fp32 W (64 x 65) in a U buffer not used before iteration 0
  // Eight waves, two per SIMD: waves 0-3 ("X waves") own the products that produce X, waves 4-7 ("T waves")
  // those that produce T and U, each on quadrant wv & 3. On every SIMD one wave's split-and-store epilogue then
  // runs while the other wave's MFMAs execute.
  const int qd = wv & 3;
  const bool active = qd < NQA;
  const bool xw = active && wv < 4, tw = active && wv >= 4;
  const int r0 = (qd & 1) * TQ, c0 = (qd >> 1) * TQ;  // first row strip and first column strip of the quadrant
  constexpr int NZ = static_cast<int>(sizeof(SplitMat) / sizeof(uint4));
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);

  if constexpr (ST == 1) {
    // K runs over 32 entries while the matrices are 16 wide: the padding must read as zero.
    for (int q = tid; q < NZ; q += NTH) {
      reinterpret_cast<uint4*>(&sX[0])[q] = zero4;
      reinterpret_cast<uint4*>(&sX[1])[q] = zero4;
      reinterpret_cast<uint4*>(&sT[0])[q] = zero4;
      reinterpret_cast<uint4*>(&sT[1])[q] = zero4;
      reinterpret_cast<uint4*>(&sU[0])[q] = zero4;
    }
  }
#pragma unroll
  for (int q = 0; q < 4096 / NTH; ++q) {
    const int idx = tid + NTH * q;
    const int i = idx >> 6, j = idx & 63;
    wf[i * 65 + j] = (i < m && j < m) ? wg[i * m + j] : 0.f;
  }
  if (tid < 3) s_max[tid] = 0u;
  __syncthreads();

  // alpha = 1 / (max_j sum_i |W_ij| * max_i sum_j |W_ij|) in float64: thread (c, quarter) sums 16 entries of
  // column c and of row c, the quarters are combined, then wave 0 takes the maxima (and max |W_ij|).
  if (tid < 256) {
    const int c = tid & 63, qtr = tid >> 6;
    double cs = 0.0, rs = 0.0, mx = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double a = fabs(static_cast<double>(wf[(qtr * 16 + k) * 65 + c]));
      cs += a;
      mx = fmax(mx, a);
      rs += fabs(static_cast<double>(wf[c * 65 + qtr * 16 + k]));
    }
    red[0][qtr][c] = cs;
    red[1][qtr][c] = rs;
    red[2][qtr][c] = mx;
  }
  __syncthreads();
  if (wv == 0) {
    double cs = red[0][0][ln] + red[0][1][ln] + red[0][2][ln] + red[0][3][ln];
    double rs = red[1][0][ln] + red[1][1][ln] + red[1][2][ln] + red[1][3][ln];
    double mx = fmax(fmax(red[2][0][ln], red[2][1][ln]), fmax(red[2][2][ln], red[2][3][ln]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      cs = fmax(cs, __shfl_xor(cs, off));
      rs = fmax(rs, __shfl_xor(rs, off));
      mx = fmax(mx, __shfl_xor(mx, off));
    }
    if (ln == 0) {
      s_alpha = static_cast<float>(1.0 / (cs * rs));
      s_wmax = static_cast<float>(mx);
    }
  }
  __syncthreads();
  const float alpha = s_alpha;
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;

  // W fragments of this wave's row strips (W is the A operand of every product with W), and X_0 = alpha W^T.
  Frags<TQ, KC> fw;
  f32x4 x0c[TQ][TQ], x0r[TQ][TQ];  // X_0 quadrant tiles in the by-columns and the by-rows lane layouts
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int a = 0; a < TQ; ++a) {
      const int i = (r0 + a) * 16 + (ln & 15);
      const int k0 = c * 32 + 8 * (ln >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 h, l;
        split_f16(active ? wf[i * 65 + k0 + e] : 0.f, h, l);
        fw.h[a][c][e] = h;
        fw.l[a][c][e] = l;
      }
    }
  bool inside[TQ][TQ][4];
  float two_i[TQ][TQ][4];  // 2 on the diagonal of the m x m block, 0 elsewhere (padding included)
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b) {
      const int j = (c0 + b) * 16 + (ln & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (r0 + a) * 16 + 4 * (ln >> 4) + r;
        inside[a][b][r] = i < m && j < m;
        two_i[a][b][r] = (i == j && i < m) ? 2.f : 0.f;
        x0c[a][b][r] = active ? alpha * wf[j * 65 + i] : 0.f;
        // by-rows tile (a, b): row (r0 + b) 16 + lane % 16, column (c0 + a) 16 + 4 (lane / 16) + r
        const int ir = (r0 + b) * 16 + (ln & 15), jr = (c0 + a) * 16 + 4 * (ln >> 4) + r;
        x0r[a][b][r] = active ? alpha * wf[jr * 65 + ir] : 0.f;
      }
    }
  __syncthreads();  // wf (inside sU[1]) is dead after this point
  if constexpr (ST == 1) {
    for (int q = tid; q < NZ; q += NTH) reinterpret_cast<uint4*>(&sU[1])[q] = zero4;
  }

  // Lane placement of quadrant tiles. By-columns tile (a, b), a product mma(rows of strips r0.., rows of strips
  // c0..): the lane holds rows col_i0(a) .. +3 of column col_j(b). By-rows tile (a, b), the same product with the
  // operand roles swapped, mma(strips c0.., strips r0..), so a indexes column strips and b row strips: the lane
  // holds columns row_j0(a) .. +3 of row row_i(b).
  auto col_j = [&](int b) { return (c0 + b) * 16 + (ln & 15); };
  auto col_i0 = [&](int a) { return (r0 + a) * 16 + 4 * (ln >> 4); };
  auto row_i = [&](int b) { return (r0 + b) * 16 + (ln & 15); };
  auto row_j0 = [&](int a) { return (c0 + a) * 16 + 4 * (ln >> 4); };
  // Split stores: by-columns tiles into a by-columns buffer, by-rows tiles into a by-rows buffer (8-byte writes).
  auto put_cols = [&](SplitMat& M, const f32x4 v[TQ][TQ], float s) {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) {
        half4 h, l;
        split_scaled4(v[a][b], s, h, l);
        put_t4(M, col_j(b), col_i0(a), h, l);
      }
  };
  auto put_rows = [&](SplitMat& M, const f32x4 v[TQ][TQ], float s) {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) {
        half4 h, l;
        split_scaled4(v[a][b], s, h, l);
        put_t4(M, row_i(b), row_j0(a), h, l);
      }
  };
  // put_rows that also returns the largest |v| (before scaling).
  auto put_rows_max = [&](SplitMat& M, const f32x4 v[TQ][TQ], float s) {
    float lm = 0.f;
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) {
        const f32x4 t = v[a][b];
        lm = fmaxf(lm, fmaxf(fmaxf(fabsf(t[0]), fabsf(t[1])), fmaxf(fabsf(t[2]), fabsf(t[3]))));
        half4 h, l;
        split_scaled4(t, s, h, l);
        put_t4(M, row_i(b), row_j0(a), h, l);
      }
    return lm;
  };
  // U = 2I - s v from by-columns tiles of T (padding rows and columns of T are exact zeros, so U is zero there).
  auto put_u = [&](SplitMat& M, const f32x4 v[TQ][TQ], float s) {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) {
        f32x4 u;
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = two_i[a][b][r] - v[a][b][r] * s;
        half4 h, l;
        split4(u, h, l);
        put_t4(M, col_j(b), col_i0(a), h, l);
      }
  };
  // Iterate k to the saved-iterates buffer, from by-rows tiles (rows_layout) or by-columns tiles.
  auto put_xs = [&](int k, const f32x4 v[TQ][TQ], float s, bool rows_layout) {
    float* xg = xs + (static_cast<size_t>(g) * (iters + 1) + k) * mm;
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = rows_layout ? row_i(b) : col_i0(a) + r;
          const int j = rows_layout ? row_j0(a) + r : col_j(b);
          if (i < m && j < m) xg[i * m + j] = v[a][b][r] * s;
        }
  };
  auto frags_of = [&](const SplitMat& M, int s0, Frags<TQ, KC>& f) {
#pragma unroll
    for (int c = 0; c < KC; ++c) load_chunk<TQ, KC>(M, s0, ln, c, f);
  };
  auto mma = [&](const Frags<TQ, KC>& A, const Frags<TQ, KC>& B, f32x4 acc[TQ][TQ]) {
    zero_acc<TQ>(acc);
#pragma unroll
    for (int c = 0; c < KC; ++c) mma_chunk<TQ, KC>(A, B, acc, c);
  };


  // The exact Newton-Schulz step X_{k+1} = X_k (2I - W X_k) equals, for T_k = W X_k, the pair
  //   T_{k+1} = T_k (2I - T_k),  X_{k+1} = X_k (2I - T_k),
  // whose two products share U_k = 2I - T_k and depend only on step k: one phase and one barrier per step
  // instead of two. Carrying T separately drops the self-correction of the exact step: a mismatch D = T - W X
  // becomes D (2I - T) in the next step, so it can double per step while T has eigenvalues far below 1, about
  // 1 / (alpha mu_min^2) ~ kappa^2 overall. Pair steps therefore run in segments of at most kPairRun, each
  // starting from T = W X formed afresh (the mismatch stays below 2^kPairRun times the rounding of one split
  // product, 2^-22), and the last step is the exact update from X_{K-1}, which squares what is left; the result
  // then tracks the exact-step iteration to rounding.
  int e_cur = store_exp(alpha * s_wmax);  // storage exponent of the iterate in sX[cur]; X_0's max is alpha max|W|
  const int xcol_first = 1;               // buffer of sT that receives X_0 by columns
  if (xw) {
    put_rows(sX[0], x0r, ldexpf(1.f, -e_cur));
    if (xs) put_xs(0, x0c, 1.f, false);
  }
  if (tw) put_cols(sT[xcol_first], x0c, ldexpf(1.f, -e_cur));
  __syncthreads();

  f32x4 accA[TQ][TQ], accB[TQ][TQ], accC[TQ][TQ];
  int xcol_buf = xcol_first;  // where the latest X by columns sits (the segment start and the exact step read it)
  // Segment start at step k: T_k = W X_k by columns (into U_k = 2I - T_k) and, with the operands swapped, by rows.
  // After the first segment, X_k by columns sits in sT[k & 1], the buffer T_k goes to: every T wave loads its
  // fragments before any of them stores.
  auto resync = [&](int k) {
    const int cur = k & 1;
    Frags<TQ, KC> fxc;
    if (tw) frags_of(sT[xcol_buf], c0, fxc);
    if (xcol_buf == cur) __syncthreads();
    if (tw) {
      mma(fw, fxc, accA);
      mma(fxc, fw, accB);
      const float unscale = ldexpf(1.f, e_cur);
      put_u(sU[cur], accA, unscale);
      put_rows(sT[cur], accB, unscale);
    }
    __syncthreads();
  };

  int e_next = e_cur;
  // One pair step; the buffer parity is a template constant so that every LDS address is a fixed offset.
  // last: the step ends a segment, so it produces X_{k+1} by columns as well and no T_{k+1} / U_{k+1}.
  auto step = [&](auto parity, int k, bool last) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
    const float unscale = ldexpf(1.f, e_cur);
    if (xw) {
      Frags<TQ, KC> fu, fx;
      frags_of(sU[cur], c0, fu);
      frags_of(sX[cur], r0, fx);
      mma(fu, fx, accC);  // (X_k U_k)^T: X_{k+1} by rows
      float lmax = put_rows_max(sX[nxt], accC, ldexpf(1.f, e_cur - e_next));
      if (xs) put_xs(k + 1, accC, unscale, true);
      lmax = wave_max_nonneg(lmax) * unscale;
      if (ln == 0) atomicMax(&s_max[k % 3], __float_as_uint(lmax));
    } else if (tw) {
      Frags<TQ, KC> fu, ft;
      frags_of(sU[cur], c0, fu);
      if (!last) {
        frags_of(sT[cur], r0, ft);
        mma(ft, fu, accA);  // T_k U_k by columns: U_{k+1}
        mma(fu, ft, accB);  // (T_k U_k)^T: T_{k+1} by rows
        put_u(sU[nxt], accA, 1.f);
        put_rows(sT[nxt], accB, 1.f);
      } else {
        frags_of(sX[cur], r0, ft);
        mma(ft, fu, accA);  // X_k U_k by columns: X_{K-1} for the exact step
        put_cols(sT[nxt], accA, ldexpf(1.f, e_cur - e_next));
      }
    }
    if (tid == 0) s_max[(k + 1) % 3] = 0u;
    __syncthreads();
    const float mx = __uint_as_float(s_max[k % 3]);
    if (mx >= ldexpf(1.f, e_next + kRestoreExp) || !(mx < 3.0e38f)) {
      // Rare: the iterate grew past the headroom of its exponent (or is not finite); store it again.
      const int e_new = store_exp(fminf(mx, 3.0e38f));
      const float rel = ldexpf(1.f, e_cur - e_new);
      if (xw) put_rows(sX[nxt], accC, rel);
      if (tw && last) put_cols(sT[nxt], accA, rel);
      e_next = e_new;
      __syncthreads();
    }
    e_cur = e_next;
    e_next = store_exp(mx);
    if (last) xcol_buf = nxt;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int k = 0; k + 1 < iters;) {
    resync(k);
    const int end = min(k + kPairRun, iters - 1);  // pair steps k .. end - 1; step K - 1 is the exact one
    // steps in (even, odd) pairs so that each step's buffer parity is a compile-time constant
    if (k & 1) {
      step(P1{}, k, k + 1 == end);
      ++k;
    }
    for (; k + 1 < end; k += 2) {
      step(P0{}, k, false);
      step(P1{}, k + 1, k + 2 == end);
    }
    if (k < end) {
      step(P0{}, k, true);
      ++k;
    }
  }

  // Final exact step (iters >= 1): X_K = X_{K-1} (2I - W X_{K-1}), X_K by columns in accC.
  const int fin = (iters >= 1) ? ((iters - 1) & 1) : 0;  // buffers holding X_{K-1}
  float out_unscale = 1.f;
  if (iters >= 1) {
    const float unscale = ldexpf(1.f, e_cur);
    if (tw) {
      Frags<TQ, KC> fxc;
      frags_of(sT[xcol_buf], c0, fxc);
      mma(fw, fxc, accA);
      put_u(sU[fin], accA, unscale);
    }
    __syncthreads();
    if (xw) {
      Frags<TQ, KC> fx, fu;
      frags_of(sX[fin], r0, fx);
      frags_of(sU[fin], c0, fu);
      mma(fx, fu, accC);
    }
    out_unscale = unscale;
  } else {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) accC[a][b] = x0c[a][b];
  }
  if (xw) {
    if (xs && iters >= 1) put_xs(iters, accC, out_unscale, false);
    float* xo = Xout + g * mm;
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inside[a][b][r]) xo[(col_i0(a) + r) * m + col_j(b)] = accC[a][b][r] * out_unscale;
  }

  if (resid) {
    // ||W X_K - I||_F with the same split products: X_K by columns goes through LDS once more.
    __syncthreads();  // every read of the buffers below is done
    const int rb = fin ^ 1;
    // accC * out_unscale is X_K; store it with the exponent of the last iterate so the fp16 halves stay in range
    const float st_scale = (iters >= 1) ? 1.f : ldexpf(1.f, -e_cur);
    const float ru = out_unscale / st_scale;
    if (xw) put_cols(sT[rb], accC, st_scale);
    __syncthreads();
    double ss = 0.0;
    if (tw) {
      Frags<TQ, KC> fxc;
      frags_of(sT[rb], c0, fxc);
      mma(fw, fxc, accA);
#pragma unroll
      for (int a = 0; a < TQ; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (inside[a][b][r]) {
              const double e2 = static_cast<double>(accA[a][b][r] * ru) -
                                (col_i0(a) + r == col_j(b) ? 1.0 : 0.0);
              ss += e2 * e2;
            }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    __syncthreads();
    if (ln == 0 && wv >= 4) red[0][0][qd] = ss;
    __syncthreads();
    if (tid == 0) resid[g] = static_cast<float>(sqrt(red[0][0][0] + red[0][0][1] + red[0][0][2] + red[0][0][3]));
  }
}

template <int ST, int KC>
__global__ __launch_bounds__(512) void k_ns_small(const float* __restrict__ We, float* __restrict__ Xout,
                                                  float* __restrict__ xs, float* __restrict__ alpha_out,
                                                  float* __restrict__ resid, int m, int iters) {
  ns_small_block<ST, KC>(static_cast<int>(blockIdx.x), We, Xout, xs, alpha_out, resid, m, iters);
}

// =====================================================================================================
// Newton-Schulz with side work. The m <= 64 solver occupies one CU per slice for its whole chain of dependent
// steps while the rest of the chip would idle, and a second stream costs more in cross-queue synchronisation than
// it saves at this size. So the same launch carries, after the G solver blocks, blocks that compute
// S = C_K^T V, each one (slice, 16-landmark tile, 16-channel tile) of S over all N tokens. No block of this launch
// waits for another: a cross-XCD hand-off of partial sums needs device-scope release and acquire fences, and
// on this chip those write back and invalidate a whole L2, which costs more than the solver itself.
// Each block holds the solver's LDS (one block per CU); the tiles fill the CUs the solver leaves free and finish
// inside the solver's time.
// =====================================================================================================

// One S tile by one 512-thread block. Wave w sums a contiguous range of 16-token groups on fp32 MFMA
// (A = C_K, landmark-major, B = V): in group q, lane (i, k) feeds landmark i and channel i of the tile with tokens
// 16q + 4k + u at k-step u, loaded from global memory straight into the MFMA operand layout. The eight wave tiles
// are then summed in LDS in wave order, so the result does not depend on timing.
template <typename T, int D>
__device__ __forceinline__ void ckv_tile_block(int blk, const float* __restrict__ C, const T* __restrict__ V,
                                               float* __restrict__ S, int N, int m, float* sRed) {
  constexpr int DT = D / 16;
  const int LT = (m + 15) / 16;
  const int ct = blk % DT;
  const int lt = (blk / DT) % LT;
  const int g = blk / (DT * LT);
  const int wv = wave_id(), ln = lane_id();
  const int i = ln & 15, k = ln >> 4;
  const bool lok = lt * 16 + i < m;
  const float* __restrict__ crow = C + (static_cast<size_t>(g) * m + (lok ? lt * 16 + i : 0)) * N;
  const T* __restrict__ vcol = V + static_cast<size_t>(g) * N * D + ct * 16 + i;
  const int groups = (N + 15) / 16, gpw = (groups + 7) / 8;
  const int q0 = min(groups, wv * gpw), q1 = min(groups, q0 + gpw);
  const int qf = max(q0, min(q1, N / 16));  // groups [q0, qf) have all 16 tokens in range
  const float amask = lok ? 1.f : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto full_groups = [&](auto vec) {
#pragma unroll 4
    for (int q = q0; q < qf; ++q) {
      const int t = q * 16 + 4 * k;
      float a[4], b[4];
      if constexpr (decltype(vec)::value) {
        const float4 c4 = load4(crow + t);
        a[0] = c4.x;
        a[1] = c4.y;
        a[2] = c4.z;
        a[3] = c4.w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = crow[t + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = to_f32(vcol[static_cast<size_t>(t + u) * D]);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = mfma16x16x4(a[u] * amask, b[u], acc);
    }
  };
  if ((N & 3) == 0)
    full_groups(std::integral_constant<bool, true>{});
  else
    full_groups(std::integral_constant<bool, false>{});
  for (int q = qf; q < q1; ++q) {  // the ragged last group
    const int t = q * 16 + 4 * k;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = t + u < N;
      const float a = in ? crow[t + u] * amask : 0.f;
      const float b = in ? to_f32(vcol[static_cast<size_t>(t + u) * D]) : 0.f;
      acc = mfma16x16x4(a, b, acc);
    }
  }
  // acc[r] is row 4k + r, column i of this wave's tile
#pragma unroll
  for (int r = 0; r < 4; ++r) sRed[wv * 256 + (4 * k + r) * 16 + i] = acc[r];
  __syncthreads();
  const int tid = static_cast<int>(threadIdx.x);
  if (tid < 256) {
    const int row = tid >> 4, col = tid & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += sRed[w * 256 + tid];
    if (lt * 16 + row < m) S[(static_cast<size_t>(g) * m + lt * 16 + row) * D + ct * 16 + col] = sum;
  }
}

template <typename T, int D, int ST, int KC>
__global__ __launch_bounds__(512) void k_ns_side(const float* __restrict__ We, float* __restrict__ Xout,
                                                 float* __restrict__ xs, float* __restrict__ alpha_out, int m,
                                                 int iters, int N, int G, const float* __restrict__ CK,
                                                 const T* __restrict__ V, float* __restrict__ S) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < G) {
    ns_small_block<ST, KC>(b, We, Xout, xs, alpha_out, nullptr, m, iters);
    return;
  }
  // The S tiles start at the first multiple of 8 after the solver blocks (the blocks in between exit at once), so
  // that tile j runs on XCD j % 8 (the hardware deals blocks to the 8 XCDs round-robin). Their order is remapped so
  // that the tiles of one slice share an XCD: each slice's C_K rows and V columns are read by several tiles, and
  // one L2 then serves the repeats.
  const int s0 = (G + 7) & ~7;
  if (b < s0) return;
  int j = b - s0;
  {
    const int total = static_cast<int>(gridDim.x) - s0, full = (total / 8) * 8;
    if (j < full) j = (j % 8) * (full / 8) + j / 8;
  }
  __shared__ float sRed[8 * 256];
  ckv_tile_block<T, D>(j, CK, V, S, N, m, sRed);
}

template <typename T, int D>
static void ns_side_st(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                       const T* V, float* S, hipStream_t st) {
  const int blocks = ((s.G + 7) & ~7) + s.G * ((s.m + 15) / 16 * (D / 16));  // solver blocks, padding, S tiles
  const int nt = (s.m + 15) / 16;
#define LF_NS_SIDE(ST_, KC_)                                                                                        \
  hipLaunchKernelGGL((k_ns_side<T, D, ST_, KC_>), dim3(blocks), dim3(512), 0, st, We, X, xs, alpha, s.m, s.ns_iters, \
                     s.N, s.G, CK, V, S)
  if (nt == 1)
    LF_NS_SIDE(1, 1);
  else if (nt == 2)
    LF_NS_SIDE(2, 1);
  else
    LF_NS_SIDE(4, 2);
#undef LF_NS_SIDE
}

bool ns_side_supported(const Shape& s) {
  return s.m <= 64 && (s.d == 16 || s.d == 32 || s.d == 64) && s.G < 256;
}

template <typename T>
static void ns_side_t(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                      const void* V, float* S, hipStream_t st) {
  const T* v = static_cast<const T*>(V);
  switch (s.d) {
    case 16: ns_side_st<T, 16>(s, We, X, xs, alpha, CK, v, S, st); break;
    case 32: ns_side_st<T, 32>(s, We, X, xs, alpha, CK, v, S, st); break;
    default: ns_side_st<T, 64>(s, We, X, xs, alpha, CK, v, S, st); break;
  }
}

hipError_t launch_ns_side(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                          const void* V, float* S, hipStream_t st) {
  if (!ns_side_supported(s)) return hipErrorInvalidValue;
  if (s.dtype == 1)
    ns_side_t<bf16_t>(s, We, X, xs, alpha, CK, V, S, st);
  else
    ns_side_t<float>(s, We, X, xs, alpha, CK, V, S, st);
  return hipGetLastError();
}

// =====================================================================================================
// m > 64: the m x m matrices do not fit one CU's LDS, so every product is a batched launch over 32 x 32 output
// tiles (4 waves of 16 x 16, fp32 MFMA), K staged through LDS in chunks of 32 with the next chunk's float4 loads
// in flight during the current chunk's MFMAs. The steps follow the small kernel: segments of at most kPairRunF32
// steps start from T_k = W X_k, then one launch per step computes both T_{k+1} = T_k U_k and X_{k+1} = X_k U_k
// with U_k = 2I - T_k formed while staging, and the last step is the exact one, X_K = X_{K-1} (2I - W X_{K-1}),
// in two launches.
// =====================================================================================================
// alpha and X_0 = alpha W^T for m > 64, over (slice, kNsRows-row chunk) blocks. Pass 1 writes per-chunk partial
// column sums and the largest row sum of the chunk; pass 2 combines them in a fixed order (deterministic) and
// writes the chunk's rows of X_0. part: G * nchunk * m doubles, rmx: G * nchunk doubles.
constexpr int kNsRows = 8;  // rows per chunk of the alpha sums and of X_0: m / 8 chunks spread a slice over blocks

__global__ __launch_bounds__(256) void k_ns_sums(const float* __restrict__ We, double* __restrict__ part,
                                                 double* __restrict__ rmx, int m) {
  __shared__ double red[4];
  const int g = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const float* wg = We + static_cast<size_t>(g) * m * m;
  const int r0 = ch * kNsRows, r1 = min(m, r0 + kNsRows);
  for (int j = tid; j < m; j += 256) {
    double cs = 0.0;
#pragma unroll 8
    for (int i = r0; i < r1; ++i) cs += fabs(static_cast<double>(wg[static_cast<size_t>(i) * m + j]));
    part[(static_cast<size_t>(g) * nch + ch) * m + j] = cs;
  }
  double rmax = 0.0;
  for (int i = r0 + wv; i < r1; i += 4) {
    double rs = 0.0;
    for (int j = ln; j < m; j += 64) rs += fabs(static_cast<double>(wg[static_cast<size_t>(i) * m + j]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) rs += __shfl_xor(rs, off);
    rmax = fmax(rmax, rs);
  }
  if (ln == 0) red[wv] = rmax;
  __syncthreads();
  if (tid == 0) rmx[static_cast<size_t>(g) * nch + ch] = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

__global__ __launch_bounds__(256) void k_ns_x0(const float* __restrict__ We, const double* __restrict__ part,
                                               const double* __restrict__ rmx, float* __restrict__ X0,
                                               float* __restrict__ X0b, size_t strideX0b,
                                               float* __restrict__ alpha_out, int m) {
  __shared__ double red[256];
  __shared__ float s_alpha;
  const int g = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  const int tid = threadIdx.x;
  double cmax = 0.0;
  constexpr int kMaxCh = 256 / kNsRows;  // chunks of the largest m
  for (int j = tid; j < m; j += 256) {
    double pv[kMaxCh];  // every chunk's partial in flight, then summed in chunk order
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c) pv[c] = c < nch ? part[(static_cast<size_t>(g) * nch + c) * m + j] : 0.0;
    double cs = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c)
      if (c < nch) cs += pv[c];
    cmax = fmax(cmax, cs);
  }
  red[tid] = cmax;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] = fmax(red[tid], red[tid + s2]);
    __syncthreads();
  }
  if (tid == 0) {
    double rmax = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c)
      if (c < nch) rmax = fmax(rmax, rmx[static_cast<size_t>(g) * nch + c]);
    s_alpha = static_cast<float>(1.0 / (red[0] * rmax));
    if (ch == 0 && alpha_out) alpha_out[g] = s_alpha;
  }
  __syncthreads();
  const float alpha = s_alpha;
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  float* x0 = X0 + g * mm;
  float* x0b = X0b ? X0b + g * strideX0b : nullptr;
  const int r0 = ch * kNsRows, r1 = min(m, r0 + kNsRows);
  // X_0[i][j] = alpha W[j][i]: thread j reads the consecutive entries W[j][r0 .. r1) of its row and writes
  // column j of rows r0 .. r1 (each store instruction covers 256 consecutive floats of one row).
  for (int j = tid; j < m; j += 256) {
#pragma unroll 8
    for (int i = r0; i < r1; ++i) {
      const float v = alpha * wg[static_cast<size_t>(j) * m + i];
      x0[static_cast<size_t>(i) * m + j] = v;
      if (x0b) x0b[static_cast<size_t>(i) * m + j] = v;
    }
  }
}

constexpr int LF_NS_KMAX = 256;  // largest m of the batched path (the library's m limit)

struct MMJob {
  const float* A[2];
  float* C[2];
  float* C2;  // job 1 only
  size_t strideC2;
};

template <int BOP, int EPI>
__global__ __launch_bounds__(256) void k_ns_mm(MMJob job, const float* __restrict__ B, int m) {
  // The whole K extent is staged at once: A strip [32 rows][m] and B strip [m][32 columns] (m <= 256), so a
  // launch pays one round of global-load latency and then runs its MFMAs back to back.
  constexpr int KMAX = LF_NS_KMAX;
  constexpr int LDA = KMAX + 4;  // A rows: 4 mod 32
  constexpr int LDB = 36;        // B rows (32 columns): 4 mod 32
  constexpr int NCH = KMAX / 32;
  __shared__ float sA[32 * LDA];
  __shared__ float sB[KMAX * LDB];
  const int g = blockIdx.z >> 1, which = blockIdx.z & 1;
  if (job.A[which] == nullptr) return;  // this launch has no such job (uniform over the block)
  const size_t mm = static_cast<size_t>(m) * m;
  const float* ag = job.A[which] + g * mm;
  const float* bg = B + g * mm;
  float* cg = job.C[which] + g * mm;
  const int tm = blockIdx.y * 32, tn = blockIdx.x * 32;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const int wr = (wv >> 1) * 16, wc = (wv & 1) * 16;
  // Staging map per 32 x 32 chunk: thread -> (row rr, columns cc .. cc + 3).
  const int rr = tid >> 3, cc = 4 * (tid & 7);
  const bool vec = (m & 3) == 0;
  const int nch = (m + 31) / 32;
  // Branch-free staging: every load address is clamped into the slice and out-of-range values are selected to
  // zero, so all chunks' loads are issued before the first wait.
  auto ld = [&](const float* base, int i, int k, bool ok) {
    return ok ? base[static_cast<size_t>(i) * m + k] : 0.f;
  };
  float4 va[NCH], vb[NCH];
  if (vec) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ai = tm + rr, ak = 32 * c + cc;  // A[ai][ak .. ak + 3]
      const int bk = 32 * c + rr, bj = tn + cc;  // B[bk][bj .. bj + 3]
      const bool aok = c < nch && ai < m && ak + 3 < m, bok = c < nch && bk < m && bj + 3 < m;
      const float4 x = load4(ag + (aok ? static_cast<size_t>(ai) * m + ak : 0));
      const float4 y = load4(bg + (bok ? static_cast<size_t>(bk) * m + bj : 0));
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      va[c] = aok ? x : z;
      vb[c] = bok ? y : z;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ai = tm + rr, ak = 32 * c + cc;
      const int bk = 32 * c + rr, bj = tn + cc;
      const bool arow = c < nch && ai < m, brow = c < nch && bk < m;
      va[c] = make_float4(ld(ag, arow ? ai : 0, arow && ak + 0 < m ? ak + 0 : 0, arow && ak + 0 < m),
                          ld(ag, arow ? ai : 0, arow && ak + 1 < m ? ak + 1 : 0, arow && ak + 1 < m),
                          ld(ag, arow ? ai : 0, arow && ak + 2 < m ? ak + 2 : 0, arow && ak + 2 < m),
                          ld(ag, arow ? ai : 0, arow && ak + 3 < m ? ak + 3 : 0, arow && ak + 3 < m));
      vb[c] = make_float4(ld(bg, brow ? bk : 0, brow && bj + 0 < m ? bj + 0 : 0, brow && bj + 0 < m),
                          ld(bg, brow ? bk : 0, brow && bj + 1 < m ? bj + 1 : 0, brow && bj + 1 < m),
                          ld(bg, brow ? bk : 0, brow && bj + 2 < m ? bj + 2 : 0, brow && bj + 2 < m),
                          ld(bg, brow ? bk : 0, brow && bj + 3 < m ? bj + 3 : 0, brow && bj + 3 < m));
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (BOP == 1) {  // 2I - B, zero outside the m x m block
      const int bk = 32 * c + rr, bj = tn + cc;
      vb[c].x = (bk < m && bj + 0 < m) ? ((bk == bj + 0) ? 2.f : 0.f) - vb[c].x : 0.f;
      vb[c].y = (bk < m && bj + 1 < m) ? ((bk == bj + 1) ? 2.f : 0.f) - vb[c].y : 0.f;
      vb[c].z = (bk < m && bj + 2 < m) ? ((bk == bj + 2) ? 2.f : 0.f) - vb[c].z : 0.f;
      vb[c].w = (bk < m && bj + 3 < m) ? ((bk == bj + 3) ? 2.f : 0.f) - vb[c].w : 0.f;
    }
    if (c < nch) {
      *reinterpret_cast<float4*>(&sA[rr * LDA + 32 * c + cc]) = va[c];
      *reinterpret_cast<float4*>(&sB[(32 * c + rr) * LDB + cc]) = vb[c];
    }
  }
  __syncthreads();
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;  // two chains over alternate k-steps
  const int ksteps = nch * 8;
#pragma unroll 4
  for (int ks = 0; ks < ksteps; ks += 2) {
    const int k = ks * 4 + (ln >> 4);
    acc0 = mfma16x16x4(sA[(wr + (ln & 15)) * LDA + k], sB[k * LDB + wc + (ln & 15)], acc0);
    acc1 = mfma16x16x4(sA[(wr + (ln & 15)) * LDA + k + 4], sB[(k + 4) * LDB + wc + (ln & 15)], acc1);
  }
  const int j = tn + wc + (ln & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = tm + wr + 4 * (ln >> 4) + r;
    if (i < m && j < m) {
      float v = acc0[r] + acc1[r];
      if (EPI == 1) v = (i == j ? 2.f : 0.f) - v;
      if (EPI == 2) v -= (i == j ? 1.f : 0.f);
      cg[static_cast<size_t>(i) * m + j] = v;
      if (which == 1 && job.C2) job.C2[g * job.strideC2 + static_cast<size_t>(i) * m + j] = v;
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
  return s.m > 64 ? 3 * static_cast<size_t>(s.G) * s.m * s.m : 0;
}

hipError_t launch_ns(const Shape& s, const float* We, float* X, float* xs, float* alpha, float* resid, float* tmp,
                     hipStream_t st) {
  const int m = s.m, K = s.ns_iters;
  if (m <= 64) {
    const int nt = (m + 15) / 16;
    const dim3 grid(s.G), block(512);
    if (nt == 1)
      hipLaunchKernelGGL((k_ns_small<1, 1>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else if (nt == 2)
      hipLaunchKernelGGL((k_ns_small<2, 1>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else
      hipLaunchKernelGGL((k_ns_small<4, 2>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    return hipGetLastError();
  }
  const size_t mm = static_cast<size_t>(m) * m, Gmm = static_cast<size_t>(s.G) * mm;
  float* Tb[2] = {tmp, tmp + Gmm};  // T_k by parity; Tb[..] also serves as U' and the residual
  float* Xalt = tmp + 2 * Gmm;
  // X_k alternates between two buffers so that X_K lands in X.
  float* Xb[2] = {X, Xalt};
  const size_t xs_stride = static_cast<size_t>(K + 1) * mm;
  const int tiles = (m + 31) / 32;
  const dim3 blk(256);
  auto slot = [&](int k) { return xs ? xs + static_cast<size_t>(k) * mm : nullptr; };
  // X_0 lands where the last exact step reads X_{K-1} from when K == 1, else where step 0 reads it.
  int xc = (K % 2 == 0) ? 0 : 1;  // parity such that X_K ends in Xb[0] = X (K steps, one flip per step)
  {
    const int nch = (m + kNsRows - 1) / kNsRows;
    // G nch m + G nch doubles fit in one T buffer (m > 64); Tb[0] starts the 256-byte aligned scratch and is not
    // written before T_0.
    double* part = reinterpret_cast<double*>(Tb[0]);
    double* rmx = part + static_cast<size_t>(s.G) * nch * m;
    hipLaunchKernelGGL(k_ns_sums, dim3(s.G, nch), blk, 0, st, We, part, rmx, m);
    hipLaunchKernelGGL(k_ns_x0, dim3(s.G, nch), blk, 0, st, We, part, rmx, Xb[xc], xs, xs_stride, alpha, m);
  }
  int tc = 0;
  for (int k = 0; k + 1 < K;) {
    // segment start: T_k = W X_k
    MMJob j0{{We, nullptr}, {Tb[tc], nullptr}, nullptr, 0};
    hipLaunchKernelGGL((k_ns_mm<0, 0>), dim3(tiles, tiles, 2 * s.G), blk, 0, st, j0, Xb[xc], m);
    const int end = std::min(k + kPairRunF32, K - 1);
    for (; k < end; ++k) {
      const bool last = k + 1 == end;
      // pair step: job 0: T_{k+1} = T_k (2I - T_k) (skipped at a segment's end), job 1: X_{k+1} = X_k (2I - T_k)
      MMJob jp{{last ? nullptr : Tb[tc], Xb[xc]}, {last ? nullptr : Tb[tc ^ 1], Xb[xc ^ 1]}, slot(k + 1),
               xs_stride};
      hipLaunchKernelGGL((k_ns_mm<1, 0>), dim3(tiles, tiles, 2 * s.G), blk, 0, st, jp, Tb[tc], m);
      tc ^= 1;
      xc ^= 1;
    }
  }
  if (K >= 1) {
    // exact step: U' = 2I - W X_{K-1} (into a T buffer), then X_K = X_{K-1} U'
    float* Up = Tb[tc ^ 1];
    MMJob ju{{We, nullptr}, {Up, nullptr}, nullptr, 0};
    hipLaunchKernelGGL((k_ns_mm<0, 1>), dim3(tiles, tiles, 2 * s.G), blk, 0, st, ju, Xb[xc], m);
    MMJob jx{{nullptr, Xb[xc]}, {nullptr, Xb[xc ^ 1]}, slot(K), xs_stride};
    hipLaunchKernelGGL((k_ns_mm<0, 0>), dim3(tiles, tiles, 2 * s.G), blk, 0, st, jx, Up, m);
    xc ^= 1;
  }
  if (resid) {
    MMJob jr{{We, nullptr}, {Tb[tc], nullptr}, nullptr, 0};
    hipLaunchKernelGGL((k_ns_mm<0, 2>), dim3(tiles, tiles, 2 * s.G), blk, 0, st, jr, Xb[xc], m);
    hipLaunchKernelGGL(k_frob, dim3(s.G), dim3(256), 0, st, Tb[tc], resid, m);
  }
  return hipGetLastError();
}

}  // namespace lf
