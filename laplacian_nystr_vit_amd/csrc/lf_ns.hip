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

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Splits two fp32 values into packed fp16 halves: hi2 = (hi(x), hi(y)) rounded to nearest, lo2 = (lo(x), lo(y))
// with lo = round_f16(v - hi); v - hi is exact in fp32, so lo is its correctly rounded fp16 value. Three
// instructions: a pack conversion and two mixed-precision FMAs that read hi as fp16.
__device__ __forceinline__ void split2(float x, float y, unsigned int& hi2, unsigned int& lo2) {
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(hi2) : "v"(x), "v"(y));
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(lo2) : "v"(x), "v"(hi2));
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(lo2) : "v"(y), "v"(hi2));
}

__device__ __forceinline__ void split4(f32x4 v, half4& h, half4& l) {
  u32x2 hh, ll;
  unsigned int h0, h1, l0, l1;
  split2(v[0], v[1], h0, l0);
  split2(v[2], v[3], h1, l1);
  hh[0] = h0;
  hh[1] = h1;
  ll[0] = l0;
  ll[1] = l1;
  h = __builtin_bit_cast(half4, hh);
  l = __builtin_bit_cast(half4, ll);
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
__global__ __launch_bounds__(256) void k_ns_small(const float* __restrict__ We, float* __restrict__ Xout,
                                                  float* __restrict__ xs, float* __restrict__ alpha_out,
                                                  float* __restrict__ resid, int m, int iters) {
  constexpr int TQ = ST >= 2 ? ST / 2 : 1;  // tiles per side of a wave's quadrant
  constexpr int NWA = ST == 1 ? 1 : 4;      // waves with work
  __shared__ SplitMat sX[2], sXt[2], sUt;
  __shared__ double red[3][4][64];
  __shared__ float s_alpha, s_wmax;
  __shared__ unsigned int s_max[2];  // bits of the largest |X| entry of the iterate written in an iteration
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  float* wf = reinterpret_cast<float*>(&sUt);  // fp32 W (64 x 65) in the not yet used U area
  const bool active = wv < NWA;
  const int r0 = (wv & 1) * TQ, c0 = (wv >> 1) * TQ;  // first row strip and first column strip of the quadrant

  if constexpr (ST == 1) {
    // K runs over 32 entries while the matrices are 16 wide: the padding must read as zero.
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    constexpr int NZ = static_cast<int>(sizeof(SplitMat) / sizeof(uint4));
    for (int q = tid; q < NZ; q += 256) {
      reinterpret_cast<uint4*>(&sX[0])[q] = zero;
      reinterpret_cast<uint4*>(&sX[1])[q] = zero;
      reinterpret_cast<uint4*>(&sXt[0])[q] = zero;
      reinterpret_cast<uint4*>(&sXt[1])[q] = zero;
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int idx = tid + 256 * q;
    const int i = idx >> 6, j = idx & 63;
    wf[i * 65 + j] = (i < m && j < m) ? wg[i * m + j] : 0.f;
  }
  if (tid < 2) s_max[tid] = 0u;
  __syncthreads();

  // alpha = 1 / (max_j sum_i |W_ij| * max_i sum_j |W_ij|) in float64: thread (c, quarter) sums 16 entries of
  // column c and of row c, the quarters are combined, then wave 0 takes the maxima (and max |W_ij|).
  {
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

  // W fragments of this wave's row strips (A operand of W X), and X_0 = alpha W^T in fp32 registers.
  Frags<TQ, KC> fw;
  f32x4 x0c[TQ][TQ], x0r[TQ][TQ];  // X_0 = alpha W^T as quadrant tiles by columns, and by rows (see put_x)
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
        // by rows: row (r0 + a) 16 + lane % 16, column (c0 + b) 16 + 4 (lane / 16) + r
        const int ir = (r0 + a) * 16 + (ln & 15), jr = (c0 + b) * 16 + 4 * (ln >> 4) + r;
        x0r[a][b][r] = active ? alpha * wf[jr * 65 + ir] : 0.f;
      }
    }
  __syncthreads();  // wf (inside sUt) is dead after this point
  if constexpr (ST == 1) {
    constexpr int NZ = static_cast<int>(sizeof(SplitMat) / sizeof(uint4));
    for (int q = tid; q < NZ; q += 256) reinterpret_cast<uint4*>(&sUt)[q] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Tile (a, b) of the quadrant: column j and first row i0 of the lane's four entries.
  auto tile_j = [&](int b) { return (c0 + b) * 16 + (ln & 15); };
  auto tile_i0 = [&](int a) { return (r0 + a) * 16 + 4 * (ln >> 4); };
  // Stores an iterate into buffer `buf`: px holds its quadrant tiles (by columns), pt the tiles of its
  // transpose (by rows), both multiplied by s on the way.
  auto put_x = [&](int buf, const f32x4 px[TQ][TQ], const f32x4 pt[TQ][TQ], float s) {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b) {
        half4 h, l;
        split_scaled4(px[a][b], s, h, l);
        put_t4(sXt[buf], tile_j(b), tile_i0(a), h, l);
        // pt[a][b]: entries (row (r0 + a) 16 + lane % 16, columns (c0 + b) 16 + 4 (lane / 16) + 0 .. 3)
        split_scaled4(pt[a][b], s, h, l);
        put_t4(sX[buf], (r0 + a) * 16 + (ln & 15), (c0 + b) * 16 + 4 * (ln >> 4), h, l);
      }
  };
  auto put_xs = [&](int k, const f32x4 px[TQ][TQ], float s) {
    float* xg = xs + (static_cast<size_t>(g) * (iters + 1) + k) * mm;
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inside[a][b][r]) xg[(tile_i0(a) + r) * m + tile_j(b)] = px[a][b][r] * s;
  };

  f32x4 accx[TQ][TQ], acct[TQ][TQ], acc[TQ][TQ];
  int e_cur = store_exp(alpha * s_wmax);  // X_0's largest entry is alpha max |W_ij|
  __syncthreads();                        // (ST == 1) padding of U cleared
  if (active) {
    put_x(0, x0c, x0r, ldexpf(1.f, -e_cur));
    if (xs) put_xs(0, x0c, 1.f);
  }
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int b = 0; b < TQ; ++b) accx[a][b] = x0c[a][b];  // the output when iters == 0
  __syncthreads();

  int e_next = e_cur;
  float last_unscale = 1.f;
  for (int it = 0; it < iters; ++it) {
    const int cur = it & 1, nxt = cur ^ 1;
    const float unscale = ldexpf(1.f, e_cur);
    // T = W X ; U = 2I - T, stored by columns. Padding rows and columns of T are exact zeros, so U is zero there.
    if (active) {
      Frags<TQ, KC> fx;
#pragma unroll
      for (int c = 0; c < KC; ++c) load_chunk<TQ, KC>(sXt[cur], c0, ln, c, fx);
      zero_acc<TQ>(acc);
#pragma unroll
      for (int c = 0; c < KC; ++c) mma_chunk<TQ, KC>(fw, fx, acc, c);
#pragma unroll
      for (int a = 0; a < TQ; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b) {
          f32x4 u;
#pragma unroll
          for (int r = 0; r < 4; ++r) u[r] = two_i[a][b][r] - acc[a][b][r] * unscale;
          half4 h, l;
          split4(u, h, l);
          put_t4(sUt, tile_j(b), tile_i0(a), h, l);
        }
    }
    __syncthreads();
    if (tid == 0) s_max[nxt] = 0u;  // read by every wave in the previous iteration, before the barrier above
    // X_next = X U, and its transpose U^T X^T from the same fragments
    if (active) {
      Frags<TQ, KC> fa, fb;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        load_chunk<TQ, KC>(sX[cur], r0, ln, c, fa);
        load_chunk<TQ, KC>(sUt, c0, ln, c, fb);
      }
      zero_acc<TQ>(accx);
      zero_acc<TQ>(acct);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        mma_chunk<TQ, KC>(fa, fb, accx, c);
        mma_chunk<TQ, KC>(fb, fa, acct, c);
      }
      float lmax = 0.f;
#pragma unroll
      for (int a = 0; a < TQ; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, fabsf(accx[a][b][r]));
      lmax = wave_max_nonneg(lmax) * unscale;
      if (ln == 0) atomicMax(&s_max[cur], __float_as_uint(lmax));
      // acct[b][a] holds the transposed tile of (a, b): swap the indices into put_x's by-rows argument
      f32x4 tt[TQ][TQ];
#pragma unroll
      for (int a = 0; a < TQ; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b) tt[a][b] = acct[b][a];
      put_x(nxt, accx, tt, ldexpf(1.f, e_cur - e_next));
      if (xs) put_xs(it + 1, accx, unscale);
    }
    __syncthreads();
    const float mx = __uint_as_float(s_max[cur]);
    if (mx >= ldexpf(1.f, e_next + kRestoreExp) || !(mx < 3.0e38f)) {
      // Rare: the iterate grew past the headroom of its exponent (or is not finite); store it again.
      const int e_new = store_exp(fminf(mx, 3.0e38f));
      if (active) {
        f32x4 tt[TQ][TQ];
#pragma unroll
        for (int a = 0; a < TQ; ++a)
#pragma unroll
          for (int b = 0; b < TQ; ++b) tt[a][b] = acct[b][a];
        put_x(nxt, accx, tt, ldexpf(1.f, e_cur - e_new));
      }
      e_next = e_new;
      __syncthreads();
    }
    last_unscale = unscale;
    e_cur = e_next;
    e_next = store_exp(mx);
  }

  float* xo = Xout + g * mm;
  if (active) {
#pragma unroll
    for (int a = 0; a < TQ; ++a)
#pragma unroll
      for (int b = 0; b < TQ; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inside[a][b][r]) xo[(tile_i0(a) + r) * m + tile_j(b)] = accx[a][b][r] * last_unscale;
  }

  if (resid) {
    // ||W X - I||_F with the same split products
    double ss = 0.0;
    if (active) {
      Frags<TQ, KC> fx;
#pragma unroll
      for (int c = 0; c < KC; ++c) load_chunk<TQ, KC>(sXt[iters & 1], c0, ln, c, fx);
      zero_acc<TQ>(acc);
#pragma unroll
      for (int c = 0; c < KC; ++c) mma_chunk<TQ, KC>(fw, fx, acc, c);
      const float unscale = ldexpf(1.f, e_cur);  // the exponent X_iters was stored with
#pragma unroll
      for (int a = 0; a < TQ; ++a)
#pragma unroll
        for (int b = 0; b < TQ; ++b) {
          const int j = (c0 + b) * 16 + (ln & 15);
          const int i0 = (r0 + a) * 16 + 4 * (ln >> 4);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (inside[a][b][r]) {
              const double e2 = static_cast<double>(acc[a][b][r] * unscale) - (i0 + r == j ? 1.0 : 0.0);
              ss += e2 * e2;
            }
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
