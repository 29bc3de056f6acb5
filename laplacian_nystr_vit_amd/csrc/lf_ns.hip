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
#include "lf_split.h"

namespace lf {

// =====================================================================================================
// m <= 64: one 512-thread block (eight waves, two per SIMD) per slice runs every iteration out of LDS.
//
// Products run on the fp16 MFMA (v_mfma_f32_16x16x32_f16, 16x the fp32 MFMA rate on gfx950) with every fp32
// operand split as x = hi + lo (two fp16 values, about 22 significant bits) and
//   A B ~= A_hi B_hi + (A_hi B_lo + A_lo B_hi),
// accumulated in fp32. Three fp16 MFMAs cost less than a fifth of one fp32 MFMA product, and the result tracks an
// fp32 product to a few units of 1e-7.
//
// Every matrix is zero-padded to 16 ST x 16 ST (ST = 1, 2 or 4 strips of 16) and stored in LDS by columns (the
// entries of column j contiguous), which is the layout the MFMA result has (four consecutive rows of one column
// per lane, one 8-byte store per split half). A product reads its B operand (columns, K-contiguous) with plain
// 16-byte reads and its A operand (rows) with gfx950's transposing LDS read, ds_read_b64_tr_b16: within each group
// of 16 lanes, result lane j, element s comes from element j % 4 of the 8 bytes lane 4 s + j / 4 addressed, so
// two such reads at columns k = 8 (lane / 16) + 4 h + (lane % 16) / 4 give a lane its row's eight consecutive K
// values. Each matrix is therefore read as itself, never as its transpose: X_k is symmetric only in exact
// arithmetic, and feeding X_k^T where the recurrence has X_k doubles the antisymmetric part of the rounding error
// every step. W, the A operand of W X, never changes: its fragments stay in registers.
//
// A step of the coupled recurrence (below) is two products that share their B operand U_k = 2I - T_k:
// T_{k+1} = T_k U_k and X_{k+1} = X_k U_k. With 64-wide matrices each wave takes one row strip and two column
// strips of a quadrant in both products (24 MFMAs, 16 KB of fragments, T_{k+1}, U_{k+1} = 2I - T_{k+1} and
// X_{k+1} stored from its accumulators), so the two waves of a SIMD carry equal work and each one's epilogue
// overlaps the other's MFMAs. With narrower matrices (one tile per quadrant) waves 0-3 form T and U and waves 4-7
// form X. Every buffer is double-buffered by step parity, so a step needs one barrier.
//
// X carries a power-of-two scale 2^-e in its fp16 halves: e follows the largest entry of the previous iterate
// so that entries sit near 2^12 (far from fp16's subnormals and its 65504 limit); an iterate that still comes
// out above 2^15 is stored again with a fresh exponent. W needs no scale (entries at most 1 + eps) and neither
// do T and U (the eigenvalues of W X stay in (0, 1]).
// =====================================================================================================

constexpr int NH = 72;  // fp16 elements per LDS column: 64 + 8 (144-byte stride, 16-byte aligned)

struct alignas(16) SplitMat {
  _Float16 hi[64 * NH];
  _Float16 lo[64 * NH];
};


// Operand fragments of TQ consecutive 16-row (or 16-column) strips over KC chunks of 32 along K.
template <int TQ, int KC>
struct Frags {
  half8 h[TQ][KC], l[TQ][KC];
};

// B operand: chunk c (K entries 32 c .. 32 c + 31) of column strips s0 .. s0+TQ-1 of a by-columns split matrix
// (element (k, j) at j*NH + k): one 16-byte read per lane and half.
template <int TQ, int KC>
__device__ __forceinline__ void load_chunk_b(const SplitMat& M, int s0, int ln, int c, Frags<TQ, KC>& f) {
#pragma unroll
  for (int a = 0; a < TQ; ++a) {
    const int j = (s0 + a) * 16 + (ln & 15);
    const int k0 = c * 32 + 8 * (ln >> 4);
    f.h[a][c] = *reinterpret_cast<const half8*>(&M.hi[j * NH + k0]);
    f.l[a][c] = *reinterpret_cast<const half8*>(&M.lo[j * NH + k0]);
  }
}


// A operand: chunk c of row strips s0 .. s0+TQ-1 of the same by-columns matrix (element (i, k) at k*NH + i), by
// transposing reads: lane t of lane group g addresses column k = 32 c + 8 g + 4 h + t / 4, rows 4 (t % 4) .. + 3
// of the strip, and receives row 16 strip + t at K = 32 c + 8 g + 4 h .. + 3.
template <int TQ, int KC>
__device__ __forceinline__ void load_chunk_a(const SplitMat& M, int s0, int ln, int c, Frags<TQ, KC>& f) {
  const int g = ln >> 4, t = ln & 15;
#pragma unroll
  for (int a = 0; a < TQ; ++a) {
    const int i = (s0 + a) * 16 + 4 * (t & 3);
    const int k0 = c * 32 + 8 * g + (t >> 2);
    const short4v h0 = lds_read_tr(&M.hi[k0 * NH + i]), h1 = lds_read_tr(&M.hi[(k0 + 4) * NH + i]);
    const short4v l0 = lds_read_tr(&M.lo[k0 * NH + i]), l1 = lds_read_tr(&M.lo[(k0 + 4) * NH + i]);
    const half4 hh0 = __builtin_bit_cast(half4, h0), hh1 = __builtin_bit_cast(half4, h1);
    const half4 ll0 = __builtin_bit_cast(half4, l0), ll1 = __builtin_bit_cast(half4, l1);
    f.h[a][c] = half8{hh0[0], hh0[1], hh0[2], hh0[3], hh1[0], hh1[1], hh1[2], hh1[3]};
    f.l[a][c] = half8{ll0[0], ll0[1], ll0[2], ll0[3], ll1[0], ll1[1], ll1[2], ll1[3]};
  }
}

template <int TA, int TB>
__device__ __forceinline__ void zero_acc(f32x4 acc[TA][TB]) {
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc[a][b] += A-strip a times B-strip b over chunk c. One fp32 accumulator per tile takes hi*hi and both cross
// terms: each MFMA step rounds at fp32 relative to the running sum, which keeps the product at fp32 accuracy.
template <int TA, int TB, int KC>
__device__ __forceinline__ void mma_chunk(const Frags<TA, KC>& A, const Frags<TB, KC>& B, f32x4 acc[TA][TB],
                                          int c) {
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[a][c], B.h[b][c], acc[a][b], 0, 0, 0);
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[a][c], B.l[b][c], acc[a][b], 0, 0, 0);
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.l[a][c], B.h[b][c], acc[a][b], 0, 0, 0);
}



// The 4 rows i0 .. i0+3 of column j into a by-columns matrix: M[j][i0 .. i0+3] (two 8-byte writes).
__device__ __forceinline__ void put_t4(SplitMat& M, int j, int i0, half4 h, half4 l) {
  *reinterpret_cast<half4*>(&M.hi[j * NH + i0]) = h;
  *reinterpret_cast<half4*>(&M.lo[j * NH + i0]) = l;
}

constexpr int kRestoreExp = 15;  // an entry at or above 2^15 * 2^e triggers a re-store with a fresh exponent
// Longest run of coupled T/X steps before T is formed again as W X: 2^kPairRun times the relative rounding of
// one split-fp16 product (2^-22) must stay well below 1.
constexpr int kPairRun = 11;



template <int ST, int KC>
__device__ __forceinline__ void ns_small_block(int g, const float* __restrict__ We, float* __restrict__ Xout,
                                               float* __restrict__ xs, float* __restrict__ alpha_out,
                                               float* __restrict__ resid, int m, int iters) {
  constexpr int TQ = ST >= 2 ? ST / 2 : 1;  // tiles per side of a quadrant
  constexpr int NQA = ST == 1 ? 1 : 4;      // quadrants with work
  constexpr int CS = TQ;                    // column strips (B operand) per wave
  constexpr bool kBoth = TQ >= 2;           // each wave takes part in both products (else one product per wave)
  constexpr int NTH = 512;
  // sT, sU, sX: T_k, U_k = 2I - T_k and X_k (times 2^-e) by columns, each double-buffered by step parity.
  __shared__ SplitMat sT[2], sU[2], sX[2];
  __shared__ double red[3][4][64];
  __shared__ double red_res[8];
  __shared__ float s_alpha, s_wmax;
  // Bits of the largest |X| entry of the iterate written in step k, in slot k % 3: slot k + 1 is cleared during
  // step k (its last readers finished before the barrier of step k - 1), so the one barrier per step suffices.
  __shared__ unsigned int s_max[3];
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  float* wf = reinterpret_cast<float*>(&sU[1]);  // fp32 W (64 x 65) in a U buffer not used before iteration 0
  // Wave w works on quadrant w & 3 of the products. With 64-wide matrices (two strips per quadrant side) wave half
  // w >> 2 takes one row strip of the quadrant and both of its column strips, in both products; with narrower
  // matrices (one tile per quadrant) half 0 forms T_{k+1} and U_{k+1}, half 1 forms X_{k+1}.
  const int qd = wv & 3, hf = wv >> 2;
  const bool act = qd < NQA;
  const bool doT = act && (kBoth || hf == 0), doX = act && (kBoth || hf == 1);
  const int rs = (qd & 1) * TQ + (kBoth ? hf : 0);  // the wave's row strip
  const int c0 = (qd >> 1) * TQ;                    // its first column strip
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
    double cs = 0.0, rsum = 0.0, mx = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double a = fabs(static_cast<double>(wf[(qtr * 16 + k) * 65 + c]));
      cs += a;
      mx = fmax(mx, a);
      rsum += fabs(static_cast<double>(wf[c * 65 + qtr * 16 + k]));
    }
    red[0][qtr][c] = cs;
    red[1][qtr][c] = rsum;
    red[2][qtr][c] = mx;
  }
  __syncthreads();
  if (wv == 0) {
    double cs = red[0][0][ln] + red[0][1][ln] + red[0][2][ln] + red[0][3][ln];
    double rsum = red[1][0][ln] + red[1][1][ln] + red[1][2][ln] + red[1][3][ln];
    double mx = fmax(fmax(red[2][0][ln], red[2][1][ln]), fmax(red[2][2][ln], red[2][3][ln]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      cs = fmax(cs, __shfl_xor(cs, off));
      rsum = fmax(rsum, __shfl_xor(rsum, off));
      mx = fmax(mx, __shfl_xor(mx, off));
    }
    if (ln == 0) {
      s_alpha = static_cast<float>(1.0 / (cs * rsum));
      s_wmax = static_cast<float>(mx);
    }
  }
  __syncthreads();
  const float alpha = s_alpha;
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;

  // W fragments of this wave's row strip (W is the A operand of every product with W).
  Frags<1, KC> fw;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int i = rs * 16 + (ln & 15);
    const int k0 = c * 32 + 8 * (ln >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h, l;
      split_f16(doT ? wf[i * 65 + k0 + e] : 0.f, h, l);
      fw.h[0][c][e] = h;
      fw.l[0][c][e] = l;
    }
  }
  // Lane placement of the wave's tile b: rows row_i0() .. +3 of column col_j(b).
  auto col_j = [&](int b) { return (c0 + b) * 16 + (ln & 15); };
  auto row_i0 = [&]() { return rs * 16 + 4 * (ln >> 4); };
  // 2 on the diagonal of the m x m block, 0 elsewhere (padding included); whether an entry is inside the block
  auto two_i = [&](int b, int r) { return (row_i0() + r == col_j(b) && col_j(b) < m) ? 2.f : 0.f; };
  auto inside = [&](int b, int r) { return row_i0() + r < m && col_j(b) < m; };
  f32x4 accT[1][CS], accX[1][CS];
#pragma unroll
  for (int b = 0; b < CS; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) accX[0][b][r] = doX ? alpha * wf[col_j(b) * 65 + row_i0() + r] : 0.f;  // X_0
  __syncthreads();  // wf (inside sU[1]) is dead after this point
  if constexpr (ST == 1) {
    for (int q = tid; q < NZ; q += NTH) reinterpret_cast<uint4*>(&sU[1])[q] = zero4;
  }

  // Split stores of the wave's tiles into a by-columns buffer (8-byte writes).
  auto put_cols = [&](SplitMat& M, const f32x4 v[1][CS], float s) {
#pragma unroll
    for (int b = 0; b < CS; ++b) {
      half4 h, l;
      split_scaled4(v[0][b], s, h, l);
      put_t4(M, col_j(b), row_i0(), h, l);
    }
  };
  // put_cols that also returns the largest |v| (before scaling).
  auto put_cols_max = [&](SplitMat& M, const f32x4 v[1][CS], float s) {
    float lm = 0.f;
#pragma unroll
    for (int b = 0; b < CS; ++b) {
      const f32x4 t = v[0][b];
      lm = fmaxf(lm, fmaxf(fmaxf(fabsf(t[0]), fabsf(t[1])), fmaxf(fabsf(t[2]), fabsf(t[3]))));
      half4 h, l;
      split_scaled4(t, s, h, l);
      put_t4(M, col_j(b), row_i0(), h, l);
    }
    return lm;
  };
  // T = s v and U = 2I - s v from the same tiles (padding rows and columns of T are exact zeros, so U is zero
  // there); U alone when T is not needed.
  auto put_tu = [&](SplitMat* Mt, SplitMat& Mu, const f32x4 v[1][CS], float s) {
#pragma unroll
    for (int b = 0; b < CS; ++b) {
      f32x4 t, u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[r] = v[0][b][r] * s;
        u[r] = two_i(b, r) - t[r];
      }
      half4 h, l;
      if (Mt) {
        split4(t, h, l);
        put_t4(*Mt, col_j(b), row_i0(), h, l);
      }
      split4(u, h, l);
      put_t4(Mu, col_j(b), row_i0(), h, l);
    }
  };
  // Iterate k to the saved-iterates buffer, from the wave's tiles.
  auto put_xs = [&](int k, const f32x4 v[1][CS], float s) {
    float* xg = xs + (static_cast<size_t>(g) * (iters + 1) + k) * mm;
#pragma unroll
    for (int b = 0; b < CS; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (inside(b, r)) xg[(row_i0() + r) * m + col_j(b)] = v[0][b][r] * s;
  };
  // W * B over the wave's tiles, W's fragments from registers.
  auto mma_w = [&](const SplitMat& B, f32x4 acc[1][CS]) {
    Frags<CS, KC> fb;
#pragma unroll
    for (int c = 0; c < KC; ++c) load_chunk_b<CS, KC>(B, c0, ln, c, fb);
    zero_acc<1, CS>(acc);
#pragma unroll
    for (int c = 0; c < KC; ++c) mma_chunk<1, CS, KC>(fw, fb, acc, c);
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
  if (doX) {
    put_cols(sX[0], accX, ldexpf(1.f, -e_cur));
    if (xs) put_xs(0, accX, 1.f);
  }
  __syncthreads();

  // Segment start at step k: T_k = W X_k (and U_k) into the buffers of parity k & 1, which no wave reads now.
  auto resync = [&](int k) {
    const int cur = k & 1;
    if (doT) {
      mma_w(sX[cur], accT);
      put_tu(&sT[cur], sU[cur], accT, ldexpf(1.f, e_cur));
    }
    __syncthreads();
  };

  int e_next = e_cur;
  // One pair step; the buffer parity is a template constant so that every LDS address is a fixed offset.
  // last: the step ends a segment, so it produces only X_{k+1} (the next segment forms T afresh).
  auto step = [&](auto parity, auto last, int k) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
    constexpr bool kLast = decltype(last)::value;
    const float unscale = ldexpf(1.f, e_cur);
    const bool wt = doT && !kLast;
    if (wt || doX) {
      // every read of both chunks is issued before the first MFMA, so chunk 0's MFMAs overlap chunk 1's reads
      Frags<CS, KC> fu;
      Frags<1, KC> ft, fx;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        load_chunk_b<CS, KC>(sU[cur], c0, ln, c, fu);
        if (wt) load_chunk_a<1, KC>(sT[cur], rs, ln, c, ft);
        if (doX) load_chunk_a<1, KC>(sX[cur], rs, ln, c, fx);
      }
      if (wt) {
        zero_acc<1, CS>(accT);
#pragma unroll
        for (int c = 0; c < KC; ++c) mma_chunk<1, CS, KC>(ft, fu, accT, c);  // T_{k+1} = T_k U_k
      }
      if (doX) {
        zero_acc<1, CS>(accX);
#pragma unroll
        for (int c = 0; c < KC; ++c) mma_chunk<1, CS, KC>(fx, fu, accX, c);  // X_{k+1} = X_k U_k, times 2^-e_cur
      }
      if (wt) put_tu(&sT[nxt], sU[nxt], accT, 1.f);
      if (doX) {
        float lmax = put_cols_max(sX[nxt], accX, ldexpf(1.f, e_cur - e_next));
        if (xs) put_xs(k + 1, accX, unscale);
        lmax = wave_max_nonneg(lmax) * unscale;
        if (ln == 0) atomicMax(&s_max[k % 3], __float_as_uint(lmax));
      }
    }
    if (tid == 0) s_max[(k + 1) % 3] = 0u;
    __syncthreads();
    const float mx = __uint_as_float(s_max[k % 3]);
    if (mx >= ldexpf(1.f, e_next + kRestoreExp) || !(mx < 3.0e38f)) {
      // Rare: the iterate grew past the headroom of its exponent (or is not finite); store it again.
      const int e_new = store_exp(fminf(mx, 3.0e38f));
      if (doX) put_cols(sX[nxt], accX, ldexpf(1.f, e_cur - e_new));
      e_next = e_new;
      __syncthreads();
    }
    e_cur = e_next;
    e_next = store_exp(mx);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<bool, false>;
  using End = std::integral_constant<bool, true>;
  for (int k = 0; k + 1 < iters;) {
    resync(k);
    const int end = min(k + kPairRun, iters - 1);  // pair steps k .. end - 1; step K - 1 is the exact one
    for (; k < end; ++k) {
      const bool lst = k + 1 == end;
      if (k & 1) {
        if (lst) step(P1{}, End{}, k); else step(P1{}, Mid{}, k);
      } else {
        if (lst) step(P0{}, End{}, k); else step(P0{}, Mid{}, k);
      }
    }
  }

  // Final exact step (iters >= 1): X_K = X_{K-1} (2I - W X_{K-1}), with X_{K-1} in sX[fin]. The U buffer of that
  // parity was neither written nor read by the last pair step.
  const int fin = (iters >= 1) ? ((iters - 1) & 1) : 0;
  float out_unscale = 1.f;
  if (iters >= 1) {
    const float unscale = ldexpf(1.f, e_cur);
    if (doT) {
      mma_w(sX[fin], accT);
      put_tu(nullptr, sU[fin], accT, unscale);
    }
    __syncthreads();
    if (doX) {
      Frags<CS, KC> fu;
      Frags<1, KC> fx;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        load_chunk_b<CS, KC>(sU[fin], c0, ln, c, fu);
        load_chunk_a<1, KC>(sX[fin], rs, ln, c, fx);
      }
      zero_acc<1, CS>(accX);
#pragma unroll
      for (int c = 0; c < KC; ++c) mma_chunk<1, CS, KC>(fx, fu, accX, c);
    }
    out_unscale = unscale;
  }  // with no step accX still holds X_0
  if (doX) {
    if (xs && iters >= 1) put_xs(iters, accX, out_unscale);
    float* xo = Xout + g * mm;
#pragma unroll
    for (int b = 0; b < CS; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (inside(b, r)) xo[(row_i0() + r) * m + col_j(b)] = accX[0][b][r] * out_unscale;
  }

  if (resid) {
    // ||W X_K - I||_F with the same split products: X_K goes through LDS once more.
    __syncthreads();  // every read of the buffers below is done
    const int rb = fin ^ 1;
    // accX * out_unscale is X_K; store it with the exponent of the last iterate so the fp16 halves stay in range
    const float st_scale = (iters >= 1) ? 1.f : ldexpf(1.f, -e_cur);
    const float ru = out_unscale / st_scale;
    if (doX) put_cols(sX[rb], accX, st_scale);
    __syncthreads();
    double ss = 0.0;
    if (doT) {
      mma_w(sX[rb], accT);
#pragma unroll
      for (int b = 0; b < CS; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inside(b, r)) {
            const double e2 = static_cast<double>(accT[0][b][r] * ru) - (row_i0() + r == col_j(b) ? 1.0 : 0.0);
            ss += e2 * e2;
          }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (ln == 0) red_res[wv] = ss;
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int q = 0; q < 8; ++q) tot += red_res[q];
      resid[g] = static_cast<float>(sqrt(tot));
    }
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

// One S tile by one block of kSideWaves waves (the solver's block size). Wave w sums a contiguous range of 16-token
// groups on fp32 MFMA (A = C_K, landmark-major, B = V): in group q, lane (i, k) feeds landmark i and channel i of
// the tile with tokens 16q + 4k + u at k-step u, loaded from global memory straight into the MFMA operand layout.
// The wave tiles are then summed in LDS in wave order, so the result does not depend on timing.
constexpr int kSideWaves = 8;

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
  const int groups = (N + 15) / 16, gpw = (groups + kSideWaves - 1) / kSideWaves;
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
  if (tid < 256) {  // one thread per entry of the 16 x 16 tile
    const int row = tid >> 4, col = tid & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kSideWaves; ++w) sum += sRed[w * 256 + tid];
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
  __shared__ float sRed[kSideWaves * 256];
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
// tiles of 256-thread blocks (4 waves of 16 x 16), each staging its 32-row A strip and 32-column B strip whole
// in LDS (one round of global-load latency per launch) and running split-fp16 MFMAs as the small kernel does.
// The iterates live in global memory in the layout the MFMA result has: split fp16 (hi, lo), by columns,
// zero-padded to mp = 32 ceil(m / 32) in both dimensions, so that staging is unguarded 16-byte copies, the B
// strip is plain LDS reads and the A strip is read with the transposing LDS read. X, whose entries start near
// alpha and end near those of W^-1, carries one power-of-two exponent per 32 x 32 tile, chosen from the tile's
// own largest entry when it is written; a product folds the exponents of its A and B tiles in per 32-wide K
// chunk. W is read as fp32 and split while it is staged.
// The steps follow the small kernel: segments of at most kPairRun steps start from T_k = W X_k, then one launch
// per step computes T_{k+1} = T_k U_k and X_{k+1} = X_k U_k (U_k = 2I - T_k stored beside T_k), and the last
// step is the exact one, X_K = X_{K-1} (2I - W X_{K-1}), in two launches. The first product launch also forms
// alpha, X_0 = alpha W^T and T_0 = W X_0 = alpha W W^T.
// =====================================================================================================
// Partial sums for alpha over (slice, kNsRows-row chunk) blocks: per-chunk column sums and the largest row sum of
// the chunk, combined later in a fixed order (deterministic). part: G * nchunk * m doubles, rmx: G * nchunk.
constexpr int kNsRows = 8;  // rows per chunk: m / 8 chunks spread a slice over blocks

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

constexpr int LF_NS_KMAX = 256;            // largest m of the batched path (the library's m limit)
constexpr int kTile = 32;                  // output tile side and K chunk
constexpr int kLdA = kTile + 8;            // A strip in LDS by columns: 32 rows + 8 (80-byte columns)
constexpr int kLdK = LF_NS_KMAX + 8;       // K-contiguous rows of the B strip and of W: 256 + 8 (528 bytes)

// One m x m matrix per slice in split fp16 by columns, [G][mp][mp] halves in each of hi and lo.
struct SplitG {
  _Float16* hi;
  _Float16* lo;
};

// What a launch writes from a product P (times `scale`) of its tiles; every pointer may be null.
struct NsOut {
  SplitG t;          // P
  SplitG u;          // 2I - P
  SplitG x;          // P 2^-e with e per tile, the tile's e in x_exp[g][ti][tj]
  int* x_exp;
  float* f32;        // P as fp32 [m][m] per slice, slice stride f32_stride (minus I when minus_eye)
  size_t f32_stride;
  float* f32b;       // a second fp32 copy (a saved iterate)
  size_t f32b_stride;
  int minus_eye;
};

// A product job: P = A B for one slice. A is W (fp32, split while staged) or a split matrix read by transposing
// reads; B is W^T (W's rows as its columns) or a split matrix; a_exp / b_exp hold per-tile exponents (null: 0).
struct NsJob {
  SplitG a;
  const int* a_exp;
  SplitG b;
  const int* b_exp;
  NsOut out;
};

// The first product launch's extra work: alpha from the k_ns_sums partials and X_0 = alpha W^T, tile by tile.
struct NsInit {
  const double* part;  // null: not the first launch
  const double* rmx;
  int nch;
  float* alpha_out;    // [G] or null
  SplitG x0;
  int* x0_exp;
  float* f32;          // X_0 as fp32 (when it is the result, no steps), or null
  float* f32b;         // the saved iterate X_0, or null
  size_t f32b_stride;
};

__device__ __forceinline__ float block4_max_nonneg(float v, float* s_red) {
  v = wave_max_nonneg(v);
  __syncthreads();  // the previous use of s_red is over
  if (lane_id() == 0) s_red[wave_id()] = v;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// W's rows r0 .. r0+31, all 32 NT columns (zero beyond m), split into LDS as [row][k] halves (hi at dh, lo at dl).
// The 4 NT values of a thread are all loaded (clamped addresses, zeroed outside W) before the first store.
template <int NT>
__device__ __forceinline__ void stage_w_rows(const float* __restrict__ wg, int r0, _Float16* dh, _Float16* dl, int m) {
  constexpr int mp = NT * kTile, NV = kTile * mp / 256;
  const int tid = threadIdx.x;
  if ((m & 3) == 0) {  // rows start 16-byte aligned: four values per load, 8-byte split stores
    constexpr int NQ = NV / 4, mq = mp / 4;
    float4 v4[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int idx = tid + 256 * q, rr = idx / mq, k = 4 * (idx % mq), r = r0 + rr;
      const bool ok = r < m && k < m;
      const float4 x = *reinterpret_cast<const float4*>(wg + (ok ? static_cast<size_t>(r) * m + k : 0));
      v4[q] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int idx = tid + 256 * q, rr = idx / mq, k = 4 * (idx % mq);
      half4 h, l;
      split4(f32x4{v4[q].x, v4[q].y, v4[q].z, v4[q].w}, h, l);
      *reinterpret_cast<half4*>(&dh[rr * kLdK + k]) = h;
      *reinterpret_cast<half4*>(&dl[rr * kLdK + k]) = l;
    }
    return;
  }
  float v[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int idx = tid + 256 * q, rr = idx / mp, k = idx % mp, r = r0 + rr;
    const bool ok = r < m && k < m;
    const float x = wg[ok ? static_cast<size_t>(r) * m + k : 0];
    v[q] = ok ? x : 0.f;
  }
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int idx = tid + 256 * q, rr = idx / mp, k = idx % mp;
    _Float16 h, l;
    split_f16(v[q], h, l);
    dh[rr * kLdK + k] = h;
    dl[rr * kLdK + k] = l;
  }
}

constexpr int kA = (LF_NS_KMAX * kLdA > kTile * kLdK) ? LF_NS_KMAX * kLdA : kTile * kLdK;  // A strip halves

struct NsTileLds {
  alignas(16) _Float16 a[2 * kA];  // hi then lo
  alignas(16) _Float16 b[2 * kTile * kLdK];
  float red[4];
  double cmax[4], rmax[4];
  float alpha;
};

// One block's work on tile (ti, tj) of slice g for job J; NT = mp / 32 tiles per side.
template <bool AW, bool BW, int NT>
__device__ __forceinline__ void ns_tile_body(const NsJob& J, const NsInit& init, const float* __restrict__ We, int m,
                                             int g, NsTileLds& L) {
  constexpr int mp = NT * kTile, nt = NT;
  _Float16* sA = L.a;
  _Float16* sB = L.b;
  float* s_red = L.red;
  double* s_cmax = L.cmax;
  double* s_rmax = L.rmax;
  const int tj = blockIdx.x, ti = blockIdx.y;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mpp = static_cast<size_t>(mp) * mp, mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;

  // 1. Stage both strips: every global load is issued before the first LDS store.
  // Each strip is 8 mp 16-byte pieces, NT per thread; a thread's loads are all issued before its first store.
  if constexpr (AW) {
    stage_w_rows<NT>(wg, ti * kTile, sA, sA + kA, m);
  } else {
    uint4 buf[NT];  // A strip: rows ti*32 .. +31 of every column k, 64 bytes per (column, half)
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int idx = tid + 256 * q, half = idx / (4 * mp), rem = idx % (4 * mp);
      const int k = rem >> 2, p8 = (rem & 3) * 8;
      const _Float16* src = (half ? J.a.lo : J.a.hi) + g * mpp + static_cast<size_t>(k) * mp + ti * kTile + p8;
      buf[q] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int idx = tid + 256 * q, half = idx / (4 * mp), rem = idx % (4 * mp);
      const int k = rem >> 2, p8 = (rem & 3) * 8;
      *reinterpret_cast<uint4*>(&sA[half * kA + k * kLdA + p8]) = buf[q];
    }
  }
  if constexpr (BW) {
    stage_w_rows<NT>(wg, tj * kTile, sB, sB + kTile * kLdK, m);
  } else {
    constexpr int pc = mp / 8;  // 16-byte pieces per column
    uint4 buf[NT];              // B strip: columns tj*32 .. +31, all mp rows
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int idx = tid + 256 * q, half = idx / (kTile * pc), rem = idx % (kTile * pc);
      const int jj = rem / pc, p8 = (rem % pc) * 8;
      const _Float16* src = (half ? J.b.lo : J.b.hi) + g * mpp + static_cast<size_t>(tj * kTile + jj) * mp + p8;
      buf[q] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int idx = tid + 256 * q, half = idx / (kTile * pc), rem = idx % (kTile * pc);
      const int jj = rem / pc, p8 = (rem % pc) * 8;
      *reinterpret_cast<uint4*>(&sB[half * kTile * kLdK + jj * kLdK + p8]) = buf[q];
    }
  }
  // alpha = 1 / (max column sum * max row sum) of |W| from the chunk partials, in a fixed order.
  float scale = 1.f;
  if (init.part) {
    // thread j sums column j's chunk partials (m <= 256 columns, at most 32 chunks), every load in flight first
    constexpr int kMaxCh = LF_NS_KMAX / kNsRows;
    double pv[kMaxCh];
    const int j = tid < m ? tid : 0;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c)
      pv[c] = init.part[(static_cast<size_t>(g) * init.nch + (c < init.nch ? c : 0)) * m + j];
    double cs = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c)
      if (c < init.nch) cs += pv[c];
    double cmax = tid < m ? cs : 0.0;
    // chunk c's largest row sum comes from thread c (at most 32 chunks)
    double rmax = tid < init.nch ? init.rmx[static_cast<size_t>(g) * init.nch + tid] : 0.0;
    for (int off = 32; off > 0; off >>= 1) {
      cmax = fmax(cmax, __shfl_xor(cmax, off));
      rmax = fmax(rmax, __shfl_xor(rmax, off));
    }
    if (ln == 0) {
      s_cmax[wv] = cmax;
      s_rmax[wv] = rmax;
    }
    __syncthreads();
    if (tid == 0) {
      const double cm = fmax(fmax(s_cmax[0], s_cmax[1]), fmax(s_cmax[2], s_cmax[3]));
      const double rm = fmax(fmax(s_rmax[0], s_rmax[1]), fmax(s_rmax[2], s_rmax[3]));
      L.alpha = static_cast<float>(1.0 / (cm * rm));
      if (ti == 0 && tj == 0 && init.alpha_out) init.alpha_out[g] = L.alpha;
    }
  }
  __syncthreads();
  if (init.part) scale = L.alpha;

  // 2. The wave's 16 x 16 sub-tile (wi, wj), chunk by chunk: three split-fp16 MFMAs per chunk into a fresh
  //    accumulator, folded into the sum with the chunk's power of two (the exponents of A's row of tiles and B's
  //    column of tiles, read before the first chunk).
  const int wi = wv & 1, wj = wv >> 1;
  int ech[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int ea = J.a_exp ? J.a_exp[(static_cast<size_t>(g) * nt + ti) * nt + c] : 0;
    const int eb = J.b_exp ? J.b_exp[(static_cast<size_t>(g) * nt + c) * nt + tj] : 0;
    ech[c] = ea + eb;
  }
  const int gq = ln >> 4, t = ln & 15;
  half8 ah[NT], al[NT], bh[NT], bl[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    if constexpr (AW) {
      const int o = (wi * 16 + t) * kLdK + c * kTile + 8 * gq;
      ah[c] = *reinterpret_cast<const half8*>(&sA[o]);
      al[c] = *reinterpret_cast<const half8*>(&sA[kA + o]);
    } else {
      const int k0 = c * kTile + 8 * gq + (t >> 2), i = wi * 16 + 4 * (t & 3);
      const half4 h0 = __builtin_bit_cast(half4, lds_read_tr(&sA[k0 * kLdA + i]));
      const half4 h1 = __builtin_bit_cast(half4, lds_read_tr(&sA[(k0 + 4) * kLdA + i]));
      const half4 l0 = __builtin_bit_cast(half4, lds_read_tr(&sA[kA + k0 * kLdA + i]));
      const half4 l1 = __builtin_bit_cast(half4, lds_read_tr(&sA[kA + (k0 + 4) * kLdA + i]));
      ah[c] = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      al[c] = half8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
    }
    const int o = (wj * 16 + t) * kLdK + c * kTile + 8 * gq;
    bh[c] = *reinterpret_cast<const half8*>(&sB[o]);
    bl[c] = *reinterpret_cast<const half8*>(&sB[kTile * kLdK + o]);
  }
  f32x4 p[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) p[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NT; ++c) p[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[c], bh[c], p[c], 0, 0, 0);
#pragma unroll
  for (int c = 0; c < NT; ++c) p[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[c], bl[c], p[c], 0, 0, 0);
#pragma unroll
  for (int c = 0; c < NT; ++c) p[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[c], bh[c], p[c], 0, 0, 0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const float f = ldexpf(1.f, ech[c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(p[c][r], f, acc[r]);
  }

  // 3. Outputs. The lane holds rows i0 .. i0+3 of column j.
  const int i0 = ti * kTile + wi * 16 + 4 * gq, j = tj * kTile + wj * 16 + t;
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = acc[r] * scale;
  const size_t so = g * mpp + static_cast<size_t>(j) * mp + i0;  // split-store offset of the lane's 4 rows
  const NsOut& O = J.out;
  if (O.t.hi) {
    half4 h, l;
    split4(v, h, l);
    *reinterpret_cast<half4*>(&O.t.hi[so]) = h;
    *reinterpret_cast<half4*>(&O.t.lo[so]) = l;
  }
  if (O.u.hi) {
    f32x4 u;
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = ((i0 + r == j && j < m) ? 2.f : 0.f) - v[r];
    half4 h, l;
    split4(u, h, l);
    *reinterpret_cast<half4*>(&O.u.hi[so]) = h;
    *reinterpret_cast<half4*>(&O.u.lo[so]) = l;
  }
  if (O.x.hi) {  // uniform over the block
    const float mx = block4_max_nonneg(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                                       s_red);
    const int e = store_exp(mx);
    half4 h, l;
    split_scaled4(v, ldexpf(1.f, -e), h, l);
    *reinterpret_cast<half4*>(&O.x.hi[so]) = h;
    *reinterpret_cast<half4*>(&O.x.lo[so]) = l;
    if (tid == 0) O.x_exp[(static_cast<size_t>(g) * nt + ti) * nt + tj] = e;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + r;
    if (i < m && j < m) {
      const float o = v[r] - ((O.minus_eye && i == j) ? 1.f : 0.f);
      if (O.f32) O.f32[g * O.f32_stride + static_cast<size_t>(i) * m + j] = o;
      if (O.f32b) O.f32b[g * O.f32b_stride + static_cast<size_t>(i) * m + j] = o;
    }
  }
  if (init.part) {
    // X_0 = alpha W^T over this tile: X_0[i][j] = alpha W[j][i] (rows i0 .. i0+3 of column j, contiguous in W).
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (i0 + r < m && j < m) ? scale * wg[static_cast<size_t>(j) * m + i0 + r] : 0.f;
    const float mx = block4_max_nonneg(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))),
                                       s_red);
    const int e = store_exp(mx);
    half4 h, l;
    split_scaled4(x, ldexpf(1.f, -e), h, l);
    *reinterpret_cast<half4*>(&init.x0.hi[so]) = h;
    *reinterpret_cast<half4*>(&init.x0.lo[so]) = l;
    if (tid == 0) init.x0_exp[(static_cast<size_t>(g) * nt + ti) * nt + tj] = e;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
      if (i < m && j < m) {
        if (init.f32) init.f32[g * mm + static_cast<size_t>(i) * m + j] = x[r];
        if (init.f32b) init.f32b[g * init.f32b_stride + static_cast<size_t>(i) * m + j] = x[r];
      }
    }
  }
}

// Block (tj, ti, z): tile (ti, tj) of slice z / njobs for job z % njobs (j0 or j1).
template <bool AW, bool BW, int NT>
__global__ __launch_bounds__(256) void k_ns_tile(NsJob j0, NsJob j1, int njobs, NsInit init,
                                                 const float* __restrict__ We, int m) {
  __shared__ NsTileLds lds;
  const int g = blockIdx.z / njobs;
  if (blockIdx.z % njobs == 0)
    ns_tile_body<AW, BW, NT>(j0, init, We, m, g, lds);
  else
    ns_tile_body<AW, BW, NT>(j1, init, We, m, g, lds);
}

// k_ns_tile for the tile count of m: 3 .. 8 (65 <= m <= 256).
template <bool AW, bool BW>
static void ns_tile_launch(int nt, dim3 grid, hipStream_t st, const NsJob& j0, const NsJob& j1, int njobs,
                           const NsInit& init, const float* We, int m) {
#define LF_NS_TILE(NT_)                                                                                        \
  hipLaunchKernelGGL((k_ns_tile<AW, BW, NT_>), grid, dim3(256), 0, st, j0, j1, njobs, init, We, m)
  switch (nt) {
    case 3: LF_NS_TILE(3); break;
    case 4: LF_NS_TILE(4); break;
    case 5: LF_NS_TILE(5); break;
    case 6: LF_NS_TILE(6); break;
    case 7: LF_NS_TILE(7); break;
    default: LF_NS_TILE(8); break;
  }
#undef LF_NS_TILE
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

// Scratch of the batched path, in floats: six split matrices (T, U and X by parity), the per-tile exponents of
// the two X buffers and the alpha partials.
static inline int ns_mp(int m) { return (m + kTile - 1) / kTile * kTile; }

size_t ns_tmp_floats(const Shape& s) {
  if (s.m <= 64) return 0;
  const size_t G = s.G, mp = ns_mp(s.m), nt = mp / kTile, nch = (s.m + kNsRows - 1) / kNsRows;
  return 6 * G * mp * mp + 2 * G * nt * nt + 2 * G * nch * (s.m + 1) + 64;
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
  const int G = s.G, mp = ns_mp(m), nt = mp / kTile, nch = (m + kNsRows - 1) / kNsRows;
  const size_t mm = static_cast<size_t>(m) * m, Gmpp = static_cast<size_t>(G) * mp * mp;
  // carve: 6 split matrices (Gmpp floats each = 2 Gmpp halves), then the exponents, then the alpha partials
  auto split_at = [&](int i) {
    _Float16* h = reinterpret_cast<_Float16*>(tmp + static_cast<size_t>(i) * Gmpp);
    return SplitG{h, h + Gmpp};
  };
  const SplitG Tb[2] = {split_at(0), split_at(1)}, Ub[2] = {split_at(2), split_at(3)},
               Xb[2] = {split_at(4), split_at(5)};
  int* ex = reinterpret_cast<int*>(tmp + 6 * Gmpp);
  int* Xe[2] = {ex, ex + static_cast<size_t>(G) * nt * nt};
  double* part = reinterpret_cast<double*>(tmp + 6 * Gmpp + 2 * static_cast<size_t>(G) * nt * nt + 2);
  part = reinterpret_cast<double*>((reinterpret_cast<uintptr_t>(part) + 7) & ~static_cast<uintptr_t>(7));
  double* rmx = part + static_cast<size_t>(G) * nch * m;
  const size_t xs_stride = static_cast<size_t>(K + 1) * mm;
  auto slot = [&](int k) { return xs ? xs + static_cast<size_t>(k) * mm : nullptr; };
  const dim3 blk(256);
  const NsInit noinit{};
  const NsJob none{};

  hipLaunchKernelGGL(k_ns_sums, dim3(G, nch), blk, 0, st, We, part, rmx, m);
  // T_0 = W X_0 = alpha W W^T, U_0, and X_0 = alpha W^T (the result itself when there is no step)
  {
    NsJob j{};
    j.out.t = Tb[0];
    j.out.u = Ub[0];
    NsInit in{part, rmx, nch, alpha, Xb[0], Xe[0], K == 0 ? X : nullptr, slot(0), xs_stride};
    ns_tile_launch<true, true>(nt, dim3(nt, nt, G), st, j, none, 1, in, We, m);
  }
  int tc = 0, xc = 0;  // buffers holding T_k, U_k and X_k
  for (int k = 0; k + 1 < K;) {
    if (k > 0) {
      // segment start: T_k = W X_k, U_k
      NsJob j{};
      j.b = Xb[xc];
      j.b_exp = Xe[xc];
      j.out.t = Tb[tc];
      j.out.u = Ub[tc];
      ns_tile_launch<true, false>(nt, dim3(nt, nt, G), st, j, none, 1, noinit, We, m);
    }
    const int end = std::min(k + kPairRun, K - 1);
    for (; k < end; ++k) {
      const bool last = k + 1 == end;
      // X_{k+1} = X_k U_k and (unless the segment ends) T_{k+1} = T_k U_k, U_{k+1}
      NsJob jx{};
      jx.a = Xb[xc];
      jx.a_exp = Xe[xc];
      jx.b = Ub[tc];
      jx.out.x = Xb[xc ^ 1];
      jx.out.x_exp = Xe[xc ^ 1];
      jx.out.f32b = slot(k + 1);
      jx.out.f32b_stride = xs_stride;
      NsJob jt{};
      jt.a = Tb[tc];
      jt.b = Ub[tc];
      jt.out.t = Tb[tc ^ 1];
      jt.out.u = Ub[tc ^ 1];
      const int nj = last ? 1 : 2;
      ns_tile_launch<false, false>(nt, dim3(nt, nt, nj * G), st, jx, jt, nj, noinit, We, m);
      tc ^= 1;
      xc ^= 1;
    }
  }
  if (K >= 1) {
    // exact step: U' = 2I - W X_{K-1} (into the U buffer the last pair step neither read nor wrote), then
    // X_K = X_{K-1} U'
    NsJob ju{};
    ju.b = Xb[xc];
    ju.b_exp = Xe[xc];
    ju.out.u = Ub[tc];
    ns_tile_launch<true, false>(nt, dim3(nt, nt, G), st, ju, none, 1, noinit, We, m);
    NsJob jx{};
    jx.a = Xb[xc];
    jx.a_exp = Xe[xc];
    jx.b = Ub[tc];
    jx.out.f32 = X;
    jx.out.f32_stride = mm;
    jx.out.f32b = slot(K);
    jx.out.f32b_stride = xs_stride;
    if (resid) {  // the residual needs X_K as a split B operand
      jx.out.x = Xb[xc ^ 1];
      jx.out.x_exp = Xe[xc ^ 1];
    }
    ns_tile_launch<false, false>(nt, dim3(nt, nt, G), st, jx, none, 1, noinit, We, m);
    xc ^= 1;
  }
  if (resid) {
    // E = W X_K - I in fp32 (into the T buffers, free now), then its Frobenius norm per slice
    float* E = tmp;
    NsJob jr{};
    jr.b = Xb[xc];  // X_K (X_0 in buffer 0 when there is no step)
    jr.b_exp = Xe[xc];
    jr.out.f32 = E;
    jr.out.f32_stride = mm;
    jr.out.minus_eye = 1;
    ns_tile_launch<true, false>(nt, dim3(nt, nt, G), st, jr, none, 1, noinit, We, m);
    hipLaunchKernelGGL(k_frob, dim3(G), dim3(256), 0, st, E, resid, m);
  }
  return hipGetLastError();
}

}  // namespace lf
