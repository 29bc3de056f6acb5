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
#include "lf_laplace.h"
#include "lf_split.h"

namespace lf {

// =====================================================================================================
// m <= 64: one 256-thread block (four waves, one per SIMD) per slice runs every iteration, with both carried
// matrices in registers.
//
// Products run on the fp16 MFMA (v_mfma_f32_16x16x32_f16, 16x the fp32 MFMA rate on gfx950) with every fp32
// operand split as x = hi + lo (two fp16 values, about 22 significant bits) and
//   A B ~= A_hi B_hi + (A_hi B_lo + A_lo B_hi),
// accumulated in fp32. Three fp16 MFMAs cost less than a fifth of one fp32 MFMA product, and the result tracks an
// fp32 product to a few units of 1e-7.
//
// The coupled recurrence (below) forms T_{k+1} = T_k U_k and X_{k+1} = X_k U_k with U_k = 2I - T_k. The kernel
// carries the transposes A_k = X_k^T and B_k = T_k^T, zero-padded to 16 ST x 16 ST, and computes
//   A_{k+1} = U_k^T A_k = 2 A_k - B_k A_k,   B_{k+1} = U_k^T B_k = 2 B_k - B_k B_k,
// the same sums, so that the carried matrices are the B operands: wave w holds column strip w (16 columns) of A
// and of B in the MFMA result layout (lane (g, t): rows 4g .. 4g+3 of column t of each 16-row tile), and one
// 32-deep K chunk of its next product takes, for lane (g, t), those four rows of two 16-row tiles (slots 0-3 from
// the first tile, 4-7 from the second). The A operand B_k is read in that same K order, so the carried strips
// feed the MFMA where they stand: no lane exchanges and no LDS round trip. Per step a wave writes its strip of
// B_{k+1} (4 KB) and reads all of B_k (16 KB); every product operand through LDS would be four times the reads
// and three times the writes. Each matrix is read as itself, never as its transpose: X_k is symmetric only in
// exact arithmetic, and feeding X_k^T where the recurrence has X_k doubles the antisymmetric part of the rounding
// error every step.
//
// B is stored by columns (the rows of column j contiguous, 160-byte pitch) and its rows are read with gfx950's
// transposing LDS read, ds_read_b64_tr_b16: within each group of 16 lanes, result lane j, element s comes from
// element j % 4 of the 8 bytes lane 4 s + j / 4 addressed, so lanes that address columns k0 + (lane % 16) / 4,
// rows 4 (lane % 4) .. + 3 of a tile receive their row at K = k0 .. k0 + 3. In columns 8 .. 15 of every 16 the
// 4-row quads are swapped in pairs (quad q at q ^ 2): with the 160-byte pitch both the tile writes (16 columns x
// 8 bytes per half-wave) and these reads (8 columns x 32 bytes) then touch every LDS bank once.
//
// A carries a power-of-two scale 2^-e per wave (its column strip alone enters its products): entries sit near
// 2^12, far from fp16's subnormals and its 65504 limit, and the strip is scaled again when its largest entry
// leaves [2^8, 2^14). W needs no scale (entries at most 1 + eps) and neither do T and U (the eigenvalues of W X
// stay in (0, 1]).
// =====================================================================================================

constexpr int kRegPitch = 80;              // fp16 elements per stored column: 64 rows + 16 (160 bytes)
constexpr int kRegPlane = 64 * kRegPitch;  // fp16 elements per plane (hi or lo) of a stored matrix

struct alignas(16) RegSplit {
  _Float16 hi[kRegPlane];
  _Float16 lo[kRegPlane];
};

// Longest run of coupled T/X steps before T is formed again as W X: 2^kPairRun times the relative rounding of
// one split-fp16 product (2^-22) must stay well below 1.
constexpr int kPairRun = 11;

// Split of two result tiles into one B operand chunk: slots 0-3 from tile a, 4-7 from tile b. lo = fma(v, one,
// -hi) is exact (hi is v rounded to fp16), and with one not a compile-time constant it stays a single
// mixed-precision fma.
__device__ __forceinline__ void split_chunk(f32x4 a, f32x4 b, float one, half8& h, half8& l) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const _Float16 ha = static_cast<_Float16>(a[e]), hb = static_cast<_Float16>(b[e]);
    h[e] = ha;
    h[4 + e] = hb;
    l[e] = static_cast<_Float16>(__builtin_fmaf(a[e], one, -static_cast<float>(ha)));
    l[4 + e] = static_cast<_Float16>(__builtin_fmaf(b[e], one, -static_cast<float>(hb)));
  }
}

// acc + A B over one 32-deep chunk, A and B split: three fp16 products into one fp32 accumulator.
__device__ __forceinline__ f32x4 mma_split3(half8 ah, half8 al, half8 bh, half8 bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc, 0, 0, 0);
}

// A operand chunk c of row tile p of a stored matrix: K tiles 2c and 2c + 1 in B-chunk order. lane_r is the
// lane's offset for row tile 0, K tile 0 (see ns_small_block); a 16-row step is 16 elements, a 16-column step
// 16 * kRegPitch.
template <int ST>
__device__ __forceinline__ void load_rows(const RegSplit& M, int lane_r, int c, int p, half8& h, half8& l) {
  const int oa = lane_r + 16 * p + 2 * c * 16 * kRegPitch;
  const half4 h0 = __builtin_bit_cast(half4, lds_read_tr(&M.hi[oa]));
  const half4 l0 = __builtin_bit_cast(half4, lds_read_tr(&M.lo[oa]));
  half4 h1 = {0, 0, 0, 0}, l1 = {0, 0, 0, 0};
  if constexpr (ST >= 2) {
    h1 = __builtin_bit_cast(half4, lds_read_tr(&M.hi[oa + 16 * kRegPitch]));
    l1 = __builtin_bit_cast(half4, lds_read_tr(&M.lo[oa + 16 * kRegPitch]));
  }
  h = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  l = half8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
}

// Barrier that orders LDS accesses only: global stores (the saved iterates) stay in flight across it, since no
// other wave of the block reads them.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS of one solver block, in bytes: two split matrices, -B_k by step parity (at a segment start the idle one
// carries -A_k), with W, W^T and the setup reductions inside them while the block starts up.
constexpr int kNsSmallLds = 2 * static_cast<int>(sizeof(RegSplit));

template <int ST>
__device__ __forceinline__ void ns_small_block(char* __restrict__ lds, int g, const float* __restrict__ We,
                                               float* __restrict__ Xout, float* __restrict__ xs,
                                               float* __restrict__ alpha_out, float* __restrict__ resid, int m,
                                               int iters) {
  constexpr int NT = ST;            // 16-row tiles per strip
  constexpr int KC = (ST + 1) / 2;  // 32-deep K chunks
  constexpr int NTH = 256;
  RegSplit* sU = reinterpret_cast<RegSplit*>(lds);
  __shared__ float s_alpha, s_wmax;
  __shared__ int s_ex[4];
  __shared__ double s_res[4];
  const int tid = threadIdx.x, ln = lane_id();
  const int cs = __builtin_amdgcn_readfirstlane(wave_id());  // the wave's column strip
  const bool act = cs < ST;
  const size_t mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;
  const float one = m > 0 ? 1.f : 0.f;  // 1 for every call that reaches here, unknown to the compiler
  const int gq = ln >> 4, t = ln & 15;
  const int col = cs * 16 + t;  // the lane's column of the strip
  // lane offsets: transposing reads (row tile 0, K tile 0) and tile writes (row tile 0) of a stored matrix
  const int lane_r = (4 * gq + (t >> 2)) * kRegPitch + 4 * ((t & 3) ^ ((gq >> 1) << 1));
  const int lane_w = col * kRegPitch + 4 * (gq ^ (((t >> 3) & 1) << 1));

  // W and W^T in fp32, zero-padded to 64 x 64, rows of kWp floats (four consecutive entries are one 16-byte
  // read), inside the U buffers, which no step uses yet. Every load of a thread is issued before any is used.
  constexpr int kWp = 68;
  float* wrow = reinterpret_cast<float*>(lds);  // W[i][j] at i * kWp + j
  float* wcol = wrow + 64 * kWp;                // W[i][j] at j * kWp + i
  double* red = reinterpret_cast<double*>(wcol + 64 * kWp);  // [3][4][64]: setup reductions
  static_assert(2 * 64 * kWp * 4 + 3 * 4 * 64 * 8 <= kNsSmallLds, "setup area exceeds the solver's LDS");
  {
    const int mc = m - 1;
    float v[4096 / NTH];
#pragma unroll
    for (int q = 0; q < 4096 / NTH; ++q) {
      const int idx = tid + NTH * q, i = idx >> 6, j = idx & 63;
      v[q] = wg[min(i, mc) * m + min(j, mc)];
    }
#pragma unroll
    for (int q = 0; q < 4096 / NTH; ++q) {
      const int idx = tid + NTH * q, i = idx >> 6, j = idx & 63;
      const float w = (i < m && j < m) ? v[q] : 0.f;
      wrow[i * kWp + j] = w;
      wcol[j * kWp + i] = w;
    }
  }
  __syncthreads();

  // alpha = 1 / (max_j sum_i |W_ij| * max_i sum_j |W_ij|) in float64: thread (c, quarter) sums 16 entries of
  // column c and of row c, the quarters are combined, then wave 0 takes the maxima (and max |W_ij|).
  {
    const int c = tid & 63, qtr = tid >> 6;
    double csum = 0.0, rsum = 0.0, mx = 0.0;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const float4 a = *reinterpret_cast<const float4*>(&wcol[c * kWp + qtr * 16 + 4 * k4]);
      const float4 r = *reinterpret_cast<const float4*>(&wrow[c * kWp + qtr * 16 + 4 * k4]);
      const double a0 = fabs(static_cast<double>(a.x)), a1 = fabs(static_cast<double>(a.y));
      const double a2 = fabs(static_cast<double>(a.z)), a3 = fabs(static_cast<double>(a.w));
      csum += (a0 + a1) + (a2 + a3);
      mx = fmax(mx, fmax(fmax(a0, a1), fmax(a2, a3)));
      rsum += (fabs(static_cast<double>(r.x)) + fabs(static_cast<double>(r.y))) +
              (fabs(static_cast<double>(r.z)) + fabs(static_cast<double>(r.w)));
    }
    red[(0 * 4 + qtr) * 64 + c] = csum;
    red[(1 * 4 + qtr) * 64 + c] = rsum;
    red[(2 * 4 + qtr) * 64 + c] = mx;
  }
  __syncthreads();
  if (cs == 0) {
    // the sums in float64, their maxima over the 64 columns (rows) in float32: alpha then differs from the
    // all-float64 value by at most a few units of 2^-24
    auto sum4 = [&](int a) {
      return red[(a * 4 + 0) * 64 + ln] + red[(a * 4 + 1) * 64 + ln] + red[(a * 4 + 2) * 64 + ln] + red[(a * 4 + 3) * 64 + ln];
    };
    const float cmax = wave_max_nonneg(static_cast<float>(sum4(0)));
    const float rmax = wave_max_nonneg(static_cast<float>(sum4(1)));
    const float mx = wave_max_nonneg(static_cast<float>(
        fmax(fmax(red[8 * 64 + ln], red[9 * 64 + ln]), fmax(red[10 * 64 + ln], red[11 * 64 + ln]))));
    if (ln == 0) {
      s_alpha = static_cast<float>(1.0 / (static_cast<double>(cmax) * static_cast<double>(rmax)));
      s_wmax = mx;
    }
  }
  __syncthreads();
  const float alpha = s_alpha;
  if (tid == 0 && alpha_out) alpha_out[g] = alpha;

  // W^T as the B operand of B_k = A_k W^T: chunk c, lane (g, t) holds W^T rows (K) 32c + 4g .. +3 and
  // 32c + 16 + 4g .. +3 of column col, i.e. W[col][K].
  half8 wth[KC], wtl[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(&wrow[col * kWp + 32 * c + 4 * gq]);
    const float4 b = *reinterpret_cast<const float4*>(&wrow[col * kWp + 32 * c + 16 * (ST >= 2) + 4 * gq]);
    split_chunk(act ? f32x4{a.x, a.y, a.z, a.w} : f32x4{0.f, 0.f, 0.f, 0.f},
                (act && ST >= 2) ? f32x4{b.x, b.y, b.z, b.w} : f32x4{0.f, 0.f, 0.f, 0.f}, one, wth[c], wtl[c]);
  }
  // The kernel carries -A and -B (see below). -A_0 = -X_0^T = -alpha W, times 2^-ex: lane (g, t) of tile p holds
  // rows 16p + 4g .. +3 of column col.
  int ex = store_exp(alpha * s_wmax);
  f32x4 ax[NT];
  {
    const float s0 = act ? -alpha * ldexpf(1.f, -ex) : 0.f;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const float4 w = *reinterpret_cast<const float4*>(&wcol[col * kWp + 16 * p + 4 * gq]);
      ax[p] = f32x4{w.x, w.y, w.z, w.w} * s0;
    }
  }
  // X_k = -(the strip)^T to global memory: row col, columns 16p + 4g .. +3 (one base address per lane; only a
  // tile that reaches past column m - 1 needs a per-entry check).
  auto store_x = [&](float* __restrict__ dst) {
    if (!act || col >= m) return;
    const float s = -ldexpf(1.f, ex);
    float* __restrict__ row = dst + static_cast<size_t>(col) * m + 4 * gq;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      if (16 * p + 16 <= m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) row[16 * p + r] = ax[p][r] * s;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * p + 4 * gq + r < m) row[16 * p + r] = ax[p][r] * s;
      }
    }
  };
  auto xs_slot = [&](int k) { return xs + (static_cast<size_t>(g) * (iters + 1) + k) * mm; };
  if (xs) store_x(xs_slot(0));
  barrier_lds();  // W and W^T (inside sU) are dead after this point

  // Keep the strip's scale near 2^12: while its largest entry (times 2^-ex) stays in [2^8, 2^14), which the lanes
  // test on their own maxima with no cross-lane reduction, nothing happens; otherwise the exact maximum sets a
  // fresh exponent (one multiply per entry).
  auto rescale = [&]() {
    float lm = 0.f;
#pragma unroll
    for (int p = 0; p < NT; ++p)
      lm = fmaxf(lm, fmaxf(fmaxf(fabsf(ax[p][0]), fabsf(ax[p][1])), fmaxf(fabsf(ax[p][2]), fabsf(ax[p][3]))));
    const bool over = __ballot(lm >= 16384.f) != 0, some = __ballot(lm >= 256.f) != 0, any = __ballot(lm > 0.f) != 0;
    if (over || (any && !some)) {
      const float wm = wave_max_nonneg(lm);
      const int d = exp_of(wm) - 12;
      const float s = ldexpf(1.f, -d);
#pragma unroll
      for (int p = 0; p < NT; ++p) ax[p] *= s;
      ex += d;
    }
  };

  f32x4 bt[NT];            // -B_k
  half8 bth[KC], btl[KC];  // its split: the B operand of the T product and, stored, the A operand of both
  // Split -B into bth/btl and store it (by columns) into M.
  auto put_b = [&](RegSplit& M) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      split_chunk(bt[2 * c], (ST >= 2) ? bt[2 * c + 1] : f32x4{0.f, 0.f, 0.f, 0.f}, one, bth[c], btl[c]);
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const int c = p >> 1, o = (p & 1) * 4;
      *reinterpret_cast<half4*>(&M.hi[lane_w + 16 * p]) = half4{bth[c][o], bth[c][o + 1], bth[c][o + 2], bth[c][o + 3]};
      *reinterpret_cast<half4*>(&M.lo[lane_w + 16 * p]) = half4{btl[c][o], btl[c][o + 1], btl[c][o + 2], btl[c][o + 3]};
    }
  };

  // -B_k = (-A_k) W^T into bt: -A_k goes through tmp (a buffer that no wave reads once the first barrier is
  // passed) with one block-wide exponent eb, and the product comes back times 2^-eb.
  auto form_t = [&](RegSplit& tmp) {
    // every strip's largest entry is below 2^14 times its exponent after the check, so 2^(2 + the largest
    // exponent) puts every stored entry at or below 2^12
    if (act) {
      rescale();
      if (ln == 0) s_ex[cs] = ex;
    }
    barrier_lds();
    int eb = s_ex[0];
#pragma unroll
    for (int w = 1; w < ST; ++w) eb = max(eb, s_ex[w]);
    eb += 2;
    if (act) {
      const float s = ldexpf(1.f, ex - eb);
#pragma unroll
      for (int p = 0; p < NT; ++p) {
        half8 h, l;
        split_chunk(ax[p] * s, ax[p] * s, one, h, l);
        *reinterpret_cast<half4*>(&tmp.hi[lane_w + 16 * p]) = half4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<half4*>(&tmp.lo[lane_w + 16 * p]) = half4{l[0], l[1], l[2], l[3]};
      }
    }
    barrier_lds();
    if (act) {
      half8 ah[NT][KC], al[NT][KC];
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int p = 0; p < NT; ++p) load_rows<ST>(tmp, lane_r, c, p, ah[p][c], al[p][c]);
      const float us = ldexpf(1.f, eb);
#pragma unroll
      for (int p = 0; p < NT; ++p) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) acc = mma_split3(ah[p][c], al[p][c], wth[c], wtl[c], acc);
        bt[p] = acc * us;
      }
    }
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
  //
  // Transposed (A = X^T, B = T^T), the pair is A' = 2A - B A and B' = 2B - B B, and with the negated matrices
  // that the kernel carries, -A' = 2 (-A) + (-B)(-A) and -B' = 2 (-B) + (-B)(-B): each product starts from twice
  // the carried strip (exact in fp32) and adds the stored split of -B times the strip's own split. No 2I term is
  // formed (the identity enters through the 2 (-A) start), and the stored matrix is the split the T product
  // uses as its B operand anyway.
  //
  // Segment start at step k: -B_k = -(W X_k)^T, stored into the buffer of parity k & 1, which no wave reads now.
  auto resync = [&](int k) {
    form_t(sU[(k & 1) ^ 1]);  // the other buffer, last read by step k - 1, carries -A_k on the way
    if (act) put_b(sU[k & 1]);
    barrier_lds();
  };

  // One pair step; the buffer parity is a template constant so that every LDS address is a fixed offset.
  // last: the step ends a segment (or is the exact last step), so it forms only X_{k+1}.
  // Order: the first chunk's reads, the scale check and split of the A strip (while they are in flight), the
  // second chunk's reads, then the products chunk by chunk, T before X, and the T epilogue.
  auto step = [&](auto parity, auto last, int k) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
    constexpr bool kLast = decltype(last)::value;
    if (act) {
      half8 uh[NT][KC], ul[NT][KC];
#pragma unroll
      for (int p = 0; p < NT; ++p) load_rows<ST>(sU[cur], lane_r, 0, p, uh[p][0], ul[p][0]);
      __builtin_amdgcn_sched_barrier(0);
      rescale();
      half8 bxh[KC], bxl[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c)
        split_chunk(ax[2 * c], (ST >= 2) ? ax[2 * c + 1] : f32x4{0.f, 0.f, 0.f, 0.f}, one, bxh[c], bxl[c]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 1; c < KC; ++c)
#pragma unroll
        for (int p = 0; p < NT; ++p) load_rows<ST>(sU[cur], lane_r, c, p, uh[p][c], ul[p][c]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < NT; ++p) {
        if constexpr (!kLast) bt[p] += bt[p];
        ax[p] += ax[p];
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if constexpr (!kLast) {
#pragma unroll
          for (int p = 0; p < NT; ++p) bt[p] = mma_split3(uh[p][c], ul[p][c], bth[c], btl[c], bt[p]);
        }
#pragma unroll
        for (int p = 0; p < NT; ++p) ax[p] = mma_split3(uh[p][c], ul[p][c], bxh[c], bxl[c], ax[p]);
      }
      if constexpr (!kLast) put_b(sU[nxt]);
      if (xs) store_x(xs_slot(k + 1));
    }
    barrier_lds();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using Mid = std::integral_constant<bool, false>;
  using End = std::integral_constant<bool, true>;
  auto seg_start = [&](int k) { return k % kPairRun == 0 || k == iters - 1; };
  for (int k = 0; k < iters; ++k) {
    if (seg_start(k)) resync(k);
    const bool lst = k == iters - 1 || seg_start(k + 1);
    if (k & 1) {
      if (lst) step(P1{}, End{}, k); else step(P1{}, Mid{}, k);
    } else {
      if (lst) step(P0{}, End{}, k); else step(P0{}, Mid{}, k);
    }
  }

  store_x(Xout + g * mm);

  if (resid) {
    // ||W X_K - I||_F with the same split products: -(W X_K)^T through the segment-start path.
    form_t(sU[0]);
    double ss = 0.0;
    if (act) {
#pragma unroll
      for (int p = 0; p < NT; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * p + 4 * gq + r;
          if (i < m && col < m) {
            const double e2 = -static_cast<double>(bt[p][r]) - (i == col ? 1.0 : 0.0);
            ss += e2 * e2;
          }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    __syncthreads();
    if (ln == 0) s_res[cs] = ss;
    __syncthreads();
    if (tid == 0) resid[g] = static_cast<float>(sqrt(s_res[0] + s_res[1] + s_res[2] + s_res[3]));
  }
}

template <int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_ns_small(
    const float* __restrict__ We, float* __restrict__ Xout, float* __restrict__ xs, float* __restrict__ alpha_out,
    float* __restrict__ resid, int m, int iters) {
  __shared__ __attribute__((aligned(16))) char lds[kNsSmallLds];
  ns_small_block<ST>(lds, static_cast<int>(blockIdx.x), We, Xout, xs, alpha_out, resid, m, iters);
}
// =====================================================================================================
// Newton-Schulz with side work. The m <= 64 solver occupies one CU per slice for its whole chain of dependent
// steps while the rest of the chip would idle, and a second stream costs more in cross-queue synchronisation than
// it saves at this size. So the same launch carries, after the G solver blocks, blocks that compute
// S = C_K^T V, each one (slice, 16-landmark tile, 16-channel tile) of S over all N tokens. No block of this launch
// waits for another: a cross-XCD hand-off of partial sums needs device-scope release and acquire fences, and
// on this chip those write back and invalidate a whole L2, which costs more than the solver itself.
// Each block holds the solver's LDS (41 KB, so three blocks share a CU); the tiles fill the CUs the solver leaves
// free and finish inside the solver's time when C_K and V come from the last-level cache. Read from HBM they take
// longer than the solver: their loads go out in batches of 12 token groups (5 memory round trips per wave at
// N = 3136), which brought that case from 10.6 to about 6 us beyond the solver.
// =====================================================================================================

// One S tile by one block of NWV waves. Wave w sums a contiguous range of 16-token groups on fp32 MFMA (A = C_K,
// landmark-major, B = V): in group q, lane (i, k) feeds landmark i and channel i of the tile with tokens
// 16q + 4k + u at k-step u, loaded from global memory straight into the MFMA operand layout. The wave tiles are
// then summed in LDS (sRed: NWV x 256 floats) in wave order, so the result does not depend on timing.
constexpr int kSideWaves = 4;  // the solver's block size
constexpr int kCkvBatch = 12;  // 16-token groups per batch of loads

template <typename T, int D, int NWV>
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
  const int groups = (N + 15) / 16, gpw = (groups + NWV - 1) / NWV;
  const int q0 = min(groups, wv * gpw), q1 = min(groups, q0 + gpw);
  const int qf = max(q0, min(q1, N / 16));  // groups [q0, qf) have all 16 tokens in range
  const float amask = lok ? 1.f : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // Groups in batches of kCkvBatch, every load of a batch issued before its first MFMA: a wave walks about N / 64
  // groups, so the batches (not the loads of one group) set how many memory round trips the tile waits for.
  auto full_groups = [&](auto vec) {
    for (int q = q0; q < qf; q += kCkvBatch) {
      float a[kCkvBatch][4], b[kCkvBatch][4];
#pragma unroll
      for (int j = 0; j < kCkvBatch; ++j) {
        // a group past the range repeats the last one with a zero weight (in bounds, adds nothing)
        const int qj = min(q + j, qf - 1);
        const int t = qj * 16 + 4 * k;
        const float wj = q + j < qf ? amask : 0.f;
        if constexpr (decltype(vec)::value) {
          const float4 c4 = load4(crow + t);
          a[j][0] = c4.x * wj;
          a[j][1] = c4.y * wj;
          a[j][2] = c4.z * wj;
          a[j][3] = c4.w * wj;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) a[j][u] = crow[t + u] * wj;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) b[j][u] = to_f32(vcol[static_cast<size_t>(t + u) * D]);
      }
#pragma unroll
      for (int j = 0; j < kCkvBatch; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma16x16x4(a[j][u], b[j][u], acc);
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
    for (int w = 0; w < NWV; ++w) sum += sRed[w * 256 + tid];
    if (lt * 16 + row < m) S[(static_cast<size_t>(g) * m + lt * 16 + row) * D + ct * 16 + col] = sum;
  }
}

// All of slice g's S = C^T V by one block of 4 waves, for launches with more slices than CUs (few tokens per
// slice): wave w takes tiles w, w + 4, .. (at most 4) of the slice and sums each over all N tokens by itself, so
// the tiles need no reduction across waves. The loads go out in batches that cover all of the wave's tiles at
// once (3 token groups of each), and the ragged last group of every tile in one more batch: a tile-by-tile walk
// waited for twice as many memory round trips.
constexpr int kSliceGpb = 3;  // 16-token groups of each tile per batch

template <typename T, int D>
__device__ __forceinline__ void ckv_slice_block(int g, const float* __restrict__ C, const T* __restrict__ V,
                                                float* __restrict__ S, int N, int m) {
  constexpr int DT = D / 16, TPW = 4;
  const int LT = (m + 15) / 16, ntile = LT * DT;
  const int wv = __builtin_amdgcn_readfirstlane(wave_id()), ln = lane_id();
  const int i = ln & 15, k = ln >> 4;
  const int groups = (N + 15) / 16, qf = N / 16;  // groups [0, qf) have all 16 tokens in range
  const float* crow[TPW];
  const T* vcol[TPW];
  float amask[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tt = min(wv + 4 * j, ntile - 1), lt = tt / DT, ct = tt % DT;
    const bool lok = lt * 16 + i < m && wv + 4 * j < ntile;
    crow[j] = C + (static_cast<size_t>(g) * m + (lt * 16 + i < m ? lt * 16 + i : 0)) * N;
    vcol[j] = V + static_cast<size_t>(g) * N * D + ct * 16 + i;
    amask[j] = lok ? 1.f : 0.f;
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < qf; q += kSliceGpb) {
    float a[TPW][kSliceGpb][4], b[TPW][kSliceGpb][4];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int h = 0; h < kSliceGpb; ++h) {
        const int qh = min(q + h, qf - 1);  // past the range: the last group again with a zero weight
        const int t = qh * 16 + 4 * k;
        const float wh = q + h < qf ? amask[j] : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[j][h][u] = crow[j][t + u] * wh;
          b[j][h][u] = to_f32(vcol[j][static_cast<size_t>(t + u) * D]);
        }
      }
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int h = 0; h < kSliceGpb; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[j] = mfma16x16x4(a[j][h][u], b[j][h][u], acc[j]);
  }
  if (qf < groups) {  // the ragged last group of every tile
    const int t = qf * 16 + 4 * k;
    float a[TPW][4], b[TPW][4];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = t + u < N;
        const size_t tc = static_cast<size_t>(in ? t + u : N - 1);
        a[j][u] = in ? crow[j][tc] * amask[j] : 0.f;
        b[j][u] = in ? to_f32(vcol[j][tc * D]) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[j] = mfma16x16x4(a[j][u], b[j][u], acc[j]);
  }
  // acc[j][r] is row 4k + r, column i of the wave's tile j
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tt = wv + 4 * j;
    if (tt >= ntile) continue;
    const int lt = tt / DT, ct = tt % DT;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lt * 16 + 4 * k + r < m)
        S[(static_cast<size_t>(g) * m + lt * 16 + 4 * k + r) * D + ct * 16 + i] = acc[j][r];
  }
}

// Tile order of the S tiles of a launch (j < total): consecutive tiles are dealt to the 8 XCDs round-robin, so the
// order is remapped to keep the tiles of one slice on one XCD: each slice's C_K rows and V columns are read by
// several tiles, and one L2 then serves the repeats.
__device__ __forceinline__ int ckv_tile_order(int j, int total) {
  const int full = (total / 8) * 8;
  return j < full ? (j % 8) * (full / 8) + j / 8 : j;
}

template <typename T, int D, int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_ns_side(const float* __restrict__ We, float* __restrict__ Xout,
                                                 float* __restrict__ xs, float* __restrict__ alpha_out, int m,
                                                 int iters, int N, int G, const float* __restrict__ CK,
                                                 const T* __restrict__ V, float* __restrict__ S, int per_slice) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < G) {
    __shared__ __attribute__((aligned(16))) char lds[kNsSmallLds];
    ns_small_block<ST>(lds, b, We, Xout, xs, alpha_out, nullptr, m, iters);
    return;
  }
  if (per_slice) {  // one block per slice (more slices than CUs): side block j is slice j
    const int s0 = (G + 7) & ~7;
    if (b >= s0) ckv_slice_block<T, D>(b - s0, CK, V, S, N, m);
    return;
  }
  // The S tiles start at the first multiple of 8 after the solver blocks (the blocks in between exit at once), so
  // that tile j runs on XCD j % 8 (the hardware deals blocks to the 8 XCDs round-robin).
  const int s0 = (G + 7) & ~7;
  if (b < s0) return;
  const int j = ckv_tile_order(b - s0, static_cast<int>(gridDim.x) - s0);
  __shared__ float sRed[kSideWaves * 256];
  ckv_tile_block<T, D, kSideWaves>(j, CK, V, S, N, m, sRed);
}

// =====================================================================================================
// Newton-Schulz beside the S tiles and the C_Q distance pass (Laplace kernel, m <= 64). C_Q is needed only after
// the solver (by the whitening statistics and the output kernel), so instead of running before the solver it runs in the solver's launch: after
// the G solver blocks come the S = C_K^T V tiles (as in the launch above; C_K and W_eps come from the distance
// launch before) and then the distance blocks for the rows of Q (four waves each, a quarter of the landmarks per
// wave). All of them fill the CUs the solver leaves free and finish in its shadow. The three kinds of block share
// one LDS allocation (the solver's 41 KB), so three blocks fit a CU.
// =====================================================================================================
template <typename T, int D, int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_ns_laplace(
    const float* __restrict__ We, float* __restrict__ Xout, float* __restrict__ xs, float* __restrict__ alpha_out,
    int m, int iters, int G, const float* __restrict__ CK, const T* __restrict__ V, float* __restrict__ S, int nS,
    const T* __restrict__ Q,
    const float* __restrict__ L, float* __restrict__ CQ, int N, int nlap, int tilesN, int lc, float scale,
    float* __restrict__ wst) {
  __shared__ __attribute__((aligned(16))) char lds[kNsSmallLds > kLaplaceLds<D> ? kNsSmallLds : kLaplaceLds<D>];
  static_assert(kSideWaves * 256 * 4 <= kNsSmallLds, "S tile reduction exceeds the shared LDS");
  const int b = static_cast<int>(blockIdx.x);
  if (b < G) {
    ns_small_block<ST>(lds, b, We, Xout, xs, alpha_out, nullptr, m, iters);
    return;
  }
  // each group of side blocks starts at a multiple of 8 (the blocks in between exit at once), so that side block j
  // of a group runs on XCD j % 8
  const int s0 = (G + 7) & ~7, s1 = s0 + ((nS + 7) & ~7);
  if (b < s0) return;
  if (b < s1) {
    if (b - s0 < nS) ckv_tile_block<T, D, kSideWaves>(ckv_tile_order(b - s0, nS), CK, V, S, N, m, reinterpret_cast<float*>(lds));
    return;
  }
  // (only rows of Q here: the W_eps and C_K outputs are never reached); with wst, also the tiles' whitening
  // partials
  if (wst)
    laplace_block<T, D, true>(reinterpret_cast<float*>(lds), b - s1, nlap, 4, Q, Q, L, CQ, CQ,
                              const_cast<float*>(We), N, m, tilesN, 0, 0, 1, lc, scale, 0.f, wst);
  else
    laplace_block<T, D>(reinterpret_cast<float*>(lds), b - s1, nlap, 4, Q, Q, L, CQ, CQ, const_cast<float*>(We), N,
                        m, tilesN, 0, 0, 1, lc, scale, 0.f);
}

template <typename T, int D>
static void ns_side_st(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                       const T* V, float* S, hipStream_t st) {
  // With at least as many slices as CUs the solver blocks alone fill the chip, and S comes from one block per
  // slice (fewer, longer side blocks) instead of one per 16 x 16 tile.
  const int per_slice = s.G >= 256 ? 1 : 0;
  const int side = per_slice ? s.G : s.G * ((s.m + 15) / 16 * (D / 16));
  const int blocks = ((s.G + 7) & ~7) + side;  // solver blocks, padding, S blocks
  const int nt = (s.m + 15) / 16;
#define LF_NS_SIDE(ST_)                                                                                        \
  hipLaunchKernelGGL((k_ns_side<T, D, ST_>), dim3(blocks), dim3(256), 0, st, We, X, xs, alpha, s.m, s.ns_iters, \
                     s.N, s.G, CK, V, S, per_slice)
  if (nt == 1)
    LF_NS_SIDE(1);
  else if (nt == 2)
    LF_NS_SIDE(2);
  else
    LF_NS_SIDE(4);
#undef LF_NS_SIDE
}

bool ns_side_supported(const Shape& s) { return s.m <= 64 && (s.d == 16 || s.d == 32 || s.d == 64); }

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

bool ns_laplace_supported(const Shape& s) { return ns_side_supported(s) && s.G < 256; }

template <typename T, int D>
static void ns_laplace_st(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                          const T* V, float* S, const T* Q, const float* L, float* CQ, float* wst, hipStream_t st) {
  const int tilesN = (s.N + 63) / 64, nlap = s.G * tilesN, lc = (s.m + 3) / 4;
  const int nS = s.G * ((s.m + 15) / 16) * (D / 16);
  const int blocks = ((s.G + 7) & ~7) + ((nS + 7) & ~7) + nlap;  // solver blocks, S tiles, C_Q distance blocks
  const float scale = static_cast<float>(-1.4426950408889634 / static_cast<double>(s.lambda));
  const int nt = (s.m + 15) / 16;
#define LF_NS_LAP(ST_)                                                                                         \
  hipLaunchKernelGGL((k_ns_laplace<T, D, ST_>), dim3(blocks), dim3(256), 0, st, We, X, xs, alpha, s.m,          \
                     s.ns_iters, s.G, CK, V, S, nS, Q, L, CQ, s.N, nlap, tilesN, lc, scale, wst)
  if (nt == 1)
    LF_NS_LAP(1);
  else if (nt == 2)
    LF_NS_LAP(2);
  else
    LF_NS_LAP(4);
#undef LF_NS_LAP
}

template <typename T>
static void ns_laplace_t(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                         const void* V, float* S, const void* Q, const float* L, float* CQ, float* wst,
                         hipStream_t st) {
  const T* v = static_cast<const T*>(V);
  const T* q = static_cast<const T*>(Q);
  switch (s.d) {
    case 16: ns_laplace_st<T, 16>(s, We, X, xs, alpha, CK, v, S, q, L, CQ, wst, st); break;
    case 32: ns_laplace_st<T, 32>(s, We, X, xs, alpha, CK, v, S, q, L, CQ, wst, st); break;
    default: ns_laplace_st<T, 64>(s, We, X, xs, alpha, CK, v, S, q, L, CQ, wst, st); break;
  }
}

hipError_t launch_ns_laplace(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                             const void* V, float* S, const void* Q, const float* L, float* CQ, hipStream_t st,
                             float* wst) {
  if (!ns_laplace_supported(s)) return hipErrorInvalidValue;
  if (s.dtype == 1)
    ns_laplace_t<bf16_t>(s, We, X, xs, alpha, CK, V, S, Q, L, CQ, wst, st);
  else
    ns_laplace_t<float>(s, We, X, xs, alpha, CK, V, S, Q, L, CQ, wst, st);
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
                                             int g, int ti, int tj, NsTileLds& L) {
  constexpr int mp = NT * kTile, nt = NT;
  _Float16* sA = L.a;
  _Float16* sB = L.b;
  float* s_red = L.red;
  double* s_cmax = L.cmax;
  double* s_rmax = L.rmax;
  const int tid = threadIdx.x, wv = wave_id(), ln = lane_id();
  const size_t mpp = static_cast<size_t>(mp) * mp, mm = static_cast<size_t>(m) * m;
  const float* wg = We + g * mm;

  // The exponents of A's row of tiles and B's column of tiles: one power of two per 32-wide K chunk, loaded with
  // the strips so that their round trip overlaps the staging.
  int ech[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int ea = J.a_exp ? J.a_exp[(static_cast<size_t>(g) * nt + ti) * nt + c] : 0;
    const int eb = J.b_exp ? J.b_exp[(static_cast<size_t>(g) * nt + c) * nt + tj] : 0;
    ech[c] = ea + eb;
  }
  // The wave's 16 x 16 sub-tile (wi, wj); the lane's output rows i0 .. i0+3 of column j.
  const int wi = wv & 1, wj = wv >> 1, gq = ln >> 4, t = ln & 15;
  const int i0 = ti * kTile + wi * 16 + 4 * gq, j = tj * kTile + wj * 16 + t;
  // The first launch's own inputs, loaded with the strips: the alpha chunk partials of column tid (m <= 256
  // columns, at most 32 chunks), chunk tid's largest row sum, and the lane's entries of W^T for X_0.
  constexpr int kMaxCh = LF_NS_KMAX / kNsRows;
  double pv[kMaxCh], rmx0 = 0.0;
  float wt[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (AW && BW) {
    if (init.part) {
      const int jc = tid < m ? tid : 0;
#pragma unroll
      for (int c = 0; c < kMaxCh; ++c)
        pv[c] = init.part[(static_cast<size_t>(g) * init.nch + (c < init.nch ? c : 0)) * m + jc];
      rmx0 = tid < init.nch ? init.rmx[static_cast<size_t>(g) * init.nch + tid] : 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = i0 + r < m && j < m;
        wt[r] = wg[ok ? static_cast<size_t>(j) * m + i0 + r : 0];
      }
    }
  }

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
  if (AW && BW && init.part) {
    // thread j sums column j's chunk partials; chunk c's largest row sum comes from thread c
    double cs = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxCh; ++c)
      if (c < init.nch) cs += pv[c];
    double cmax = tid < m ? cs : 0.0;
    double rmax = rmx0;
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
  if (AW && BW && init.part) scale = L.alpha;

  // 2. The wave's 16 x 16 sub-tile (wi, wj), chunk by chunk: three split-fp16 MFMAs per chunk into a fresh
  //    accumulator, folded into the sum with the chunk's power of two.
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
  if (AW && BW && init.part) {
    // X_0 = alpha W^T over this tile: X_0[i][j] = alpha W[j][i] (rows i0 .. i0+3 of column j, contiguous in W).
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (i0 + r < m && j < m) ? scale * wt[r] : 0.f;
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

// One block per output tile of nz products (z = slice * njobs + job; job z % njobs is j0 or j1). The 8 XCDs take
// blocks round robin (block b on XCD b % 8), so when the tile count is a multiple of 8 block b takes tile
// (b % 8) (count / 8) + b / 8: each XCD gets a contiguous run of whole rows of tiles of one product and reads few
// distinct A strips, instead of every XCD reading every A strip. Any bijection is correct; this one is for L2.
template <bool AW, bool BW, int NT>
__global__ __launch_bounds__(256) void k_ns_tile(NsJob j0, NsJob j1, int njobs, NsInit init,
                                                 const float* __restrict__ We, int m) {
  __shared__ NsTileLds lds;
  const int nb = gridDim.x, b = blockIdx.x;
  const int t = (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int z = t / (NT * NT), r = t % (NT * NT), ti = r / NT, tj = r % NT;
  const int g = z / njobs;
  if (z % njobs == 0)
    ns_tile_body<AW, BW, NT>(j0, init, We, m, g, ti, tj, lds);
  else
    ns_tile_body<AW, BW, NT>(j1, init, We, m, g, ti, tj, lds);
}

// k_ns_tile for the tile count of m: 3 .. 8 (65 <= m <= 256), over nz products.
template <bool AW, bool BW>
static void ns_tile_launch(int nt, int nz, hipStream_t st, const NsJob& j0, const NsJob& j1, int njobs,
                           const NsInit& init, const float* We, int m) {
  const dim3 grid(nt * nt * nz);
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
    const dim3 grid(s.G), block(256);
    if (nt == 1)
      hipLaunchKernelGGL((k_ns_small<1>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else if (nt == 2)
      hipLaunchKernelGGL((k_ns_small<2>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
    else
      hipLaunchKernelGGL((k_ns_small<4>), grid, block, 0, st, We, X, xs, alpha, resid, m, K);
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
    ns_tile_launch<true, true>(nt, G, st, j, none, 1, in, We, m);
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
      ns_tile_launch<true, false>(nt, G, st, j, none, 1, noinit, We, m);
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
      ns_tile_launch<false, false>(nt, nj * G, st, jx, jt, nj, noinit, We, m);
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
    ns_tile_launch<true, false>(nt, G, st, ju, none, 1, noinit, We, m);
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
    ns_tile_launch<false, false>(nt, G, st, jx, none, 1, noinit, We, m);
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
    ns_tile_launch<true, false>(nt, G, st, jr, none, 1, noinit, We, m);
    hipLaunchKernelGGL(k_frob, dim3(G), dim3(256), 0, st, E, resid, m);
  }
  return hipGetLastError();
}

}  // namespace lf
