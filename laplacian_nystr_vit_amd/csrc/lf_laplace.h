// The distance kernel's block (shared by the distance launch and the launch that runs it beside the small
// Newton-Schulz solver).
#pragma once

#include "lf_device.h"

namespace lf {

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
// Grid: one block per (slice, source, 64-row tile, landmark super-chunk) of nw waves. The block stages its 64 rows
// in LDS once (as float32) and wave w of super-chunk sc takes the landmarks [(sc nw + w) lc, + lc): every row
// leaves HBM once per super-chunk instead of once per wave, and the waves still split the landmark loop finely
// enough that each SIMD holds several of them.
// Block order: the super-chunks of one tile are consecutive, and blocks are remapped so that consecutive ones
// run on one XCD (each XCD has its own L2 and the hardware deals blocks to the XCDs round-robin). A slice's
// blocks then stay on few XCDs, so the CUs of an XCD share one slice's landmark rows in their scalar caches and
// the super-chunks of a tile share its rows through L2.
// =====================================================================================================
// Rows staged by one block: 64 rows of D floats at a stride of D + 4 (8 lanes of a float4 read cover all 32 banks).
template <int D>
constexpr int kLaplaceLds = 64 * (D + 4) * 4;

// Sum over the wave, wave-uniform, in a fixed order: DPP steps inside each row of 16 lanes (quad swaps, then
// rotations by 4 and 8), then the four row sums through scalar reads of lanes 0, 16, 32 and 48.
__device__ __forceinline__ float wave_sum_fixed(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// One block of the distance kernel: b is the block's index among nblocks such blocks, which run nw waves each and
// were dealt to the XCDs round-robin from a multiple of 8; sX is kLaplaceLds<D> bytes of LDS.
// tilesQ / tilesK / tilesL: 64-row tiles of Q, K and L rows per slice (0 leaves that source out).
// STATS (Q rows only): per (slice, landmark, Q tile) the tile's sum of C and sum of squared deviations from the
// tile's mean go to wst[2 ((g m + l) tilesQ + tile)] and + 1, for the whitening statistics of C_Q (Design 1 of
// the note).
template <typename T, int D, bool STATS = false>
__device__ __forceinline__ void laplace_block(float* __restrict__ sX, int b, int nblocks, int nw,
                                              const T* __restrict__ Q, const T* __restrict__ K,
                                              const float* __restrict__ L, float* __restrict__ CQ,
                                              float* __restrict__ CK, float* __restrict__ We, int N, int m,
                                              int tilesQ, int tilesK, int tilesL, int nsc, int lc, float scale,
                                              float eps, float* __restrict__ wst = nullptr) {
  constexpr int LDX = D + 4;
  {
    const int full = (nblocks / 8) * 8;
    if (b < full) b = (b % 8) * (full / 8) + b / 8;
  }
  const int tid = static_cast<int>(threadIdx.x), lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());  // uniform, so landmark loads stay scalar
  const int sc = b % nsc;
  b /= nsc;
  const int per_slice = tilesQ + tilesK + tilesL;
  const int local = b % per_slice;
  const int g = b / per_slice;
  int src, tile;
  if (local < tilesQ) {
    src = 0;
    tile = local;
  } else if (local < tilesQ + tilesK) {
    src = 1;
    tile = local - tilesQ;
  } else {
    src = 2;
    tile = local - tilesQ - tilesK;
  }
  const int rows = (src == 2) ? m : N;
  const float* __restrict__ Lg = L + static_cast<size_t>(g) * m * D;
  const T* __restrict__ xg = (src == 0 ? Q : K) + static_cast<size_t>(g) * N * D;
  const int l0 = (sc * nw + wv) * lc;
  const int l1 = min(l0 + lc, m);
  // The wave's first landmark row is fetched (scalar loads, wave-uniform address) before the rows are staged, so
  // its latency overlaps the staging instead of following it.
  float lfirst[D];
  {
    const float* __restrict__ lp = Lg + static_cast<size_t>(min(l0, m - 1)) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) lfirst[c] = lp[c];
  }
  for (int e = tid; e < 16 * D; e += 64 * nw) {  // float4 index over [64 rows][D / 4]
    const int r = e / (D / 4), c4 = e % (D / 4);
    const int row = tile * 64 + r;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < rows) v = (src == 2) ? load4(Lg + static_cast<size_t>(row) * D + 4 * c4)
                                   : load4(xg + static_cast<size_t>(row) * D + 4 * c4);
    store4(sX + r * LDX + 4 * c4, v);
  }
  __syncthreads();
  const int row = tile * 64 + lane;
  // With the statistics every lane stays (rows past the end compute on zeros and store nothing); otherwise they
  // leave here.
  const bool stats = STATS && src == 0;
  if ((row >= rows && !stats) || l0 >= l1) return;
  const bool valid = row < rows;

  float x[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const float4 v = *reinterpret_cast<const float4*>(sX + lane * LDX + c);
    x[c] = v.x;
    x[c + 1] = v.y;
    x[c + 2] = v.z;
    x[c + 3] = v.w;
  }
  float* out;  // this row's output, element l at out[l * ostride]
  size_t ostride;
  if (src == 2) {
    out = We + (static_cast<size_t>(g) * m + row) * m;
    ostride = 1;
  } else {
    // C is stored landmark-major (C[g][l][i]): for a fixed landmark the 64 lanes of a wave write 64 consecutive
    // floats, one 256-byte segment per store instruction.
    out = (src == 0 ? CQ : CK) + static_cast<size_t>(g) * m * N + row;
    ostride = static_cast<size_t>(N);
  }

  auto one = [&](int l, const float* lp) {
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
    if (!STATS || valid) out[l * ostride] = v;
    if (STATS && stats) {
      const int n = min(64, rows - tile * 64);
      const float sum = wave_sum_fixed(valid ? v : 0.f);
      const float dv = valid ? v - sum / static_cast<float>(n) : 0.f;
      const float ssd = wave_sum_fixed(dv * dv);
      if (lane == 0) {
        float* w = wst + 2 * ((static_cast<size_t>(g) * m + l) * tilesQ + tile);
        w[0] = sum;
        w[1] = ssd;
      }
    }
  };
  one(l0, lfirst);
  for (int l = l0 + 1; l < l1; ++l) one(l, Lg + static_cast<size_t>(l) * D);
}

}  // namespace lf
