// Host-side launch interface between the C ABI layer (lf_api.cpp) and the kernel translation units.
// Every launcher enqueues on `stream` and returns hipGetLastError()'s status; shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

struct Shape {
  int G, heads, H, W, d, r, m, N;
  int dtype;  // 0 = float32, 1 = bf16
  float lambda, eps;
  int ns_iters;
  float whiten_eps;
};

// Number of row splits of the C_K^T V reduction, and the rows each split covers (a multiple of 64).
void ckv_split(const Shape& s, int* nsplit, int* rows_per_split);

hipError_t launch_landmark_pool(const Shape& s, const void* Q, float* L, hipStream_t st);
// srcmask selects the row sources: 1 = Q rows (C_Q), 2 = K rows (C_K), 4 = landmark rows (W_eps).
hipError_t launch_laplace(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                          float* We, hipStream_t st, int srcmask = 7);
// Gaussian-kernel variant of launch_laplace (all three sources): C_Q, C_K from ||x||^2 + ||l||^2 - 2 x.l on fp32
// MFMA, W_eps from the differences.
hipError_t launch_gauss(const Shape& s, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                        float* We, hipStream_t st);
hipError_t launch_whiten_stats(const Shape& s, const float* CQ, float* mu, float* rstd, hipStream_t st);
hipError_t launch_ckv(const Shape& s, const float* CK, const void* V, float* partial, float* S, hipStream_t st);
// Same reduction with an optional appended column of ones in C (ones = 1): S gets m + ones rows.
// `partial` must hold G * nsplit * (m + ones) * d floats.
hipError_t launch_ckv_general(const Shape& s, const float* C, int ones, const void* V, float* partial, float* S,
                              hipStream_t st);
hipError_t launch_mix(const Shape& s, const float* X, const float* S, const float* rstd, float* P, float* Praw,
                      hipStream_t st);
// launch_mix with the whitening statistics finished first from the per-tile partials wst (written by the C_Q
// blocks of launch_ns_laplace): mu and rstd are written, and P = rstd (X S).
hipError_t launch_mix_whiten(const Shape& s, const float* X, const float* S, const float* wst, float* mu, float* rstd,
                             float* P, float* Praw, hipStream_t st);
hipError_t launch_out(const Shape& s, const float* CQ, const float* P, const float* mu, const void* V,
                      const float* w, void* Y, hipStream_t st);
// Y = C_Q (X S) + DWC(V) with P = X S formed in the output kernel (no whitening; out_mix_supported: m <= 64, d >= 32).
bool out_mix_supported(const Shape& s);
// Whether the inference forward recomputes C_Q inside the output kernel (launch_out_fused) rather than storing it
// from the distance launch and reading it back (measured per shape).
bool out_fused_pays(const Shape& s);
hipError_t launch_out_mix(const Shape& s, const float* CQ, const float* X, const float* S, const void* V,
                          const float* w, void* Y, hipStream_t st);
// Y = C_Q P + DWC(V) with C_Q computed in the kernel from Q and L (no whitening); C_Q is never stored.
hipError_t launch_out_fused(const Shape& s, const void* Q, const float* L, const float* P, const void* V,
                            const float* w, void* Y, hipStream_t st);
// out = C P + DWC^T(U): the output kernel with the 3x3 filter rotated by 180 degrees (adjoint stencil).
hipError_t launch_out_adjoint(const Shape& s, const float* C, const float* P, const void* U, const float* w, void* out,
                              hipStream_t st);

// Newton-Schulz. `tmp` is a [G][m][m] float32 scratch (used when m > 64); xs may be null.
size_t ns_tmp_floats(const Shape& s);
hipError_t launch_ns(const Shape& s, const float* We, float* X, float* xs, float* alpha, float* resid, float* tmp,
                     hipStream_t st);
// Newton-Schulz (m <= 64) in one launch with S = C_K^T V computed in the CUs the solver leaves idle.
// ns_side_supported: m <= 64 and d in {16, 32, 64}. ns_laplace_supported also needs fewer slices than CUs.
bool ns_side_supported(const Shape& s);
// Newton-Schulz beside S = C_K^T V and the C_Q distance pass in one launch (Laplace kernel; C_K and W_eps from a
// prior distance launch over the K and landmark rows). xs: saved iterates or null.
bool ns_laplace_supported(const Shape& s);
// wst: when not null, the C_Q blocks also write the per-tile whitening partials (2 G m ceil(N / 64) floats) that
// launch_mix_whiten finishes.
hipError_t launch_ns_laplace(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                             const void* V, float* S, const void* Q, const float* L, float* CQ, hipStream_t st,
                             float* wst = nullptr);
hipError_t launch_ns_side(const Shape& s, const float* We, float* X, float* xs, float* alpha, const float* CK,
                          const void* V, float* S, hipStream_t st);

// Device address of this device's copy of the static scratch array behind lf_attn_fwd_noalloc
// (LF_NOALLOC_SCRATCH_BYTES bytes), for the device `st` belongs to; looked up on the first call per device.
hipError_t noalloc_scratch(hipStream_t st, void** out);

// A second stream the caller owns, with two events of its own, for backward work that does not depend on the
// rest: the caller's stream forks to it through `fork` and waits on `join`. Null members are never passed here.
struct AuxStream {
  hipStream_t s;
  hipEvent_t fork, join;
};

// Conjugate gradients for W_eps X = I, one column per CG solve (cg_supported: 1 <= m <= 64). resid: NULL or
// [G][iters] receiving ||W_eps X_k - I||_F after every step. iters <= kCgItersMax.
constexpr int kCgItersMax = 256;
bool cg_supported(const Shape& s);
hipError_t launch_cg(const Shape& s, const float* We, float* X, float* resid, int iters, hipStream_t st);

}  // namespace lf
