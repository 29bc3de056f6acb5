// C ABI of liblf_attn: parameter validation, workspace planning and the launch sequence of the forward and
// backward passes. Host code only; the kernels live in lf_fwd.hip, lf_ns.hip, lf_bwd.hip, lf_cg.hip and lf_gauss.hip.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/lf_attn.h"
#include "lf_internal.h"
#include "lf_bwd_internal.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Checks everything that can be checked without touching the device.
int validate(const lf_attn_params* p) {
  if (!p) return LF_EINVAL;
  if (p->B < 1 || p->heads < 1 || p->H < 1 || p->W < 1 || p->d < 1 || p->r < 1) return LF_EINVAL;
  if (p->H % p->r != 0 || p->W % p->r != 0) return LF_EINVAL;
  if (!(p->lambda > 0.f) || !std::isfinite(p->lambda)) return LF_EINVAL;
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return LF_EINVAL;
  if (p->ns_iters < 0 || p->ns_iters > LF_NS_ITERS_MAX) return LF_EINVAL;
  if (p->whiten != 0 && p->whiten != 1) return LF_EINVAL;
  if (p->whiten == 1 && (!(p->whiten_eps > 0.f) || !std::isfinite(p->whiten_eps))) return LF_EINVAL;
  if (p->dtype != LF_F32 && p->dtype != LF_BF16) return LF_EINVAL;
  if (p->kernel != LF_KERNEL_LAPLACE && p->kernel != LF_KERNEL_GAUSS) return LF_EINVAL;
  // Sizes: keep every element index inside int range for the per-slice arithmetic, and totals in size_t.
  const int64_t N = static_cast<int64_t>(p->H) * p->W;
  if (N > (1 << 24)) return LF_EUNSUPPORTED;
  const int64_t G = static_cast<int64_t>(p->B) * p->heads;
  if (G > (1 << 20)) return LF_EUNSUPPORTED;
  if (p->d != 16 && p->d != 32 && p->d != 64 && p->d != 128) return LF_EUNSUPPORTED;
  const int64_t m = static_cast<int64_t>(p->H / p->r) * (p->W / p->r);
  if (m > LF_M_MAX) return LF_EUNSUPPORTED;
  return LF_OK;
}

lf::Shape make_shape(const lf_attn_params* p) {
  lf::Shape s;
  s.G = p->B * p->heads;
  s.heads = p->heads;
  s.H = p->H;
  s.W = p->W;
  s.d = p->d;
  s.r = p->r;
  s.m = (p->H / p->r) * (p->W / p->r);
  s.N = p->H * p->W;
  s.dtype = p->dtype;
  s.lambda = p->lambda;
  s.eps = p->eps;
  s.ns_iters = p->ns_iters;
  s.whiten_eps = p->whiten_eps;
  return s;
}

inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

lf_saved_layout saved_layout(const lf::Shape& s) {
  const size_t G = s.G, N = s.N, m = s.m, d = s.d, K = s.ns_iters;
  Carver c;
  lf_saved_layout L;
  L.L = c.take(4 * G * m * d);
  L.CQ = c.take(4 * G * N * m);
  L.CK = c.take(4 * G * N * m);
  L.We = c.take(4 * G * m * m);
  L.xs = c.take(4 * G * (K + 1) * m * m);
  L.mu = c.take(4 * G * m);
  L.rstd = c.take(4 * G * m);
  L.S = c.take(4 * G * m * d);
  L.P = c.take(4 * G * m * d);
  L.alpha = c.take(4 * G);
  L.total = c.off;
  return L;
}

// Forward workspace. Without a saved buffer every intermediate lives here; with one, only X, the scaled P,
// the C_K^T V partials and the Newton-Schulz scratch do.
struct FwdWs {
  size_t L, CQ, CK, We, X, S, P, Pw, mu, rstd, alpha, part, nstmp, wst, total;
};

FwdWs fwd_ws(const lf::Shape& s) {
  const size_t G = s.G, N = s.N, m = s.m, d = s.d;
  int nsplit, rps;
  lf::ckv_split(s, &nsplit, &rps);
  Carver c;
  FwdWs w;
  w.L = c.take(4 * G * m * d);
  w.CQ = c.take(4 * G * N * m);
  w.CK = c.take(4 * G * N * m);
  w.We = c.take(4 * G * m * m);
  w.X = c.take(4 * G * m * m);
  w.S = c.take(4 * G * m * d);
  w.P = c.take(4 * G * m * d);
  w.Pw = c.take(4 * G * m * d);
  w.mu = c.take(4 * G * m);
  w.rstd = c.take(4 * G * m);
  w.alpha = c.take(4 * G);
  w.part = c.take(nsplit > 1 ? 4 * G * static_cast<size_t>(nsplit) * m * d : 0);
  w.nstmp = c.take(4 * lf::ns_tmp_floats(s));
  w.wst = c.take(4 * 2 * G * m * ((N + 63) / 64));
  w.total = c.off;
  return w;
}

template <typename T>
inline T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? LF_OK : LF_EHIP; }


#define LF_TRY(expr)                        \
  do {                                      \
    const int _rc = hip_status(expr);       \
    if (_rc != LF_OK) return _rc;           \
  } while (0)

}  // namespace

extern "C" {

const char* lf_strerror(int code) {
  switch (code) {
    case LF_OK: return "ok";
    case LF_EINVAL: return "invalid argument (shape, parameter, null or misaligned pointer)";
    case LF_EWORKSPACE: return "workspace too small";
    case LF_EUNSUPPORTED: return "unsupported configuration";
    case LF_EHIP: return "HIP kernel launch failed";
    default: return "unknown lf_attn status";
  }
}

int lf_attn_query(const lf_attn_params* p, size_t* fwd_ws_bytes, size_t* saved_bytes, size_t* bwd_ws_bytes) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  const lf::Shape s = make_shape(p);
  if (fwd_ws_bytes) *fwd_ws_bytes = fwd_ws(s).total;
  if (saved_bytes) *saved_bytes = saved_layout(s).total;
  if (bwd_ws_bytes) *bwd_ws_bytes = lf::bwd_ws_bytes(s);
  return LF_OK;
}

int lf_attn_saved_layout(const lf_attn_params* p, lf_saved_layout* out) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!out) return LF_EINVAL;
  *out = saved_layout(make_shape(p));
  return LF_OK;
}

}  // extern "C"

namespace {

// Checks of the forward's arguments other than the workspace.
int validate_fwd(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                 const void* Y, const void* saved) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!Q || !K || !V || !Y) return LF_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Y)) return LF_EINVAL;
  if ((dwc_w && !aligned16(dwc_w)) || (saved && !aligned16(saved))) return LF_EINVAL;
  if (Y == Q || Y == K || Y == V) return LF_EINVAL;
  return LF_OK;
}

// The forward launch sequence on a validated call; ws holds at least fwd_ws(s).total bytes.
int fwd_launch(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w, void* Y,
               void* saved, void* ws, hipStream_t st) {
  const lf::Shape s = make_shape(p);
  const FwdWs w = fwd_ws(s);
  const bool wh = p->whiten == 1;

  float *L, *CQ, *CK, *We, *xs, *mu, *rstd, *S, *Praw, *alpha;
  if (saved) {
    const lf_saved_layout sl = saved_layout(s);
    L = at<float>(saved, sl.L);
    CQ = at<float>(saved, sl.CQ);
    CK = at<float>(saved, sl.CK);
    We = at<float>(saved, sl.We);
    xs = at<float>(saved, sl.xs);
    mu = at<float>(saved, sl.mu);
    rstd = at<float>(saved, sl.rstd);
    S = at<float>(saved, sl.S);
    Praw = at<float>(saved, sl.P);
    alpha = at<float>(saved, sl.alpha);
  } else {
    L = at<float>(ws, w.L);
    CQ = at<float>(ws, w.CQ);
    CK = at<float>(ws, w.CK);
    We = at<float>(ws, w.We);
    xs = nullptr;
    mu = at<float>(ws, w.mu);
    rstd = at<float>(ws, w.rstd);
    S = at<float>(ws, w.S);
    Praw = nullptr;
    alpha = at<float>(ws, w.alpha);
  }
  float* X = at<float>(ws, w.X);
  float* P = at<float>(ws, w.Pw);
  float* part = at<float>(ws, w.part);
  float* nstmp = at<float>(ws, w.nstmp);

  // C_Q is either materialised by the distance launch and read back by the output kernel, or recomputed inside the
  // output kernel from Q and the landmarks (the distance launch then forms C_K and W_eps only). The backward pass
  // and the whitening statistics need the stored C_Q; for inference the choice follows measurement
  // (lf::out_fused_pays).
  const bool fuse_cq = !saved && !wh && p->kernel != LF_KERNEL_GAUSS && lf::out_fused_pays(s);
  LF_TRY(lf::launch_landmark_pool(s, Q, L, st));
  // With whitening on this path the C_Q blocks leave per-tile partial statistics and the landmark mix finishes
  // them (no separate statistics pass over C_Q).
  float* wst = nullptr;
  if (p->kernel == LF_KERNEL_LAPLACE && !fuse_cq && lf::ns_laplace_supported(s)) {
    // C_K and W_eps first, then the solver beside S = C_K^T V and the C_Q pass in one launch.
    if (wh) wst = at<float>(ws, w.wst);
    LF_TRY(lf::launch_laplace(s, Q, K, L, CQ, CK, We, st, 6));
    LF_TRY(lf::launch_ns_laplace(s, We, X, xs, alpha, CK, V, S, Q, L, CQ, st, wst));
  } else {
    if (p->kernel == LF_KERNEL_GAUSS)
      LF_TRY(lf::launch_gauss(s, Q, K, L, CQ, CK, We, st));
    else
      LF_TRY(lf::launch_laplace(s, Q, K, L, CQ, CK, We, st, fuse_cq ? 6 : 7));
    if (wh) LF_TRY(lf::launch_whiten_stats(s, CQ, mu, rstd, st));
    // The solver stays on the caller's stream: a fork of it to the side stream, concurrent with the C_Q / C_K
    // launch and S = C_K^T V, measured slower on every shape (the event hand-off costs more than the solver hides).
    if (lf::ns_side_supported(s)) {
      // One launch: Newton-Schulz on G CUs, S = C_K^T V on the others.
      LF_TRY(lf::launch_ns_side(s, We, X, xs, alpha, CK, V, S, st));
    } else {
      LF_TRY(lf::launch_ns(s, We, X, xs, alpha, nullptr, nstmp, st));
      LF_TRY(lf::launch_ckv(s, CK, V, part, S, st));
    }
  }
  if (fuse_cq) {
    LF_TRY(lf::launch_mix(s, X, S, nullptr, P, nullptr, st));
    LF_TRY(lf::launch_out_fused(s, Q, L, P, V, dwc_w, Y, st));
  } else if (!saved && !wh && lf::out_mix_supported(s)) {
    // Inference: P = X S is formed inside the output kernel (no landmark-mix launch, P never stored).
    LF_TRY(lf::launch_out_mix(s, CQ, X, S, V, dwc_w, Y, st));
  } else {
    if (wst)
      LF_TRY(lf::launch_mix_whiten(s, X, S, wst, mu, rstd, P, Praw, st));
    else
      LF_TRY(lf::launch_mix(s, X, S, wh ? rstd : nullptr, P, Praw, st));
    LF_TRY(lf::launch_out(s, CQ, P, wh ? mu : nullptr, V, dwc_w, Y, st));
  }
  return LF_OK;
}

}  // namespace

extern "C" {

int lf_attn_fwd(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w, void* Y,
                void* saved, void* ws, size_t ws_bytes, lf_stream_t stream) {
  const int rc = validate_fwd(p, Q, K, V, dwc_w, Y, saved);
  if (rc != LF_OK) return rc;
  if (!ws || !aligned16(ws)) return LF_EINVAL;
  if (ws_bytes < fwd_ws(make_shape(p)).total) return LF_EWORKSPACE;
  return fwd_launch(p, Q, K, V, dwc_w, Y, saved, ws, reinterpret_cast<hipStream_t>(stream));
}

int lf_attn_fwd_noalloc(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                        void* Y, lf_stream_t stream) {
  static_assert(LF_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size keeps the workspace carve aligned");
  const int rc = validate_fwd(p, Q, K, V, dwc_w, Y, nullptr);
  if (rc != LF_OK) return rc;
  if (fwd_ws(make_shape(p)).total > static_cast<size_t>(LF_NOALLOC_SCRATCH_BYTES)) return LF_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (lf::noalloc_scratch(st, &scratch) != hipSuccess) return LF_EHIP;
  return fwd_launch(p, Q, K, V, dwc_w, Y, nullptr, scratch, st);
}

int lf_attn_bwd(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                const void* saved, const void* dY, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                lf_stream_t stream) {
  return lf_attn_bwd_ex(p, Q, K, V, dwc_w, saved, dY, dQ, dK, dV, nullptr, nullptr, 0, ws, ws_bytes, stream,
                        nullptr);
}

int lf_attn_bwd_ex(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                   const void* saved, const void* dY, void* dQ, void* dK, void* dV, float* d_dwc_w, float* d_lambda,
                   int flags, void* ws, size_t ws_bytes, lf_stream_t stream, const lf_aux_stream* aux) {
  if (flags & ~LF_BWD_EXACT_ALPHA) return LF_EINVAL;
  if (d_dwc_w && !aligned16(d_dwc_w)) return LF_EINVAL;
  lf::AuxStream side{};
  if (aux) {
    if (!aux->stream || !aux->fork || !aux->join || aux->fork == aux->join) return LF_EINVAL;
    side.s = reinterpret_cast<hipStream_t>(aux->stream);
    side.fork = reinterpret_cast<hipEvent_t>(aux->fork);
    side.join = reinterpret_cast<hipEvent_t>(aux->join);
    if (side.s == reinterpret_cast<hipStream_t>(stream)) return LF_EINVAL;
    // Both streams must belong to one device (the events are recorded on both).
    hipDevice_t da = 0, dc = 0;
    if (hipStreamGetDevice(side.s, &da) != hipSuccess ||
        hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dc) != hipSuccess || da != dc)
      return LF_EINVAL;
  }
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  const lf::Shape s = make_shape(p);
  if (s.m > 64 || s.d > 64 || p->kernel != LF_KERNEL_LAPLACE) return LF_EUNSUPPORTED;
  if (!Q || !K || !V || !saved || !dY || !dQ || !dK || !dV || !ws) return LF_EINVAL;
  const void* ptrs[] = {Q, K, V, saved, dY, dQ, dK, dV, ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LF_EINVAL;
  if (dwc_w && !aligned16(dwc_w)) return LF_EINVAL;
  if (ws_bytes < lf::bwd_ws_bytes(s)) return LF_EWORKSPACE;
  const lf_saved_layout sl = saved_layout(s);
  lf::SavedPtrs sp;
  const char* sb = static_cast<const char*>(saved);
  sp.L = reinterpret_cast<const float*>(sb + sl.L);
  sp.CQ = reinterpret_cast<const float*>(sb + sl.CQ);
  sp.CK = reinterpret_cast<const float*>(sb + sl.CK);
  sp.We = reinterpret_cast<const float*>(sb + sl.We);
  sp.xs = reinterpret_cast<const float*>(sb + sl.xs);
  sp.mu = reinterpret_cast<const float*>(sb + sl.mu);
  sp.rstd = reinterpret_cast<const float*>(sb + sl.rstd);
  sp.S = reinterpret_cast<const float*>(sb + sl.S);
  sp.P = reinterpret_cast<const float*>(sb + sl.P);
  sp.alpha = reinterpret_cast<const float*>(sb + sl.alpha);
  lf::BwdExtras ex;
  ex.d_dwc_w = d_dwc_w;
  ex.d_lambda = d_lambda;
  ex.exact_alpha = (flags & LF_BWD_EXACT_ALPHA) != 0;
  return hip_status(lf::launch_backward(s, p->whiten == 1, Q, K, V, dwc_w, sp, dY, dQ, dK, dV, ws,
                                        reinterpret_cast<hipStream_t>(stream), ex, aux ? &side : nullptr));
}

// ---- stage entry points ----

int lf_landmark_pool(const lf_attn_params* p, const void* Q, float* L, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!Q || !L || !aligned16(Q) || !aligned16(L)) return LF_EINVAL;
  return hip_status(lf::launch_landmark_pool(make_shape(p), Q, L, reinterpret_cast<hipStream_t>(stream)));
}

int lf_laplace_l1_exp(const lf_attn_params* p, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                      float* We, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  const void* ptrs[] = {Q, K, L, CQ, CK, We};
  for (const void* ptr : ptrs)
    if (!ptr || !aligned16(ptr)) return LF_EINVAL;
  return hip_status(lf::launch_laplace(make_shape(p), Q, K, L, CQ, CK, We, reinterpret_cast<hipStream_t>(stream)));
}

int lf_gauss_l2_exp(const lf_attn_params* p, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                    float* We, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  const void* ptrs[] = {Q, K, L, CQ, CK, We};
  for (const void* ptr : ptrs)
    if (!ptr || !aligned16(ptr)) return LF_EINVAL;
  return hip_status(lf::launch_gauss(make_shape(p), Q, K, L, CQ, CK, We, reinterpret_cast<hipStream_t>(stream)));
}

int lf_ns_pinv(const lf_attn_params* p, const float* We, float* X, float* xs, float* alpha_out, float* resid,
               void* ws, size_t ws_bytes, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!We || !X || !aligned16(We) || !aligned16(X)) return LF_EINVAL;
  if ((xs && !aligned16(xs)) || (alpha_out && !aligned16(alpha_out)) || (resid && !aligned16(resid)))
    return LF_EINVAL;
  const lf::Shape s = make_shape(p);
  const FwdWs w = fwd_ws(s);
  if (lf::ns_tmp_floats(s) > 0 && (!ws || ws_bytes < w.total)) return LF_EWORKSPACE;
  float* tmp = ws ? at<float>(ws, w.nstmp) : nullptr;
  return hip_status(lf::launch_ns(s, We, X, xs, alpha_out, resid, tmp, reinterpret_cast<hipStream_t>(stream)));
}

int lf_cg_pinv(const lf_attn_params* p, const float* We, float* X, float* resid, int32_t iters, lf_stream_t stream) {
  static_assert(LF_CG_ITERS_MAX == lf::kCgItersMax, "CG step limit of the header and the kernel differ");
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!We || !X || !aligned16(We) || !aligned16(X) || (resid && !aligned16(resid))) return LF_EINVAL;
  if (iters < 0 || iters > LF_CG_ITERS_MAX) return LF_EINVAL;
  const lf::Shape s = make_shape(p);
  if (!lf::cg_supported(s)) return LF_EUNSUPPORTED;
  return hip_status(lf::launch_cg(s, We, X, resid, iters, reinterpret_cast<hipStream_t>(stream)));
}

int lf_ckv_reduce(const lf_attn_params* p, const float* CK, const void* V, float* S, void* ws, size_t ws_bytes,
                  lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!CK || !V || !S || !aligned16(CK) || !aligned16(V) || !aligned16(S)) return LF_EINVAL;
  const lf::Shape s = make_shape(p);
  const FwdWs w = fwd_ws(s);
  if (!ws || ws_bytes < w.total) return LF_EWORKSPACE;
  return hip_status(lf::launch_ckv(s, CK, V, at<float>(ws, w.part), S, reinterpret_cast<hipStream_t>(stream)));
}

int lf_whiten_stats(const lf_attn_params* p, const float* CQ, float* mu, float* rstd, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!CQ || !mu || !rstd || !aligned16(CQ) || !aligned16(mu) || !aligned16(rstd)) return LF_EINVAL;
  if (!(p->whiten_eps > 0.f)) return LF_EINVAL;
  return hip_status(lf::launch_whiten_stats(make_shape(p), CQ, mu, rstd, reinterpret_cast<hipStream_t>(stream)));
}

int lf_landmark_mix(const lf_attn_params* p, const float* X, const float* S, const float* rstd, float* P,
                    lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!X || !S || !P || !aligned16(X) || !aligned16(S) || !aligned16(P)) return LF_EINVAL;
  if (rstd && !aligned16(rstd)) return LF_EINVAL;
  return hip_status(lf::launch_mix(make_shape(p), X, S, rstd, P, nullptr, reinterpret_cast<hipStream_t>(stream)));
}

int lf_out_gemm_dwc_fused(const lf_attn_params* p, const void* Q, const float* L, const float* P, const void* V,
                          const float* dwc_w, void* Y, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!Q || !L || !P || !V || !Y) return LF_EINVAL;
  if (!aligned16(Q) || !aligned16(L) || !aligned16(P) || !aligned16(V) || !aligned16(Y)) return LF_EINVAL;
  if (dwc_w && !aligned16(dwc_w)) return LF_EINVAL;
  if (p->kernel != LF_KERNEL_LAPLACE) return LF_EUNSUPPORTED;
  return hip_status(
      lf::launch_out_fused(make_shape(p), Q, L, P, V, dwc_w, Y, reinterpret_cast<hipStream_t>(stream)));
}

int lf_out_gemm_dwc(const lf_attn_params* p, const float* CQ, const float* P, const float* mu, const void* V,
                    const float* dwc_w, void* Y, lf_stream_t stream) {
  const int rc = validate(p);
  if (rc != LF_OK) return rc;
  if (!CQ || !P || !V || !Y || !aligned16(CQ) || !aligned16(P) || !aligned16(V) || !aligned16(Y)) return LF_EINVAL;
  if ((mu && !aligned16(mu)) || (dwc_w && !aligned16(dwc_w))) return LF_EINVAL;
  return hip_status(
      lf::launch_out(make_shape(p), CQ, P, mu, V, dwc_w, Y, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
