/*
 * lf_attn.h — C ABI of liblf_attn.so, the LaplacianFormer attention block on AMD Instinct MI355X (gfx950).
 *
 * Sources. The operation is defined by the papernotes.org ICLR 2026 reading note
 * "LaplacianFormer：用拉普拉斯核重新思考线性注意力" (cited below as [note]). Its sections used here are:
 *   - motivation, "core idea" paragraph: the Laplacian kernel k(x,y) = exp(-||x-y||_1/lambda) and its gradient;
 *   - framework: the flowchart Q,K,V -> kernel -> whitening -> landmarks -> Nystrom -> Newton-Schulz -> ZV + DWC(V);
 *   - Design 1: injective normalisation by diagonal whitening, output = ZV + DWC(V);
 *   - Design 2: Nystrom approximation C W^+ C^T with landmarks from r x r average pooling of the query map;
 *   - Design 3: W + eps I, Newton-Schulz X_0 = alpha W^T, X_{k+1} = X_k (2I - W X_k), fused kernels.
 * The arXiv 2604.20368 abstract ([abs]) adds that the kernel and the solver have forward and backward passes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Shapes:   G = B*heads independent slices; N = H*W tokens, row-major (token n = y*W + x);
 *            m = (H/r)*(W/r) landmarks, landmark index l = Y*(W/r) + X for the r x r block at (Y, X).
 *  Tensors:  Q, K, V, Y, dY, dQ, dK, dV are [B][heads][N][d], contiguous, in params->dtype (float32 or the bf16
 *            bit pattern). Intermediates are float32: L [G][m][d]; C_Q and C_K landmark-major [G][m][N] (element
 *            [g][l][i] is C[i][l] of the formulas); W_eps and X [G][m][m]; S and P [G][m][d]; mu and rstd [G][m].
 *            The DWC weight is float32 [heads*d][3][3].
 *  Pointers: every pointer is a device pointer owned by the caller, 16-byte aligned. The library never allocates
 *            or frees memory, never synchronises and holds no state between calls: no stream, event or buffer of
 *            its own. Work is enqueued on `stream` (a hipStream_t; NULL means the null stream) and the call returns
 *            as soon as it is enqueued. Only lf_attn_bwd_ex can spread its work over a second stream, and only one
 *            the caller lends it (lf_aux_stream). A call enqueues kernels (and, for lf_attn_bwd_ex with a lent
 *            stream, event records and waits) and nothing else: no copy, clear or synchronisation, so it can be
 *            captured in a HIP graph (the lent stream joins the capture through its events) and replayed.
 *  Errors:   every entry point returns LF_OK (0) or a negative code. Parameters, pointers and workspace sizes are
 *            checked on the host before anything is launched; on an error nothing is launched. LF_EHIP reports a
 *            failed launch (hipGetLastError). Nothing throws across this ABI. Calls are reentrant; calls that
 *            share output or workspace buffers must be ordered by the caller.
 *  Readings: where the pages are silent the library takes these readings: landmarks come from Q and serve C_Q,
 *            C_K and W; the cross form Y = A_hat X (C_K^T V); alpha = 1/(||W_eps||_1 ||W_eps||_inf); sign(0) = 0;
 *            alpha is held constant in the backward pass; whitening centres and scales the landmark columns of
 *            C_Q over the slice's N tokens (biased variance); DWC is a 3x3 zero-padded cross-correlation, no bias.
 */
#ifndef LF_ATTN_H
#define LF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* lf_stream_t; /* same type as hipStream_t */
typedef struct ihipEvent_t* lf_event_t;   /* same type as hipEvent_t */

enum lf_status {
  LF_OK = 0,
  LF_EINVAL = -1,       /* bad shape, parameter, null or misaligned pointer */
  LF_EWORKSPACE = -2,   /* workspace smaller than lf_attn_query reports */
  LF_EUNSUPPORTED = -3, /* valid but not implemented: d not in {16,32,64,128}, m > LF_M_MAX, backward with m or d > 64 */
  LF_EHIP = -4          /* a kernel launch failed */
};

enum lf_dtype { LF_F32 = 0, LF_BF16 = 1 };

/* Similarity kernel of the block. LF_KERNEL_LAPLACE is the method: k(x,y) = exp(-||x-y||_1/lambda) ([note]
 * motivation, "core idea"). LF_KERNEL_GAUSS is the kernel the note sets it against (its motivation: the Gaussian
 * kernel of earlier linear attentions decays with the squared l2 distance; its key findings: replacing it by the
 * Laplacian one): k(x,y) = exp(-||x-y||_2^2/lambda), with every other step unchanged. The Gaussian variant is
 * forward only (backward and the fused output stage return LF_EUNSUPPORTED). */
enum lf_kernel { LF_KERNEL_LAPLACE = 0, LF_KERNEL_GAUSS = 1 };

#define LF_M_MAX 256
#define LF_NS_ITERS_MAX 64

typedef struct lf_attn_params {
  int32_t B, heads, H, W, d; /* N = H*W */
  int32_t r;                 /* pooling window and stride; H % r == 0 and W % r == 0 */
  float lambda;              /* kernel scale, > 0 ([note] ablation default 4) */
  float eps;                 /* >= 0, added to the diagonal of W ([note] Design 3) */
  int32_t ns_iters;          /* 0..LF_NS_ITERS_MAX Newton-Schulz steps, no early exit (0 gives X = alpha W_eps^T) */
  int32_t whiten;            /* 0 or 1: diagonal whitening of C_Q's landmark columns ([note] Design 1) */
  float whiten_eps;          /* > 0, added to the column variance when whiten = 1 */
  int32_t dtype;             /* LF_F32 or LF_BF16: type of Q, K, V, Y, dY, dQ, dK, dV */
  int32_t kernel;            /* LF_KERNEL_LAPLACE (0, a zero-initialised struct) or LF_KERNEL_GAUSS: the kernel
                                lf_attn_fwd uses for C_Q, C_K and W */
} lf_attn_params;

/* Byte offsets of the intermediates inside the `saved` buffer written by lf_attn_fwd (each 256-byte aligned).
 * xs holds X_0 .. X_{ns_iters} ([G][ns_iters+1][m][m]); alpha is float32 [G]. mu and rstd are written only
 * when whiten = 1. The layout is fixed for given params; lf_attn_bwd reads it. */
typedef struct lf_saved_layout {
  size_t L, CQ, CK, We, xs, mu, rstd, S, P, alpha, total;
} lf_saved_layout;

/* Sizes, in bytes, of the forward workspace, the saved buffer and the backward workspace for `p`.
 * Any pointer may be NULL. Host-only; launches nothing. Returns LF_EINVAL / LF_EUNSUPPORTED for bad params. */
int lf_attn_query(const lf_attn_params* p, size_t* fwd_ws_bytes, size_t* saved_bytes, size_t* bwd_ws_bytes);

/* Layout of the saved buffer (host-only). */
int lf_attn_saved_layout(const lf_attn_params* p, lf_saved_layout* out);

/* Forward pass ([note] framework flowchart; Designs 1-3), k the kernel p->kernel names:
 *   L = pool_r(Q); C_Q = k(Q, L); C_K = k(K, L); W_eps = k(L, L) + eps I; X = NS^{ns_iters}(W_eps);
 *   A_hat = C_Q, or its whitened form when whiten = 1; Y = A_hat X (C_K^T V) + DWC(V).
 * dwc_w: [heads*d][3][3] float32, or NULL for the attention branch alone (Y = A_hat X C_K^T V).
 * saved: NULL, or a buffer of lf_attn_query's saved_bytes that receives the intermediates for lf_attn_bwd.
 * ws/ws_bytes: device workspace of at least fwd_ws_bytes. Y must not alias Q, K or V. */
int lf_attn_fwd(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w, void* Y,
                void* saved, void* ws, size_t ws_bytes, lf_stream_t stream);

/* The same forward pass (saved = NULL) for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Instead of a workspace argument it uses a static device
 * array of the library's, LF_NOALLOC_SCRATCH_BYTES (128 MiB), which every GPU the library runs on holds from the
 * first launch on it until the process ends; its address on a device is looked up once, on the first call for that
 * device. The call allocates nothing (no hipMalloc, no library that does) and launches the kernels lf_attn_fwd
 * launches, so Y is bitwise lf_attn_fwd's. Every call on one GPU shares that GPU's array: calls on one device that
 * may overlap in time (other streams, other host threads) race, and the caller must order them. No kernel reads
 * the array before the same call has written it, so nothing in it needs clearing between calls. Shapes whose
 * forward workspace (lf_attn_query's fwd_ws_bytes) exceeds the array return LF_EWORKSPACE before anything is
 * launched. Other arguments, rules and errors as lf_attn_fwd; LF_EHIP if the array's address cannot be found. */
#define LF_NOALLOC_SCRATCH_BYTES (128 * 1024 * 1024)
int lf_attn_fwd_noalloc(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                        void* Y, lf_stream_t stream);

/* Backward pass of <dY, Y> with respect to Q, K and V ([abs]: forward and backward; [note] motivation "core idea"
 * for the kernel gradient, with the sign read as d/dx exp(-||x-y||_1/lambda) = -(1/lambda) sign(x-y) k).
 * saved: the buffer filled by lf_attn_fwd with the same params and inputs. ws: at least bwd_ws_bytes.
 * dQ, dK, dV are overwritten. Every launch goes to `stream`. Supports m <= 64, d <= 64 and the Laplacian kernel
 * (LF_EUNSUPPORTED otherwise). */
int lf_attn_bwd(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                const void* saved, const void* dY, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                lf_stream_t stream);

/* A second stream lent by the caller to lf_attn_bwd_ex, with two events of the caller's (create them with
 * hipEventDisableTiming). Parts of the call's work that do not depend on each other run on `stream` after an
 * event recorded on the call's stream (`fork`, recorded twice per call: at its start and after the first small
 * products); the call's stream then waits on `join`, recorded after those parts,
 * so everything the call does is complete when work enqueued on the call's stream after it starts. The stream must
 * be another stream than the call's, on the same device (LF_EINVAL otherwise). The library keeps none of these
 * handles after the call returns; calls that lend the same lf_aux_stream must be ordered by the caller. */
typedef struct lf_aux_stream {
  lf_stream_t stream;
  lf_event_t fork, join;
} lf_aux_stream;

/* The training op's full set of gradients: everything lf_attn_bwd writes, plus, each optional (NULL skips it):
 *   d_dwc_w: [heads*d][3][3] float32, the gradient of <dY, Y> with respect to the DWC weights, summed over the
 *            batch ([note] Design 1: Y = ... + DWC(V), which is linear in the weights);
 *   d_lambda: one float32, the gradient with respect to lambda, summed over every slice (each kernel entry
 *            k = exp(-D/lambda) moves by k D / lambda^2; [note] motivation "core idea" for the kernel).
 * flags: LF_BWD_EXACT_ALPHA takes the gradient through the Newton-Schulz start alpha = 1/(||W_eps||_1 ||W_eps||_inf)
 *        ([note] Design 3 for X_0 = alpha W_eps^T), differentiated at the first largest column and row sum;
 *        without it alpha is held constant as in lf_attn_bwd. Other bits: LF_EINVAL.
 * aux:   NULL runs everything on `stream` (as lf_attn_bwd does), or a lent second stream (lf_aux_stream): the
 *        reverse Newton-Schulz chain, the landmark-matrix terms of dL and of the lambda gradient, and the DWC
 *        weight gradient then overlap the first small products, the row gradients and the sign reductions (two
 *        forks, one join).
 * Same saved buffer, workspace (bwd_ws_bytes), alignment and errors as lf_attn_bwd; d_dwc_w is 16-byte aligned. */
#define LF_BWD_EXACT_ALPHA 1
int lf_attn_bwd_ex(const lf_attn_params* p, const void* Q, const void* K, const void* V, const float* dwc_w,
                   const void* saved, const void* dY, void* dQ, void* dK, void* dV, float* d_dwc_w, float* d_lambda,
                   int flags, void* ws, size_t ws_bytes, lf_stream_t stream, const lf_aux_stream* aux);

/* Static description of a status code. */
const char* lf_strerror(int code);

/* ---- Stage entry points: each step of the forward pass on its own, same conventions as above. ---- */

/* L[g][l][c] = (1/r^2) sum_{a,b<r} Q[g][(Y r + a) W + X r + b][c]   ([note] Design 2: r x r average pooling). */
int lf_landmark_pool(const lf_attn_params* p, const void* Q, float* L, lf_stream_t stream);

/* C_Q[g][l][i] = exp(-sum_c |Q[g][i][c] - L[g][l][c]| / lambda) (landmark-major); C_K likewise with K;
 * W_eps[g][l][l'] = exp(-||L_l - L_l'||_1 / lambda) + eps [l == l']   ([note] motivation; Designs 2 and 3). */
int lf_laplace_l1_exp(const lf_attn_params* p, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                      float* We, lf_stream_t stream);

/* The Gaussian-kernel variant of the same stage (see lf_kernel): C_Q[g][l][i] = exp(-||Q[g][i] - L[g][l]||_2^2 /
 * lambda) (landmark-major), C_K likewise with K, W_eps[g][l][l'] = exp(-||L_l - L_l'||_2^2 / lambda) + eps [l == l'].
 * C_Q and C_K come from ||x||^2 + ||l||^2 - 2 x.l (fp32 MFMA for x.l, clamped at 0); W_eps from the differences,
 * so it is exactly symmetric with a unit diagonal before the shift. Computes the Gaussian kernel whatever
 * p->kernel holds; same layouts, pointer rules and errors as lf_laplace_l1_exp. */
int lf_gauss_l2_exp(const lf_attn_params* p, const void* Q, const void* K, const float* L, float* CQ, float* CK,
                    float* We, lf_stream_t stream);

/* Newton-Schulz pseudo-inverse ([note] Design 3): alpha = 1/(||W_eps||_1 ||W_eps||_inf), X_0 = alpha W_eps^T,
 * X_{k+1} = X_k (2I - W_eps X_k) for p->ns_iters steps. X: [G][m][m] receives X_{ns_iters}.
 * xs: NULL or [G][ns_iters+1][m][m] receiving X_0..X_{ns_iters}; alpha_out: NULL or [G];
 * resid: NULL or [G] receiving ||W_eps X - I||_F. ws: at least fwd_ws_bytes. */
int lf_ns_pinv(const lf_attn_params* p, const float* We, float* X, float* xs, float* alpha_out, float* resid,
               void* ws, size_t ws_bytes, lf_stream_t stream);

/* S[g][l][c] = sum_i C_K[g][l][i] V[g][i][c]: the "K^T V first" association of linear attention, as a
 * deterministic split-N reduction ([note] motivation; Design 2). ws: at least fwd_ws_bytes. */
int lf_ckv_reduce(const lf_attn_params* p, const float* CK, const void* V, float* S, void* ws, size_t ws_bytes,
                  lf_stream_t stream);

/* Diagonal whitening statistics of C_Q ([note] Design 1): mu[g][l] = mean_i C_Q[g][l][i],
 * rstd[g][l] = 1/sqrt(mean_i (C_Q[g][l][i] - mu)^2 + whiten_eps). */
int lf_whiten_stats(const lf_attn_params* p, const float* CQ, float* mu, float* rstd, lf_stream_t stream);

/* P[g][l][c] = rstd[g][l] * sum_k X[g][l][k] S[g][k][c]; rstd may be NULL (then 1). */
int lf_landmark_mix(const lf_attn_params* p, const float* X, const float* S, const float* rstd, float* P,
                    lf_stream_t stream);

/* Y[g][i][c] = sum_l C_Q[g][l][i] P[g][l][c] - sum_l mu[g][l] P[g][l][c] + DWC(V)[g][i][c]
 * ([note] Design 1 and flowchart nodes G, H, I). mu may be NULL (no whitening bias); dwc_w may be NULL. */
int lf_out_gemm_dwc(const lf_attn_params* p, const float* CQ, const float* P, const float* mu, const void* V,
                    const float* dwc_w, void* Y, lf_stream_t stream);

/* The same output without a materialised C_Q (no whitening): every 8 x 8 token tile computes its C_Q block
 * exp(-||q_i - l||_1 / lambda) from Q [B][heads][N][d] (the dtype of p) and the landmarks L [G][m][d] fp32, then
 * Y = C_Q P + DWC(V). Distance fused with the product, as the output stage of [note] Design 3 suggests to save
 * memory traffic. Same conventions and errors as lf_out_gemm_dwc; p->kernel must be LF_KERNEL_LAPLACE
 * (LF_EUNSUPPORTED otherwise). */
int lf_out_gemm_dwc_fused(const lf_attn_params* p, const void* Q, const float* L, const float* P, const void* V,
                          const float* dwc_w, void* Y, lf_stream_t stream);

/* Conjugate gradients for W_eps X = I: the solver that [note] Design 3 (and the solver row of its ablation table)
 * finds less robust than Newton-Schulz at a condition number of 50, provided to measure that claim. Column j of
 * X[g] is the CG solve of W_eps[g] x = e_j from x = 0: r = e_j, p = r; each step a = r.r / p.(W p), x += a p,
 * r -= a W p, p = r + (r'.r' / r.r) p. `iters` steps (0..LF_CG_ITERS_MAX), no early exit; a column whose r.r is
 * exactly 0 holds still. We: [G][m][m] float32, meant to be symmetric positive definite (not checked); X: [G][m][m]
 * float32 output. resid: NULL or [G][iters] float32 receiving ||W_eps X_k - I||_F after steps k = 1..iters,
 * formed from X_k itself (a second product per step). p is validated as for every entry point; only its G and m
 * are used, and m > 64 gives LF_EUNSUPPORTED. */
#define LF_CG_ITERS_MAX 256
int lf_cg_pinv(const lf_attn_params* p, const float* We, float* X, float* resid, int32_t iters, lf_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LF_ATTN_H */
