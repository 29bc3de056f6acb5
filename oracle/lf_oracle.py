"""fp64 CPU oracle for the LaplacianFormer attention block (forward and backward).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU library never calls it, and it shares no code with the GPU library: no kernels,
headers, helpers or constants.

What it computes
----------------
Citations name the page and the section on it:

  [note]  papernotes.org ICLR 2026 reading note "LaplacianFormer：用拉普拉斯核重新思考线性注意力".
          Sections: 研究背景与动机 (motivation, with the "core idea" paragraph), 整体框架 (framework, with the
          flowchart), 关键设计 1/2/3 (Design 1: injective normalisation, Design 2: Nystrom, Design 3:
          Newton-Schulz plus fused kernels).
  [abs]   the arXiv 2604.20368 abstract (shd-paper.top digest and fugumt.com page), which says the kernel and the
          solver have custom forward and backward implementations.

The block, per independent (batch, head) slice, in the pages' notation (all arithmetic float64):

  1. Landmarks: view the query tokens as their H x W spatial map and average-pool non-overlapping r x r blocks,
     giving m = (H/r)(W/r) landmark tokens [note, Design 2; flowchart node D].
  2. Laplacian kernel k(x, y) = exp(-||x - y||_1 / lambda) [note, motivation "core idea"; Design 2]. Cross-kernels
     C_Q[i, l] = k(q_i, L_l) and C_K[j, l] = k(k_j, L_l); landmark kernel W[l, l'] = k(L_l, L_l').
  3. W_eps = W + eps*I, then the Newton-Schulz pseudo-inverse with X_0 = alpha*W_eps^T and
     X_{k+1} = X_k (2I - W_eps X_k) [note, Design 3; flowchart node F].
  4. Optional diagonal whitening of the similarity vectors: every landmark column of C_Q is centred by its mean
     over the slice's N tokens and scaled by 1/sqrt(var + eps_w) [note, Design 1].
  5. Nystrom output Y_attn = A_hat * X_K * (C_K^T V) with A_hat = C_Q or its whitened form [note, Design 2;
     flowchart nodes E, G].
  6. Output Y = Y_attn + DWC(V): a depthwise 3x3 convolution of V adds local context [note, Design 1 and
     flowchart nodes H, I].

Readings where the pages are silent, ambiguous or wrong (each one is listed in the design notes):
  R1  landmarks come from Q and the same landmarks serve C_Q, C_K and W (Design 2 pools the query map).
  R2  cross form Y = C_Q X (C_K^T V); it equals the page's symmetric C W^+ C^T form when K = Q.
  R3  alpha = 1 / (||W_eps||_1 ||W_eps||_inf), computed after the eps shift. The page's 2/||W||_2 does not make
      ||I - alpha W W^T|| < 1 for a unit-diagonal W (the top eigenvalue gives 1 - 2||W||_2 <= -1); this alpha
      satisfies 0 < alpha*mu^2 <= 1 for every eigenvalue mu.
  R4  dk/dx = -(1/lambda) sign(x - y) k (the page drops the minus sign); dk/dy = +(1/lambda) sign(x - y) k.
  R5  sign(0) = 0.
  R6  alpha is treated as a constant in the backward pass, unless the exact gradient through alpha is asked for:
      then the adjoint of X_0 also flows through alpha = 1/(max column sum * max row sum) of |W_eps|, whose
      derivative is taken at the first maximising column and row (the maximum is a kink only at ties).
  R7  whitening: columns of C_Q only, statistics per slice over its N tokens, biased variance, no row
      centring and no +1/N term.
  R8  no row normalisation and no 1/sqrt(d) scale; lambda is the only scale.
  R9  non-overlapping r x r pooling with stride r; H and W divisible by r; tokens row-major n = y*W + x.
  R10 DWC is a 3x3 cross-correlation, stride 1, zero padding 1, no bias, one filter per channel h*d + c.
  R18 the Gaussian-kernel variant that the pages compare against (motivation: the Gaussian kernel decays with the
      squared l2 distance) is k(x, y) = exp(-||x - y||_2^2 / lambda): the same lambda slot, nothing else
      changed (same landmarks, eps shift, solver, whitening, DWC). Forward only.

Layouts: Q, K, V, Y, dY are [B, heads, N, d] float64; the DWC weight is [heads*d, 3, 3].
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass
class Params:
    B: int
    heads: int
    H: int
    W: int
    d: int
    r: int
    lam: float
    eps: float
    ns_iters: int
    whiten: bool = False
    whiten_eps: float = 1e-5
    kernel: str = "laplace"  # or "gauss" (reading R18)

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def m(self) -> int:
        return (self.H // self.r) * (self.W // self.r)


# ----------------------------------------------------------------------------------------------------------
# Step 1: landmarks by r x r average pooling of the query map  [note, Design 2; flowchart node D]
# ----------------------------------------------------------------------------------------------------------
def landmark_pool(q: np.ndarray, H: int, W: int, r: int) -> np.ndarray:
    """L[Y*(W/r) + X, c] = (1/r^2) * sum_{a,b < r} q[(Y*r + a)*W + (X*r + b), c]   (reading R9)."""
    N, d = q.shape
    assert N == H * W and H % r == 0 and W % r == 0
    grid = q.reshape(H // r, r, W // r, r, d)  # [Y, a, X, b, c]
    return grid.sum(axis=(1, 3)).reshape((H // r) * (W // r), d) / float(r * r)


# ----------------------------------------------------------------------------------------------------------
# Step 2: the Laplacian kernel  [note, motivation "core idea"; Design 2]
# ----------------------------------------------------------------------------------------------------------
def l1_distance(x: np.ndarray, y: np.ndarray, row_chunk: int = 512) -> np.ndarray:
    """D[i, l] = sum_c |x[i, c] - y[l, c]|, computed in row chunks to bound memory."""
    out = np.empty((x.shape[0], y.shape[0]), dtype=np.float64)
    for s in range(0, x.shape[0], row_chunk):
        xs = x[s:s + row_chunk]
        out[s:s + row_chunk] = np.abs(xs[:, None, :] - y[None, :, :]).sum(axis=2)
    return out


def laplacian_kernel(x: np.ndarray, y: np.ndarray, lam: float) -> np.ndarray:
    """K[i, l] = exp(-||x_i - y_l||_1 / lambda)."""
    return np.exp(-l1_distance(x, y) / lam)


# Gaussian-kernel variant  [note, motivation: the Gaussian kernel of earlier linear attentions decays with the
# squared l2 distance; key findings, first item: swapping that kernel for the Laplacian one; reading R18]
def sq_l2_distance(x: np.ndarray, y: np.ndarray, row_chunk: int = 512) -> np.ndarray:
    """D[i, l] = sum_c (x[i, c] - y[l, c])^2 from the differences themselves, in row chunks."""
    out = np.empty((x.shape[0], y.shape[0]), dtype=np.float64)
    for s in range(0, x.shape[0], row_chunk):
        diff = x[s:s + row_chunk][:, None, :] - y[None, :, :]
        out[s:s + row_chunk] = (diff * diff).sum(axis=2)
    return out


def gaussian_kernel(x: np.ndarray, y: np.ndarray, lam: float) -> np.ndarray:
    """K[i, l] = exp(-||x_i - y_l||_2^2 / lambda)."""
    return np.exp(-sq_l2_distance(x, y) / lam)


def kernel_of(p: "Params"):
    """The similarity kernel a parameter set names: Laplacian (the method) or Gaussian (the variant, R18)."""
    if p.kernel == "laplace":
        return laplacian_kernel
    if p.kernel == "gauss":
        return gaussian_kernel
    raise ValueError(f"unknown kernel {p.kernel!r}")


# ----------------------------------------------------------------------------------------------------------
# Step 3: eps shift and Newton-Schulz pseudo-inverse  [note, Design 3; flowchart node F]
# ----------------------------------------------------------------------------------------------------------
def ns_alpha(w: np.ndarray) -> float:
    """alpha = 1 / (||w||_1 * ||w||_inf): max absolute column sum times max absolute row sum (reading R3)."""
    norm_1 = np.abs(w).sum(axis=0).max()
    norm_inf = np.abs(w).sum(axis=1).max()
    return 1.0 / (norm_1 * norm_inf)


def newton_schulz(w_eps: np.ndarray, iters: int, alpha: Optional[float] = None):
    """X_0 = alpha * w_eps^T; X_{k+1} = X_k (2I - w_eps X_k), exactly `iters` times, no early exit.

    Returns (X_iters, [X_0, ..., X_iters], alpha). `alpha` may be forced (used by the finite-difference tests,
    which hold it fixed as the backward pass does).
    """
    m = w_eps.shape[0]
    if alpha is None:
        alpha = ns_alpha(w_eps)
    two_i = 2.0 * np.eye(m)
    x = alpha * w_eps.T
    xs = [x]
    for _ in range(iters):
        x = x @ (two_i - w_eps @ x)
        xs.append(x)
    return x, xs, alpha


# ----------------------------------------------------------------------------------------------------------
# Solver comparator: conjugate gradients for W_eps X = I  [note, Design 3 (the robustness claim against CG at a
# condition number of 50); ablation table, solver row; key findings, second item]
# ----------------------------------------------------------------------------------------------------------
def cg_pinv(w_eps: np.ndarray, iters: int):
    """Conjugate gradients for W_eps X = I. Column j is an independent CG solve of W_eps x = e_j from x = 0 with
    the textbook recurrences (residual r = b - W x, search direction p, step a = r.r / p.Wp, then
    p <- r' + (r'.r' / r.r) p). Returns X and, per iteration, the Frobenius norm of the residual W_eps X - I.
    A column whose residual is exactly zero stops."""
    m = w_eps.shape[0]
    X = np.zeros((m, m))
    R = np.eye(m)
    P = R.copy()
    rr = np.sum(R * R, axis=0)
    hist = []
    for _ in range(iters):
        Q = w_eps @ P
        pq = np.sum(P * Q, axis=0)
        a = np.where(rr > 0, rr / np.where(pq != 0, pq, 1.0), 0.0)
        X = X + P * a
        R = R - Q * a
        rr_new = np.sum(R * R, axis=0)
        beta = np.where(rr > 0, rr_new / np.where(rr > 0, rr, 1.0), 0.0)
        P = R + P * beta
        rr = rr_new
        hist.append(float(np.linalg.norm(w_eps @ X - np.eye(m))))
    return X, hist


# ----------------------------------------------------------------------------------------------------------
# Step 4: diagonal whitening of the similarity vectors  [note, Design 1]
# ----------------------------------------------------------------------------------------------------------
def whiten_columns(c: np.ndarray, eps_w: float):
    """A_hat[i, l] = (c[i, l] - mu_l) / sqrt(var_l + eps_w); mu, var over the N rows (biased), reading R7."""
    mu = c.mean(axis=0)
    var = ((c - mu) ** 2).mean(axis=0)
    rstd = 1.0 / np.sqrt(var + eps_w)
    return (c - mu) * rstd, mu, rstd


# ----------------------------------------------------------------------------------------------------------
# Step 6: depthwise 3x3 convolution of V  [note, Design 1; flowchart nodes H, I]
# ----------------------------------------------------------------------------------------------------------
def dwc(v: np.ndarray, w: np.ndarray, H: int, W: int) -> np.ndarray:
    """out[(y,x), c] = sum_{a,b in {-1,0,1}} w[c, a+1, b+1] * v[(y+a, x+b), c], zero outside the grid (R10)."""
    N, d = v.shape
    grid = np.zeros((H + 2, W + 2, d))
    grid[1:H + 1, 1:W + 1] = v.reshape(H, W, d)
    out = np.zeros((H, W, d))
    for a in range(3):
        for b in range(3):
            out += w[:, a, b] * grid[a:a + H, b:b + W]
    return out.reshape(N, d)


def dwc_weight_grad(v: np.ndarray, dy: np.ndarray, H: int, W: int) -> np.ndarray:
    """Gradient of <dy, dwc(v, w)> with respect to w: the DWC is linear in w and its tap (a, b) of channel c
    multiplies v[(y+a-1, x+b-1), c] into out[(y,x), c], so the gradient is the sum over the grid of
    dy[(y,x), c] * v[(y+a-1, x+b-1), c] (zero outside the grid). Returns [d, 3, 3]."""
    N, d = v.shape
    grid = np.zeros((H + 2, W + 2, d))
    grid[1:H + 1, 1:W + 1] = v.reshape(H, W, d)
    g = dy.reshape(H, W, d)
    out = np.zeros((d, 3, 3))
    for a in range(3):
        for b in range(3):
            out[:, a, b] = np.sum(g * grid[a:a + H, b:b + W], axis=(0, 1))
    return out


def dwc_adjoint(u: np.ndarray, w: np.ndarray, H: int, W: int) -> np.ndarray:
    """Adjoint of `dwc` in V: out[(y,x), c] = sum_{a,b} w[c, a+1, b+1] * u[(y-a, x-b), c] (zero outside)."""
    N, d = u.shape
    grid = np.zeros((H + 2, W + 2, d))
    grid[1:H + 1, 1:W + 1] = u.reshape(H, W, d)
    out = np.zeros((H, W, d))
    for a in range(3):
        for b in range(3):
            out += w[:, a, b] * grid[2 - a:2 - a + H, 2 - b:2 - b + W]
    return out.reshape(N, d)


# ----------------------------------------------------------------------------------------------------------
# Whole block, one slice
# ----------------------------------------------------------------------------------------------------------
def forward_slice(q, k, v, w_dwc, p: Params, alpha: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Forward of one (batch, head) slice. w_dwc is this head's [d, 3, 3] filter bank or None."""
    L = landmark_pool(q, p.H, p.W, p.r)
    kern = kernel_of(p)
    CQ = kern(q, L, p.lam)
    CK = kern(k, L, p.lam)
    Wm = kern(L, L, p.lam)
    We = Wm + p.eps * np.eye(L.shape[0])
    X, xs, alpha = newton_schulz(We, p.ns_iters, alpha)
    if p.whiten:
        A, mu, rstd = whiten_columns(CQ, p.whiten_eps)
    else:
        A, mu, rstd = CQ, None, None
    S = CK.T @ v
    P = X @ S
    Yattn = A @ P
    D = dwc(v, w_dwc, p.H, p.W) if w_dwc is not None else np.zeros_like(Yattn)
    resid = np.linalg.norm(We @ X - np.eye(L.shape[0]))
    return dict(L=L, CQ=CQ, CK=CK, W=Wm, We=We, X=X, xs=xs, alpha=alpha, A=A, mu=mu, rstd=rstd, S=S, P=P,
                Yattn=Yattn, D=D, Y=Yattn + D, resid=resid)


def _sign(x: np.ndarray) -> np.ndarray:
    return np.sign(x)  # sign(0) = 0 (reading R5)


def backward_slice(q, k, v, w_dwc, dy, p: Params, fwd: Optional[Dict] = None,
                   alpha: Optional[float] = None, exact_alpha: bool = False) -> Dict[str, np.ndarray]:
    """Gradients of <dy, Y> with respect to q, k, v, the DWC weights and lambda for one slice.

    Chain rule through the forward steps, last step first. The kernel derivative is reading R4:
    d/dx exp(-||x-y||_1/lambda) = -(1/lambda) sign(x - y) exp(...), and +(1/lambda) sign(x - y) exp(...) in y.
    In lambda: d/dlambda exp(-D/lambda) = exp(-D/lambda) D / lambda^2 for the distance D. alpha is held constant
    (reading R6) unless exact_alpha is set. The Gaussian-kernel variant has no backward here (reading R18).
    """
    if p.kernel != "laplace":
        raise NotImplementedError("the Gaussian-kernel variant is forward only")
    f = fwd if fwd is not None else forward_slice(q, k, v, w_dwc, p, alpha)
    A, P, S, X, xs, We = f["A"], f["P"], f["S"], f["X"], f["xs"], f["We"]
    CQ, CK, Wm, L = f["CQ"], f["CK"], f["W"], f["L"]
    lam = p.lam
    N = q.shape[0]

    # Y = A P + DWC(V)
    dV = dwc_adjoint(dy, w_dwc, p.H, p.W) if w_dwc is not None else np.zeros_like(v)
    dA = dy @ P.T
    dP = A.T @ dy
    # P = X S
    dX = dP @ S.T
    dS = X.T @ dP
    # S = CK^T V
    dV = dV + CK @ dS
    dCK = v @ dS.T
    # A = whiten(CQ) (batch-norm style backward over the N rows of each column) or A = CQ
    if p.whiten:
        rstd = f["rstd"]
        dCQ = rstd * (dA - dA.mean(axis=0) - A * (dA * A).mean(axis=0))
    else:
        dCQ = dA
    # Newton-Schulz, reverse order: X_{k+1} = 2 X_k - X_k We X_k
    G = dX
    dWe = np.zeros_like(We)
    for kk in range(p.ns_iters - 1, -1, -1):
        Xk = xs[kk]
        dWe += -Xk.T @ G @ Xk.T
        G = 2.0 * G - G @ (We @ Xk).T - (Xk @ We).T @ G
    dWe += f["alpha"] * G.T  # X_0 = alpha We^T
    if exact_alpha:
        # alpha = 1 / (c r), c = max_j sum_i |We_ij|, r = max_i sum_j |We_ij|; d alpha = <G, We^T> (X_0 = alpha We^T)
        aw = np.abs(We)
        colsum, rowsum = aw.sum(axis=0), aw.sum(axis=1)
        jc, ir = int(np.argmax(colsum)), int(np.argmax(rowsum))
        a = f["alpha"]
        dalpha = float(np.sum(G * We.T))
        dadW = np.zeros_like(We)
        dadW[:, jc] -= a / colsum[jc] * np.sign(We[:, jc])
        dadW[ir, :] -= a / rowsum[ir] * np.sign(We[ir, :])
        dWe += dalpha * dadW
    # Kernel entries -> points. The eps diagonal carries no gradient to L.
    Gq = dCQ * CQ / lam
    Gk = dCK * CK / lam
    Gw = dWe * Wm / lam
    sq = _sign(q[:, None, :] - L[None, :, :])  # [N, m, d]
    sk = _sign(k[:, None, :] - L[None, :, :])
    sl = _sign(L[:, None, :] - L[None, :, :])  # [m, m, d]
    dQ = -np.einsum("il,ilc->ic", Gq, sq)
    dK = -np.einsum("jl,jlc->jc", Gk, sk)
    dL = (np.einsum("il,ilc->lc", Gq, sq) + np.einsum("jl,jlc->lc", Gk, sk)
          - np.einsum("ab,abc->ac", Gw + Gw.T, sl))
    # Landmarks are block means of q: each query token receives its block's dL / r^2.
    Wr = p.W // p.r
    ys, xs_ = np.divmod(np.arange(N), p.W)
    owner = (ys // p.r) * Wr + (xs_ // p.r)
    dQ = dQ + dL[owner] / float(p.r * p.r)
    # lambda: every kernel entry k = exp(-D/lambda) moves by k D / lambda^2 (the eps diagonal does not depend on it)
    dlam = float(np.sum(dCQ * CQ * l1_distance(q, L)) + np.sum(dCK * CK * l1_distance(k, L))
                 + np.sum(dWe * Wm * l1_distance(L, L))) / (lam * lam)
    d_dwc = dwc_weight_grad(v, dy, p.H, p.W)
    return dict(dQ=dQ, dK=dK, dV=dV, dL=dL, dWe=dWe, dCQ=dCQ, dCK=dCK, dA=dA, dP=dP, dS=dS, dX=dX, dlam=dlam,
                d_dwc=d_dwc)


# ----------------------------------------------------------------------------------------------------------
# Batched wrappers over the B*heads independent slices
# ----------------------------------------------------------------------------------------------------------
def _head_w(w_dwc, h, d):
    return None if w_dwc is None else w_dwc[h * d:(h + 1) * d]


def forward(Q, K, V, w_dwc, p: Params, keep: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """Forward over [B, heads, N, d] inputs. Returns stacked per-slice results for the keys in `keep`."""
    keep = keep or ["Y", "Yattn", "L", "CQ", "CK", "We", "X", "S", "P", "mu", "rstd", "resid"]
    out: Dict[str, list] = {key: [] for key in keep}
    for b in range(p.B):
        for h in range(p.heads):
            f = forward_slice(Q[b, h], K[b, h], V[b, h], _head_w(w_dwc, h, p.d), p)
            for key in keep:
                out[key].append(f[key])
    res = {}
    for key, vals in out.items():
        if vals and vals[0] is None:
            res[key] = None
            continue
        arr = np.stack([np.asarray(x) for x in vals])
        res[key] = arr.reshape((p.B, p.heads) + arr.shape[1:])
    return res


def backward(Q, K, V, w_dwc, dY, p: Params, exact_alpha: bool = False) -> Dict[str, np.ndarray]:
    """dQ, dK, dV over [B, heads, N, d] inputs; the DWC weight gradient [heads*d, 3, 3] (summed over the batch)
    and the lambda gradient (summed over every slice)."""
    dQ = np.empty_like(Q)
    dK = np.empty_like(K)
    dV = np.empty_like(V)
    d_dwc = np.zeros((p.heads * p.d, 3, 3))
    dlam = 0.0
    for b in range(p.B):
        for h in range(p.heads):
            g = backward_slice(Q[b, h], K[b, h], V[b, h], _head_w(w_dwc, h, p.d), dY[b, h], p,
                               exact_alpha=exact_alpha)
            dQ[b, h], dK[b, h], dV[b, h] = g["dQ"], g["dK"], g["dV"]
            d_dwc[h * p.d:(h + 1) * p.d] += g["d_dwc"]
            dlam += g["dlam"]
    return dict(dQ=dQ, dK=dK, dV=dV, d_dwc=d_dwc, dlam=dlam)
