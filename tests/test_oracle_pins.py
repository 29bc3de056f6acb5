"""Pins for the fp64 oracle: every check compares it with something other than itself.

The checks are brute force on tiny inputs, closed forms, invariants, special cases that reduce to a library
routine, hand-worked fixtures (tests/golden) and finite differences. Each one is chosen so that a plausible slip in
the oracle fails it: a dropped term, a wrong sign or index, or a transposed operand. No value here comes from the
GPU library.
"""

import json
import math
import os

import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from laplacian_nystr_vit_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ev(expr, **env):
    scope = {"exp": math.exp, "__builtins__": {}}
    scope.update(env)
    return float(eval(expr, scope))


def _params(wl, **kw):
    p = O.Params(B=wl.B, heads=wl.heads, H=wl.H, W=wl.W, d=wl.d, r=wl.r, lam=wl.lam, eps=wl.eps,
                 ns_iters=wl.ns_iters, whiten=wl.whiten, whiten_eps=wl.whiten_eps, kernel=wl.kernel)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------------------------- pooling
def test_pool_bruteforce_loops():
    H, W, r, d = 4, 6, 2, 3
    q = _rng(1).standard_normal((H * W, d))
    L = O.landmark_pool(q, H, W, r)
    Wr = W // r
    for Y in range(H // r):
        for X in range(Wr):
            for c in range(d):
                vals = [q[(Y * r + a) * W + (X * r + b), c] for a in range(r) for b in range(r)]
                assert abs(L[Y * Wr + X, c] - math.fsum(vals) / (r * r)) < 1e-15


def test_pool_r1_is_identity_and_mean_preserved():
    q = _rng(2).standard_normal((8 * 8, 5))
    assert np.array_equal(O.landmark_pool(q, 8, 8, 1), q)
    L = O.landmark_pool(q, 8, 8, 4)
    assert np.allclose(L.mean(axis=0), q.mean(axis=0), atol=1e-15)


# ----------------------------------------------------------------------------------------------- kernel
def test_laplacian_kernel_bruteforce():
    rng = _rng(3)
    x, y, lam = rng.standard_normal((7, 5)), rng.standard_normal((4, 5)), 4.0
    K = O.laplacian_kernel(x, y, lam)
    for i in range(7):
        for l in range(4):
            ref = math.exp(-math.fsum(abs(x[i, c] - y[l, c]) for c in range(5)) / lam)
            assert abs(K[i, l] - ref) <= 1e-15 * ref + 1e-300


def test_kernel_identity_symmetry_scale():
    rng = _rng(4)
    x = rng.standard_normal((6, 8))
    Kxx = O.laplacian_kernel(x, x, 2.0)
    assert np.allclose(np.diag(Kxx), 1.0, atol=0, rtol=0)
    assert np.array_equal(Kxx, Kxx.T)
    y = rng.standard_normal((3, 8))
    # k(s x, s y; s lambda) = k(x, y; lambda)
    assert np.allclose(O.laplacian_kernel(3 * x, 3 * y, 6.0), O.laplacian_kernel(x, y, 2.0), rtol=1e-14)


def test_translation_invariance_of_block():
    """Shifting Q and K by one vector shifts L with them and leaves C_Q, C_K, W and Y_attn unchanged."""
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=5)
    p = _params(wl)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    shift = _rng(6).standard_normal(wl.d)
    f0 = O.forward_slice(q, k, v, None, p)
    f1 = O.forward_slice(q + shift, k + shift, v, None, p)
    for key in ("CQ", "CK", "We", "Yattn"):
        assert np.allclose(f0[key], f1[key], rtol=1e-12, atol=1e-14), key


def test_landmark_kernel_strictly_positive_definite():
    """The L1 Laplacian kernel is a product of 1-D Laplace kernels (positive Cauchy spectral density): W is PD."""
    for seed in range(3):
        L = 0.5 * _rng(seed).standard_t(3, size=(49, 64))
        W = O.laplacian_kernel(L, L, 4.0)
        assert np.array_equal(W, W.T)
        assert np.linalg.eigvalsh(W).min() > 0


def test_golden_hand_grid_m1():
    g = _load("hand_grid2x2_m1.json")
    pr = g["params"]
    p = O.Params(B=1, heads=1, H=pr["H"], W=pr["W"], d=pr["d"], r=pr["r"], lam=pr["lam"], eps=pr["eps"],
                 ns_iters=pr["ns_iters"])
    f = O.forward_slice(np.array(g["Q"], float), np.array(g["K"], float), np.array(g["V"], float), None, p)
    env = dict(eps=pr["eps"])
    ex = g["expected"]
    for key in ("L", "CQ", "CK", "X", "S"):
        want = np.array([[_ev(e, **env) for e in row] for row in ex[key]])
        assert np.allclose(f[key], want, rtol=1e-14, atol=1e-15), key
    row = np.array([_ev(e, **env) for e in ex["Yattn_row"]])
    assert np.allclose(f["Yattn"], np.tile(row, (4, 1)), rtol=1e-14)


# ----------------------------------------------------------------------------------------------- Newton-Schulz
def test_golden_ns_alpha_and_first_step():
    g = _load("ns_alpha_2x2.json")
    W = np.array(g["W"], float)
    assert abs(O.ns_alpha(W) - _ev(g["alpha"])) < 1e-17
    _, xs, _ = O.newton_schulz(W, 1)
    X0 = np.array([[_ev(e) for e in row] for row in g["X0"]])
    X1 = np.array([[_ev(e) for e in row] for row in g["X1"]])
    assert np.allclose(xs[0], X0, rtol=1e-15, atol=0)
    assert np.allclose(xs[1], X1, rtol=1e-14, atol=0)


def _ns_closed_form(We, K):
    """X_0 = alpha We is symmetric, so E_k = I - We X_k obeys E_{k+1} = E_k^2 and
    X_K = U diag((1 - (1 - alpha mu^2)^(2^K)) / mu) U^T."""
    mu, U = np.linalg.eigh(We)
    alpha = O.ns_alpha(We)
    t = np.exp((2.0 ** K) * np.log1p(-alpha * mu * mu))
    return (U * ((1.0 - t) / mu)) @ U.T


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.PVT_S3], ids=lambda w: w.name)
def test_ns_matches_eigen_closed_form(wl):
    inp = WL.make_inputs(wl, seed=0)
    p = _params(wl)
    L = O.landmark_pool(inp["Q"][0, 0], wl.H, wl.W, wl.r)
    We = O.laplacian_kernel(L, L, wl.lam) + wl.eps * np.eye(wl.m)
    X, _, _ = O.newton_schulz(We, p.ns_iters)
    ref = _ns_closed_form(We, p.ns_iters)
    assert np.linalg.norm(X - ref) / np.linalg.norm(ref) < 1e-12


def test_ns_matches_closed_form_unconverged_m256():
    """The 128x128 / r=8 shape (m=256, K=16) is not converged at K; the closed form still pins it."""
    wl = WL.HIRES_BF16
    inp = WL.make_inputs(wl.replace(B=1), seed=0)
    L = O.landmark_pool(inp["Q"][0, 0], wl.H, wl.W, wl.r)
    We = O.laplacian_kernel(L, L, wl.lam) + wl.eps * np.eye(wl.m)
    X, _, _ = O.newton_schulz(We, wl.ns_iters)
    ref = _ns_closed_form(We, wl.ns_iters)
    assert np.linalg.norm(X - ref) / np.linalg.norm(ref) < 1e-10


def test_ns_converges_to_inverse_tiny():
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=0)
    L = O.landmark_pool(inp["Q"][0, 0], wl.H, wl.W, wl.r)
    We = O.laplacian_kernel(L, L, wl.lam) + wl.eps * np.eye(wl.m)
    X, _, _ = O.newton_schulz(We, wl.ns_iters)
    inv = np.linalg.inv(We)
    assert np.linalg.norm(X - inv) / np.linalg.norm(inv) < 1e-12
    assert np.linalg.norm(We @ X - np.eye(wl.m)) < 1e-12


def test_ns_nonsymmetric_converges_to_inverse():
    """On a non-symmetric matrix only X_0 = alpha W^T (not alpha W) is guaranteed to converge."""
    rng = _rng(7)
    A = np.eye(6) * 3 + rng.standard_normal((6, 6))
    X, _, _ = O.newton_schulz(A, 40)
    assert np.allclose(X, np.linalg.inv(A), rtol=1e-10, atol=1e-12)


def test_ns_kappa50_converges_within_predicted_iterations():
    """The pages claim NS copes with a condition number of 50; predict K from alpha*mu_min^2 and check."""
    rng = _rng(8)
    Qm, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    mu = np.geomspace(1.0, 50.0, 32)
    A = (Qm * mu) @ Qm.T
    A = 0.5 * (A + A.T)
    alpha = O.ns_alpha(A)
    delta = 1e-10
    rho = 1.0 - alpha * mu.min() ** 2
    K = int(math.ceil(math.log2(math.log(delta) / math.log(rho))))
    X, _, _ = O.newton_schulz(A, K)
    assert np.linalg.norm(A @ X - np.eye(32), 2) < delta * 10


def test_m1_scalar_newton_schulz_and_rank1_output():
    """r = H = W gives m = 1: alpha = 1/w^2, X_0 = 1/w is already the fixed point, and Y_attn is rank one."""
    wl = WL.TINY.replace(H=4, W=4, r=4)
    inp = WL.make_inputs(wl, seed=9)
    p = _params(wl)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    f = O.forward_slice(q, k, v, None, p)
    w = 1.0 + wl.eps
    assert abs(f["X"][0, 0] - 1.0 / w) < 1e-15
    lvec = q.mean(axis=0)
    cq = np.exp(-np.abs(q - lvec).sum(axis=1) / wl.lam)
    ck = np.exp(-np.abs(k - lvec).sum(axis=1) / wl.lam)
    ref = np.outer(cq, (ck @ v) / w)
    assert np.allclose(f["Yattn"], ref, rtol=1e-13)


# ----------------------------------------------------------------------------------------------- Nystrom
def test_nystrom_r1_equals_regularised_exact_kernel():
    """r = 1 gives m = N and L = Q, so C_Q = W, C_K^T = G with G_ij = k(q_i, k_j), and
    Y_attn = W (W + eps I)^-1 G V, which is within eps/(lambda_min(W)+eps) of the exact kernel product G V."""
    wl = WL.TINY_R1
    inp = WL.make_inputs(wl, seed=0)
    p = _params(wl)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    f = O.forward_slice(q, k, v, None, p)
    G = np.array([[math.exp(-sum(abs(q[i, c] - k[j, c]) for c in range(wl.d)) / wl.lam)
                   for j in range(wl.N)] for i in range(wl.N)])
    Wm = f["W"]
    closed = Wm @ np.linalg.solve(Wm + wl.eps * np.eye(wl.N), G @ v)
    assert np.linalg.norm(f["Yattn"] - closed) / np.linalg.norm(closed) < 1e-10
    exact = G @ v
    lam_min = np.linalg.eigvalsh(Wm).min()
    bound = wl.eps / (lam_min + wl.eps)
    assert np.linalg.norm(f["Yattn"] - exact) / np.linalg.norm(exact) <= bound * (1 + 1e-9)
    # and with eps = 0 the product is the exact kernel product up to the NS residual
    f0 = O.forward_slice(q, k, v, None, _params(wl, eps=0.0, ns_iters=40))
    assert np.linalg.norm(f0["Yattn"] - exact) / np.linalg.norm(exact) < 1e-8


def _bruteforce_forward(q, k, v, w, H, W, r, lam, eps, iters):
    """Pure-Python loops on a tiny slice, associating the Nystrom product as (C_Q X C_K^T) V."""
    N, d = len(q), len(q[0])
    Wr = W // r
    m = (H // r) * Wr
    L = [[math.fsum(q[(Y * r + a) * W + X * r + b][c] for a in range(r) for b in range(r)) / (r * r)
          for c in range(d)] for Y in range(H // r) for X in range(Wr)]

    def kern(x, y):
        return math.exp(-math.fsum(abs(x[c] - y[c]) for c in range(d)) / lam)

    CQ = [[kern(q[i], L[l]) for l in range(m)] for i in range(N)]
    CK = [[kern(k[j], L[l]) for l in range(m)] for j in range(N)]
    We = [[kern(L[a], L[b]) + (eps if a == b else 0.0) for b in range(m)] for a in range(m)]

    def mm(A, B):
        return [[math.fsum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))]
                for i in range(len(A))]

    n1 = max(math.fsum(abs(We[i][j]) for i in range(m)) for j in range(m))
    ninf = max(math.fsum(abs(We[i][j]) for j in range(m)) for i in range(m))
    alpha = 1.0 / (n1 * ninf)
    X = [[alpha * We[j][i] for j in range(m)] for i in range(m)]
    for _ in range(iters):
        T = mm(We, X)
        U = [[(2.0 if i == j else 0.0) - T[i][j] for j in range(m)] for i in range(m)]
        X = mm(X, U)
    CKt = [[CK[j][l] for j in range(N)] for l in range(m)]
    Ghat = mm(mm(CQ, X), CKt)  # explicit N x N Nystrom matrix
    Y = mm(Ghat, v)
    for yy in range(H):
        for xx in range(W):
            for c in range(d):
                acc = 0.0
                for a in (-1, 0, 1):
                    for b in (-1, 0, 1):
                        if 0 <= yy + a < H and 0 <= xx + b < W:
                            acc += w[c][a + 1][b + 1] * v[(yy + a) * W + xx + b][c]
                Y[yy * W + xx][c] += acc
    return Y


def test_end_to_end_bruteforce_tiny():
    wl = WL.TINY.replace(H=4, W=6, d=5, r=2)  # ragged grid, m = 6
    inp = WL.make_inputs(wl, seed=11)
    p = _params(wl)
    q, k, v, w = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0], inp["w64"]
    f = O.forward_slice(q, k, v, w, p)
    ref = np.array(_bruteforce_forward(q.tolist(), k.tolist(), v.tolist(), w.tolist(), wl.H, wl.W, wl.r,
                                       wl.lam, wl.eps, wl.ns_iters))
    assert np.linalg.norm(f["Y"] - ref) / np.linalg.norm(ref) < 1e-12


def test_batched_wrapper_uses_each_heads_dwc_filters():
    """Channel h*d + c of the weight belongs to head h: compare DWC against torch's grouped conv2d (fp64, CPU)."""
    wl = WL.TINY.replace(B=2, heads=3, H=5, W=7, d=4, r=1)
    inp = WL.make_inputs(wl, seed=12)
    p = _params(wl)
    out = O.forward(inp["Q"], inp["K"], inp["V"], inp["w64"], p, keep=["Y", "Yattn"])
    D = out["Y"] - out["Yattn"]
    V = torch.from_numpy(inp["V"])  # [B, h, N, d]
    x = V.reshape(wl.B, wl.heads, wl.H, wl.W, wl.d).permute(0, 1, 4, 2, 3).reshape(wl.B, wl.heads * wl.d, wl.H,
                                                                                     wl.W)
    wt = torch.from_numpy(inp["w64"]).reshape(wl.heads * wl.d, 1, 3, 3)
    ref = torch.nn.functional.conv2d(x, wt, padding=1, groups=wl.heads * wl.d)
    ref = ref.reshape(wl.B, wl.heads, wl.d, wl.H, wl.W).permute(0, 1, 3, 4, 2).reshape(wl.B, wl.heads, wl.N, wl.d)
    assert np.allclose(D, ref.numpy(), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------------- whitening
def test_whitening_moments_and_loops():
    rng = _rng(13)
    c = np.exp(-rng.uniform(0, 5, size=(40, 6)))
    for eps_w in (1e-5, 0.0):
        A, mu, rstd = O.whiten_columns(c, eps_w)
        assert np.allclose(A.mean(axis=0), 0, atol=1e-15)
        var = c.var(axis=0)
        assert np.allclose(A.var(axis=0), var / (var + eps_w), rtol=1e-12)
    A, mu, rstd = O.whiten_columns(c, 1e-5)
    for l in range(6):
        col = [c[i, l] for i in range(40)]
        m_ = math.fsum(col) / 40
        v_ = math.fsum((x - m_) ** 2 for x in col) / 40
        for i in range(40):
            assert abs(A[i, l] - (c[i, l] - m_) / math.sqrt(v_ + 1e-5)) < 1e-12


# ----------------------------------------------------------------------------------------------- DWC
def test_golden_dwc_cross_correlation():
    g = _load("dwc_cross_correlation_3x3.json")
    V = np.array(g["V"], float).reshape(9, 1)
    for case in g["cases"]:
        w = np.array(case["w"], float).reshape(1, 3, 3)
        out = O.dwc(V, w, g["H"], g["W"]).reshape(3, 3)
        assert np.array_equal(out, np.array(case["out"], float))


def test_dwc_delta_box_and_adjoint():
    rng = _rng(14)
    H, W, d = 5, 6, 3
    v = rng.standard_normal((H * W, d))
    delta = np.zeros((d, 3, 3))
    delta[:, 1, 1] = 1
    assert np.array_equal(O.dwc(v, delta, H, W), v)
    ones = np.ones((d, 3, 3))
    box = O.dwc(v, ones, H, W).reshape(H, W, d)
    g = v.reshape(H, W, d)
    for y in range(H):
        for x in range(W):
            s = g[max(0, y - 1):y + 2, max(0, x - 1):x + 2].sum(axis=(0, 1))
            assert np.allclose(box[y, x], s, rtol=1e-14)
    w = rng.standard_normal((d, 3, 3))
    u = rng.standard_normal((H * W, d))
    assert abs(np.sum(O.dwc(v, w, H, W) * u) - np.sum(v * O.dwc_adjoint(u, w, H, W))) < 1e-12


# ----------------------------------------------------------------------------------------------- gradients
def test_kernel_gradient_sign_by_finite_differences():
    rng = _rng(15)
    x, y, lam, h = rng.standard_normal(6), rng.standard_normal(6), 4.0, 1e-6

    def k(a, b):
        return math.exp(-np.abs(a - b).sum() / lam)

    kv = k(x, y)
    for i in range(6):
        e = np.zeros(6)
        e[i] = h
        fd_x = (k(x + e, y) - k(x - e, y)) / (2 * h)
        fd_y = (k(x, y + e) - k(x, y - e)) / (2 * h)
        assert abs(fd_x - (-(1 / lam) * np.sign(x[i] - y[i]) * kv)) < 1e-8
        assert abs(fd_y - ((1 / lam) * np.sign(x[i] - y[i]) * kv)) < 1e-8


def _crop(wl, inp, hh=4, ww=4):
    """Tokens y < hh, x < ww of batch 0, head 0."""
    idx = np.array([y * wl.W + x for y in range(hh) for x in range(ww)])
    return {k: inp[k][0, 0][idx] for k in ("Q", "K", "V", "dY")}


@pytest.mark.parametrize("whiten", [True, False])
def test_backward_matches_finite_differences_on_crop(whiten):
    """4x4 crop of the training workload, r=2 (m=4), d=64, K=12, alpha held fixed as in the backward pass."""
    wl = WL.TRAIN_S1
    inp = WL.make_inputs(wl, seed=0)
    c = _crop(wl, inp)
    p = O.Params(B=1, heads=1, H=4, W=4, d=wl.d, r=2, lam=wl.lam, eps=wl.eps, ns_iters=wl.ns_iters,
                 whiten=whiten, whiten_eps=wl.whiten_eps)
    w = inp["w64"][:wl.d]
    q, k, v, dy = c["Q"], c["K"], c["V"], c["dY"]
    f = O.forward_slice(q, k, v, w, p)
    alpha = f["alpha"]
    g = O.backward_slice(q, k, v, w, dy, p, fwd=f)
    g0 = O.backward_slice(q, k, v, None, dy, p, fwd=O.forward_slice(q, k, v, None, p))
    h = 1e-6

    def loss(qq, kk, vv, ww):
        return float(np.sum(dy * O.forward_slice(qq, kk, vv, ww, p, alpha=alpha)["Y"]))

    L = f["L"]
    for name, arr in (("dQ", q), ("dK", k), ("dV", v)):
        fd = np.zeros_like(arr)
        for i in range(arr.shape[0]):
            for cc in range(arr.shape[1]):
                e = np.zeros_like(arr)
                e[i, cc] = h
                args_p = [q, k, v]
                args_m = [q, k, v]
                slot = {"dQ": 0, "dK": 1, "dV": 2}[name]
                args_p[slot] = arr + e
                args_m[slot] = arr - e
                # Every difference is taken on the attention branch alone. DWC(V) does not depend on Q or K, and
                # its part of dV (the adjoint stencil of dY) is ~1e2-1e4 times the attention part C_K dS, so with
                # DWC on, a dV check at 1e-6 would barely see C_K dS. The DWC part is pinned below.
                fd[i, cc] = (loss(*args_p, None) - loss(*args_m, None)) / (2 * h)
        # skip coordinates within the FD step of a kink of |x - l| (none expected for continuous draws)
        if name != "dV":
            near = np.abs(arr[:, None, :] - L[None, :, :]).min(axis=1) < 1e-5
            fd[near] = g0[name][near]
        err = np.linalg.norm(g0[name] - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (name, err)
    # With DWC on, dQ and dK do not change and dV gains exactly the adjoint stencil of dy: the difference of the two
    # gradients is the gradient of <dy, DWC(V)>, which is linear in V, so central differences give it exactly.
    assert np.array_equal(g["dQ"], g0["dQ"]) and np.array_equal(g["dK"], g0["dK"])
    fd_dwc = np.zeros_like(v)
    for i in range(v.shape[0]):
        for cc in range(v.shape[1]):
            e = np.zeros_like(v)
            e[i, cc] = 1.0
            fd_dwc[i, cc] = 0.5 * float(np.sum(dy * (O.dwc(v + e, w, p.H, p.W) - O.dwc(v - e, w, p.H, p.W))))
    assert np.linalg.norm((g["dV"] - g0["dV"]) - fd_dwc) <= 1e-12 * np.linalg.norm(fd_dwc)


def test_alpha_dependence_vanishes_at_convergence():
    """Reading R6: once NS has converged X_K no longer depends on alpha, so freezing alpha changes nothing."""
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=0)
    p = _params(wl)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    f = O.forward_slice(q, k, v, None, p)
    f2 = O.forward_slice(q, k, v, None, p, alpha=f["alpha"] * 0.9)
    assert np.linalg.norm(f["Yattn"] - f2["Yattn"]) / np.linalg.norm(f["Yattn"]) < 1e-12


# ------------------------------------------------------------------------------------------- parameter gradients
def _crop_case(whiten, ns_iters=None):
    wl = WL.TRAIN_S1
    inp = WL.make_inputs(wl, seed=0)
    c = _crop(wl, inp)
    p = O.Params(B=1, heads=1, H=4, W=4, d=wl.d, r=2, lam=wl.lam, eps=wl.eps,
                 ns_iters=wl.ns_iters if ns_iters is None else ns_iters, whiten=whiten, whiten_eps=wl.whiten_eps)
    return p, c["Q"], c["K"], c["V"], c["dY"], inp["w64"][:wl.d]


def test_dwc_weight_grad_matches_finite_differences():
    """Y is linear in the DWC weights, so central differences of <dy, Y> give the weight gradient exactly (up to
    rounding); every one of the d x 9 taps is checked, on a grid with border tokens in every direction."""
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=0)
    p = _params(wl)
    q, k, v, w = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0], inp["w64"][:wl.d]
    dy = np.random.default_rng(5).standard_normal(v.shape)
    g = O.backward_slice(q, k, v, w, dy, p)
    h = 1e-3
    fd = np.zeros_like(w)
    for c in range(w.shape[0]):
        for a in range(3):
            for b in range(3):
                e = np.zeros_like(w)
                e[c, a, b] = h
                yp = O.forward_slice(q, k, v, w + e, p)["Y"]
                ym = O.forward_slice(q, k, v, w - e, p)["Y"]
                fd[c, a, b] = np.sum(dy * (yp - ym)) / (2 * h)
    assert np.linalg.norm(g["d_dwc"] - fd) / np.linalg.norm(fd) < 1e-9


@pytest.mark.parametrize("whiten", [True, False])
def test_lambda_grad_matches_finite_differences(whiten):
    """d<dy, Y>/dlambda with alpha held at its value (reading R6), against central differences on the crop."""
    p, q, k, v, dy, w = _crop_case(whiten)
    f = O.forward_slice(q, k, v, w, p)
    g = O.backward_slice(q, k, v, w, dy, p, fwd=f)
    h = 1e-6

    def loss(lam):
        pp = dataclasses.replace(p, lam=lam)
        return float(np.sum(dy * O.forward_slice(q, k, v, None, pp, alpha=f["alpha"])["Y"]))

    fd = (loss(p.lam + h) - loss(p.lam - h)) / (2 * h)
    assert abs(g["dlam"] - fd) <= 1e-6 * abs(fd), (g["dlam"], fd)


def test_batched_backward_accumulates_per_head_and_over_slices():
    """The batched backward() adds each (batch, head) slice's DWC weight gradient into the filter bank of its own
    head (channels h*d .. h*d + d - 1) and sums the lambda gradient over every slice. Pinned by central differences
    of the total loss sum_{b,h} <dY[b,h], Y[b,h]>: Y is linear in the weights, so unit differences of the batched
    forward give their gradient exactly; for lambda each slice keeps its own alpha fixed (reading R6). Two batch
    entries and three heads, so that overwriting instead of adding, or filing a slice under the wrong head, fails."""
    wl = WL.TINY.replace(B=2, heads=3, H=6, W=6, d=8, r=2, whiten=True, backward=True, qk_dist="student_t")
    inp = WL.make_inputs(wl, seed=21, with_dy=True)
    p = _params(wl)
    Q, K, V, w, dY = inp["Q"], inp["K"], inp["V"], inp["w64"], inp["dY"]
    g = O.backward(Q, K, V, w, dY, p)

    def total(ww):
        return float(np.sum(dY * O.forward(Q, K, V, ww, p, keep=["Y"])["Y"]))

    fd = np.zeros_like(w)
    for idx in np.ndindex(*w.shape):
        e = np.zeros_like(w)
        e[idx] = 1.0
        fd[idx] = 0.5 * (total(w + e) - total(w - e))
    assert np.linalg.norm(g["d_dwc"] - fd) <= 1e-12 * np.linalg.norm(fd)

    alphas = {(b, h): O.forward_slice(Q[b, h], K[b, h], V[b, h], None, p)["alpha"]
              for b in range(wl.B) for h in range(wl.heads)}

    def total_lam(lam):
        pp = dataclasses.replace(p, lam=lam)
        return math.fsum(float(np.sum(dY[b, h] * O.forward_slice(Q[b, h], K[b, h], V[b, h], None, pp,
                                                                  alpha=alphas[b, h])["Y"]))
                         for b in range(wl.B) for h in range(wl.heads))

    hl = 1e-6
    fd_lam = (total_lam(p.lam + hl) - total_lam(p.lam - hl)) / (2 * hl)
    assert abs(g["dlam"] - fd_lam) <= 1e-6 * abs(fd_lam), (g["dlam"], fd_lam)
    # every slice contributes: the sum is not carried by one of them
    per = [O.backward_slice(Q[b, h], K[b, h], V[b, h], None, dY[b, h], p)["dlam"]
           for b in range(wl.B) for h in range(wl.heads)]
    assert min(abs(x) for x in per) > 1e-3 * max(abs(x) for x in per)


def test_exact_alpha_gradient_matches_finite_differences():
    """With two Newton-Schulz steps X_K still depends on alpha. The exact gradient (alpha recomputed from W_eps in
    the forward of every difference) must match central differences in Q, K and lambda, and the stop-gradient
    reading must visibly miss them, so the alpha path is really exercised. lambda = 64 makes the landmark kernel
    matrix far from diagonal (at lambda = 4 its off-diagonal entries are ~exp(-30) and alpha hardly moves)."""
    p, q, k, v, dy, w = _crop_case(True, ns_iters=2)
    p = dataclasses.replace(p, lam=64.0)
    f = O.forward_slice(q, k, v, w, p)
    g = O.backward_slice(q, k, v, w, dy, p, fwd=f, exact_alpha=True)
    g0 = O.backward_slice(q, k, v, w, dy, p, fwd=f)
    h = 1e-6
    L = f["L"]

    def loss(qq, kk, pp):
        return float(np.sum(dy * O.forward_slice(qq, kk, v, None, pp)["Y"]))

    for name, arr in (("dQ", q), ("dK", k)):
        fd = np.zeros_like(arr)
        for i in range(arr.shape[0]):
            for cc in range(arr.shape[1]):
                e = np.zeros_like(arr)
                e[i, cc] = h
                if name == "dQ":
                    fd[i, cc] = (loss(q + e, k, p) - loss(q - e, k, p)) / (2 * h)
                else:
                    fd[i, cc] = (loss(q, k + e, p) - loss(q, k - e, p)) / (2 * h)
        near = np.abs(arr[:, None, :] - L[None, :, :]).min(axis=1) < 1e-5
        fd[near] = g[name][near]
        err = np.linalg.norm(g[name] - fd) / np.linalg.norm(fd)
        err0 = np.linalg.norm(g0[name] - fd) / np.linalg.norm(fd)
        assert err < 1e-6, (name, err)
        if name == "dQ":
            assert err0 > 100 * err and err0 > 1e-4, (name, err0)
        else:
            # K enters neither W_eps nor alpha (the landmarks are pooled from Q): the alpha path leaves dK alone
            assert np.array_equal(g["dK"], g0["dK"])
    fd = (loss(q, k, dataclasses.replace(p, lam=p.lam + h)) - loss(q, k, dataclasses.replace(p, lam=p.lam - h))) / (2 * h)
    assert abs(g["dlam"] - fd) <= 1e-6 * abs(fd), (g["dlam"], fd)
    assert abs(g0["dlam"] - fd) > 1e-4 * abs(fd), (g0["dlam"], fd)


# ------------------------------------------------------------------------------------------------ CG comparator
def test_cg_reaches_the_inverse():
    """CG terminates in as many steps as W has distinct eigenvalues (exact arithmetic): a 32 x 32 SPD matrix with
    three eigenvalues {1, 7, 50} is inverted to rounding after 3 steps and not after 2. With 32 distinct eigenvalues
    (kappa = 50) rounding delays termination a little, so 1.5 m steps reach the inverse; so does a workload's
    landmark kernel matrix after 2 m steps."""
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    B = (Qm * np.repeat([1.0, 7.0, 50.0], [10, 12, 10])) @ Qm.T
    B = 0.5 * (B + B.T)
    inv = np.linalg.inv(B)
    X2, _ = O.cg_pinv(B, 2)
    X3, _ = O.cg_pinv(B, 3)
    assert np.linalg.norm(X2 - inv) / np.linalg.norm(inv) > 0.1
    assert np.linalg.norm(X3 - inv) / np.linalg.norm(inv) < 1e-12
    A = WL.spd_matrix(32, 50.0, 3)
    X, hist = O.cg_pinv(A, 48)
    assert np.linalg.norm(X - np.linalg.inv(A)) / np.linalg.norm(np.linalg.inv(A)) < 1e-12
    wl = WL.PVT_S1
    inp = WL.make_inputs(wl, seed=0)
    L = O.landmark_pool(inp["Q"][0, 0], wl.H, wl.W, wl.r)
    We = O.laplacian_kernel(L, L, wl.lam) + wl.eps * np.eye(len(L))
    X, hist = O.cg_pinv(We, 2 * len(L))
    assert hist[-1] < 1e-8 * np.sqrt(len(L))


def test_cg_energy_error_decreases_and_first_step_is_the_line_search():
    """CG minimises the W-norm of the error over growing Krylov spaces, so it never increases; its first step from
    x = 0 is the exact line search along b: x_1 = (b.b / b.Wb) b, column by column."""
    A = WL.spd_matrix(24, 50.0, 4)
    inv = np.linalg.inv(A)
    prev = None
    for k in range(1, 20):
        X, _ = O.cg_pinv(A, k)
        E = X - inv
        energy = float(np.sum(E * (A @ E)))
        if prev is not None:
            assert energy <= prev * (1 + 1e-12)
        prev = energy
    X1, _ = O.cg_pinv(A, 1)
    expect = np.eye(24) * (1.0 / np.diag(A))  # b = e_j: b.b = 1, b.Wb = A_jj
    assert np.allclose(X1, expect, rtol=1e-14, atol=0)


# ------------------------------------------------------------------------------------- Gaussian-kernel variant
def test_gaussian_kernel_bruteforce():
    rng = _rng(30)
    x, y, lam = rng.standard_normal((7, 5)), rng.standard_normal((4, 5)), 4.0
    K = O.gaussian_kernel(x, y, lam)
    for i in range(7):
        for l in range(4):
            ref = math.exp(-math.fsum((x[i, c] - y[l, c]) ** 2 for c in range(5)) / lam)
            assert abs(K[i, l] - ref) <= 1e-15 * ref + 1e-300


def test_gaussian_kernel_identity_symmetry_scale_separable_and_definite():
    rng = _rng(31)
    x = rng.standard_normal((9, 6))
    Kxx = O.gaussian_kernel(x, x, 3.0)
    assert np.array_equal(np.diag(Kxx), np.ones(9)) and np.array_equal(Kxx, Kxx.T)
    y = rng.standard_normal((4, 6))
    # k(s x, s y; s^2 lambda) = k(x, y; lambda): the distance is squared
    assert np.allclose(O.gaussian_kernel(3 * x, 3 * y, 27.0), O.gaussian_kernel(x, y, 3.0), rtol=1e-13)
    # separable: the kernel is the product over coordinates of one-dimensional kernels
    prod = np.ones((9, 4))
    for c in range(6):
        prod *= O.gaussian_kernel(x[:, c:c + 1], y[:, c:c + 1], 3.0)
    assert np.allclose(O.gaussian_kernel(x, y, 3.0), prod, rtol=1e-13)
    # the Gram matrix of distinct points is positive definite
    assert np.linalg.eigvalsh(Kxx).min() > 0


def test_gaussian_variant_changes_only_the_kernel():
    """kernel = "gauss" swaps C_Q, C_K and W for their Gaussian versions and keeps every other step: the landmarks
    are the same, W_eps is the Gaussian Gram matrix of the landmarks plus eps I, and the Nystrom output follows
    from those with the same solver. Also translation invariant, like the Laplacian block."""
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=5)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    fl = O.forward_slice(q, k, v, None, _params(wl))
    fg = O.forward_slice(q, k, v, None, _params(wl, kernel="gauss"))
    assert np.array_equal(fl["L"], fg["L"])
    L = fg["L"]
    G = np.array([[math.exp(-math.fsum((L[a, c] - L[b, c]) ** 2 for c in range(wl.d)) / wl.lam)
                   for b in range(wl.m)] for a in range(wl.m)])
    assert np.allclose(fg["We"], G + wl.eps * np.eye(wl.m), rtol=1e-14, atol=0)
    X, _, _ = O.newton_schulz(fg["We"], wl.ns_iters)
    Y = fg["CQ"] @ X @ (fg["CK"].T @ v)
    assert np.linalg.norm(fg["Yattn"] - Y) / np.linalg.norm(Y) < 1e-12
    assert np.linalg.norm(fg["Yattn"] - fl["Yattn"]) > 1e-3 * np.linalg.norm(fl["Yattn"])
    shift = _rng(6).standard_normal(wl.d)
    f1 = O.forward_slice(q + shift, k + shift, v, None, _params(wl, kernel="gauss"))
    for key in ("CQ", "CK", "We", "Yattn"):
        assert np.allclose(fg[key], f1[key], rtol=1e-11, atol=1e-14), key


def test_gaussian_nystrom_r1_equals_regularised_exact_kernel():
    """r = 1 with the Gaussian kernel: Y_attn = W (W + eps I)^-1 G V with G_ij = exp(-||q_i - k_j||^2 / lambda)."""
    wl = WL.TINY_R1
    inp = WL.make_inputs(wl, seed=0)
    p = _params(wl, kernel="gauss", ns_iters=40)
    q, k, v = inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0]
    f = O.forward_slice(q, k, v, None, p)
    G = np.array([[math.exp(-math.fsum((q[i, c] - k[j, c]) ** 2 for c in range(wl.d)) / wl.lam)
                   for j in range(wl.N)] for i in range(wl.N)])
    Wm = f["W"]
    closed = Wm @ np.linalg.solve(Wm + wl.eps * np.eye(wl.N), G @ v)
    assert np.linalg.norm(f["Yattn"] - closed) / np.linalg.norm(closed) < 1e-9


def test_gaussian_variant_has_no_backward():
    wl = WL.TINY
    inp = WL.make_inputs(wl, seed=0, with_dy=True)
    with pytest.raises(NotImplementedError):
        O.backward_slice(inp["Q"][0, 0], inp["K"][0, 0], inp["V"][0, 0], None, inp["dY"][0, 0],
                         _params(wl, kernel="gauss"))
