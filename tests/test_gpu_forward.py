"""GPU parity of the forward pass: every stage and the whole block against the fp64 oracle, through the C ABI.

Bars: relative Frobenius error <= 1e-4 for float32 inputs and <= 2e-2 for bf16 inputs (fp32 accumulation), on the
attention branch alone (no DWC) and on the full output separately. Stage inputs are the oracle's own values rounded
to float32, so that each kernel is checked in isolation.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (TOL_STAGE, dev, gpu_forward, host, inputs, note, oparams, oracle_forward, params, relF,
                      tol, upload)
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

pytestmark = pytest.mark.gpu

# The five workload shapes plus edge cases: m = 1; N < 64 with several heads (channel h*d + c); a ragged grid with
# m = 99 > 64 (multi-launch Newton-Schulz with ragged tiles) and d = 128; no NS steps; bf16 at the stage-1 shape;
# whitening on a small grid; N = 196 tokens that end in a ragged 64-row tile; N = m = 63 (rows not a multiple of 4);
# the largest step count on both solver variants and on the m > 64 path.
MAIN = [WL.TINY, WL.TINY_R1, WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16, WL.TRAIN_S1]
EDGE = [
    WL.TINY.replace(name="m1_8x8_r8", r=8),
    WL.TINY.replace(name="ragged_10x6_d32_h3", B=2, heads=3, H=10, W=6, d=32, r=2),
    WL.TINY.replace(name="ragged_18x22_d128_m99", H=18, W=22, d=128, r=2, qk_dist="student_t"),
    WL.TINY.replace(name="ns_iters0", ns_iters=0),
    WL.PVT_S1.replace(name="s1_bf16_B2", B=2, dtype=WL.BF16),
    WL.TINY.replace(name="whiten_12x12_d16_B2", B=2, H=12, W=12, r=3, whiten=True),
    WL.PVT_S3.replace(name="s3_B2_h5", B=2),
    WL.TINY.replace(name="d64_20x20_m100_bf16", H=20, W=20, d=64, r=2, dtype=WL.BF16, qk_dist="student_t"),
    WL.TINY.replace(name="odd_9x7_r1_m63", H=9, W=7, r=1),
    # the most Newton-Schulz steps the library accepts (LF_NS_ITERS_MAX = 64): six runs of coupled steps
    WL.TINY.replace(name="tiny_K64_m16", ns_iters=64),
    WL.PVT_S1.replace(name="s1_B1_K64", B=1, ns_iters=64),
    # the m > 64 path (split-fp16 tile products, one launch per coupled step) over four runs of coupled steps
    WL.TINY.replace(name="ragged_20x20_m100_K40", H=20, W=20, d=64, r=2, ns_iters=40, qk_dist="student_t"),
    # d = 128 with m <= 64: the output kernel forms P = X S in its prologue with more than 64 KB of LDS
    WL.TINY.replace(name="d128_14x14_m49_B2", B=2, H=14, W=14, d=128, r=2, qk_dist="student_t"),
]
ALL = MAIN + EDGE


@pytest.mark.parametrize("wl", ALL, ids=lambda w: w.name)
def test_forward_end_to_end(wl):
    note(f"[gpu] forward {wl.name}")
    ref = oracle_forward(wl)
    # With and without a saved buffer (the saved one receives every intermediate), with and without DWC.
    Y, sv, p = gpu_forward(wl, dwc=True, save=True)
    Ya_s, _, _ = gpu_forward(wl, dwc=False, save=True)
    Yf, _, _ = gpu_forward(wl, dwc=True, save=False)
    Ya, _, _ = gpu_forward(wl, dwc=False, save=False)
    e_full = relF(host(Y), ref["Y"])
    e_attn = relF(host(Ya), ref["Yattn"])
    e_full_f = relF(host(Yf), ref["Y"])
    e_attn_s = relF(host(Ya_s), ref["Yattn"])
    G = wl.G
    worst = max(relF(host(Ya).reshape(G, -1)[g], ref["Yattn"].reshape(G, -1)[g]) for g in range(G))
    note(f"    relF full={e_full:.3e}/{e_full_f:.3e} attn={e_attn_s:.3e}/{e_attn:.3e} (saved/no saved) "
         f"worst-slice attn={worst:.3e}")
    assert e_full <= tol(wl)
    assert e_attn <= tol(wl)
    assert e_full_f <= tol(wl)
    assert e_attn_s <= tol(wl)
    # intermediates the forward kept in the saved buffer
    rs = lambda a: np.asarray(a).reshape((G,) + np.asarray(a).shape[2:])
    assert relF(host(sv["L"]), rs(ref["L"])) <= 1e-6
    # the library stores C_Q and C_K landmark-major: [G][m][N]
    assert relF(host(sv["CQ"]).transpose(0, 2, 1), rs(ref["CQ"])) <= 1e-5
    assert relF(host(sv["CK"]).transpose(0, 2, 1), rs(ref["CK"])) <= 1e-5
    assert relF(host(sv["We"]), rs(ref["We"])) <= 1e-5
    Xk = host(sv["xs"])[:, wl.ns_iters]
    e_x, e_s, e_p = (relF(Xk, rs(ref["X"])), relF(host(sv["S"]), rs(ref["S"])), relF(host(sv["P"]), rs(ref["P"])))
    note(f"    relF X_K={e_x:.3e} S={e_s:.3e} P={e_p:.3e}")
    assert e_x <= TOL_STAGE
    assert e_s <= TOL_STAGE
    assert e_p <= TOL_STAGE
    if wl.whiten:
        assert relF(host(sv["mu"]), rs(ref["mu"])) <= 1e-5
        assert relF(host(sv["rstd"]), rs(ref["rstd"])) <= 1e-5


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16], ids=lambda w: w.name)
def test_forward_is_deterministic(wl):
    note(f"[gpu] determinism {wl.name}")
    Y1, _, _ = gpu_forward(wl, save=False)
    Y2, _, _ = gpu_forward(wl, save=False)
    assert torch.equal(Y1, Y2)


# ------------------------------------------------------------------------------------------------ stages alone
def _f32(x):
    return dev(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))


def _r32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.HIRES_BF16, EDGE[1]], ids=lambda w: w.name)
def test_stage_pool_and_laplace(wl):
    note(f"[gpu] stages pool+laplace {wl.name}")
    p = params(wl)
    inp = inputs(wl)
    t = upload(wl)
    G, N, m, d = p.G, p.N, p.m, p.d
    L = torch.empty(G * m * d, device="cuda")
    lf.lf_landmark_pool(p, t["Q"], L)
    Lref = np.stack([O.landmark_pool(q, wl.H, wl.W, wl.r) for q in inp["Q"].reshape(G, N, d)])
    assert relF(host(L).reshape(G, m, d), Lref) <= 1e-6
    # laplace on the oracle's landmarks rounded to float32
    L32 = _f32(Lref)
    CQ = torch.empty(G * N * m, device="cuda")
    CK = torch.empty_like(CQ)
    We = torch.empty(G * m * m, device="cuda")
    lf.lf_laplace_l1_exp(p, t["Q"], t["K"], L32, CQ, CK, We)
    torch.cuda.synchronize()
    Lr = _r32(Lref)
    for g in range(G):
        q, k = inp["Q"].reshape(G, N, d)[g], inp["K"].reshape(G, N, d)[g]
        assert relF(host(CQ).reshape(G, m, N)[g].T, O.laplacian_kernel(q, Lr[g], wl.lam)) <= 1e-5
        assert relF(host(CK).reshape(G, m, N)[g].T, O.laplacian_kernel(k, Lr[g], wl.lam)) <= 1e-5
        Wref = O.laplacian_kernel(Lr[g], Lr[g], wl.lam) + wl.eps * np.eye(m)
        assert relF(host(We).reshape(G, m, m)[g], Wref) <= 1e-5


@pytest.mark.parametrize("wl", [WL.TINY, WL.TINY.replace(name="m25_10x10", H=10, W=10, r=2, B=2),
                                WL.PVT_S1.replace(name="s1_B2", B=2), EDGE[1], EDGE[8]],
                         ids=lambda w: w.name)
def test_forward_newton_schulz_iterates(wl):
    """Every Newton-Schulz iterate the fused forward saves tracks the oracle's iterates on the same W (a case with
    20 iterations included, where rounding that the iteration does not damp would show), and W = k(L, L) + eps I
    and the result come out symmetric."""
    note(f"[gpu] forward NS iterates {wl.name}")
    Y, sv, p = gpu_forward(wl, dwc=True, save=True)
    G, m, K = p.G, p.m, p.ns_iters
    We = host(sv["We"]).reshape(G, m, m)
    xs = host(sv["xs"]).reshape(G, K + 1, m, m)
    for g in range(G):
        assert np.array_equal(We[g], We[g].T)  # the distance kernel's W is bitwise symmetric
        _, xs_ref, _ = O.newton_schulz(We[g].astype(np.float64), K)
        for k in range(K + 1):
            assert relF(xs[g, k], xs_ref[k]) <= TOL_STAGE, (g, k)
        assert relF(xs[g, K], xs[g, K].T) <= 1e-5


@pytest.mark.parametrize("wl", [WL.TINY, WL.TINY_R1, WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16, EDGE[2]],
                         ids=lambda w: w.name)
def test_stage_newton_schulz(wl):
    note(f"[gpu] stage ns_pinv {wl.name}")
    p = params(wl)
    ref = oracle_forward(wl)
    G, m, K = p.G, p.m, p.ns_iters
    We64 = _r32(np.asarray(ref["We"]).reshape(G, m, m))
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    X = torch.empty(G * m * m, device="cuda")
    xs = torch.empty(G * (K + 1) * m * m, device="cuda")
    alpha = torch.empty(G, device="cuda")
    resid = torch.empty(G, device="cuda")
    lf.lf_ns_pinv(p, _f32(We64), X, xs, alpha, resid, ws)
    torch.cuda.synchronize()
    Xh = host(X).reshape(G, m, m)
    for g in range(G):
        Xref, xs_ref, aref = O.newton_schulz(We64[g], K)
        assert abs(host(alpha)[g] - aref) <= 1e-6 * aref
        e_x = relF(Xh[g], Xref)
        note(f"    slice {g}: X_K relF {e_x:.3e}")
        assert e_x <= TOL_STAGE
        assert relF(host(xs).reshape(G, K + 1, m, m)[g, 0], xs_ref[0]) <= 1e-6
        assert np.array_equal(host(xs).reshape(G, K + 1, m, m)[g, K], Xh[g])
        r_ref = np.linalg.norm(We64[g] @ Xref - np.eye(m))
        r_gpu = float(host(resid)[g])
        # fp32 NS cannot go below ~1e-6 * sqrt(m); above that it must track the oracle's residual
        assert r_gpu <= max(2 * r_ref, 1e-4)


def test_stage_newton_schulz_kappa50():
    """The pages' claim: NS copes with condition number 50. Synthetic SPD W, m = 32, enough steps to converge."""
    note("[gpu] stage ns_pinv kappa=50")
    rng = np.random.default_rng(8)
    Qm, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    A = (Qm * np.geomspace(1.0, 50.0, 32)) @ Qm.T
    A = 0.5 * (A + A.T)
    wl = WL.TINY.replace(H=8, W=16, r=2, ns_iters=30)  # m = 32
    p = params(wl)
    X = torch.empty(32 * 32, device="cuda")
    resid = torch.empty(1, device="cuda")
    lf.lf_ns_pinv(p, _f32(A), X, None, None, resid, None)
    torch.cuda.synchronize()
    A32 = _r32(A)
    inv = np.linalg.inv(A32)
    assert relF(host(X).reshape(32, 32), inv) <= 1e-4
    assert float(host(resid)[0]) <= 1e-4


@pytest.mark.parametrize("m,grid", [(49, (14, 14, 2)), (100, (20, 20, 2))], ids=["m49", "m100"])
def test_stage_newton_schulz_ill_conditioned(m, grid):
    """kappa = 300 SPD W and 26 steps: past the solver's runs of coupled T/X steps (T is formed again as W X between
    runs), X_K tracks the oracle's exact-step iteration and reaches W^-1 to float32 accuracy. The iterates inside a
    run carry the coupled recurrence's drift (bounded by 2^run times the rounding of one product) and get a looser
    bar."""
    note(f"[gpu] stage ns_pinv kappa=300 m={m}")
    H, W_, r = grid
    A = np.stack([WL.spd_matrix(m, 300.0, 50 + g) for g in range(2)])
    wl = WL.TINY.replace(B=2, H=H, W=W_, r=r, ns_iters=26)
    p = params(wl)
    assert p.m == m
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    X = torch.empty(2 * m * m, device="cuda")
    xs = torch.empty(2 * 27 * m * m, device="cuda")
    lf.lf_ns_pinv(p, _f32(A), X, xs, None, None, ws)
    torch.cuda.synchronize()
    A32 = _r32(A)
    xg = host(xs).reshape(2, 27, m, m)
    for g in range(2):
        _, xs_ref, _ = O.newton_schulz(A32[g], 26)
        errs = [relF(xg[g, k], xs_ref[k]) for k in range(27)]
        note(f"    slice {g}: worst iterate relF {max(errs):.3e}, X_K relF {errs[-1]:.3e}")
        assert errs[-1] <= 1e-4 and max(errs) <= 1e-3
        assert relF(host(X).reshape(2, m, m)[g], np.linalg.inv(A32[g])) <= 1e-4


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16, EDGE[2]], ids=lambda w: w.name)
def test_stage_ckv_mix_out(wl):
    note(f"[gpu] stages ckv+mix+out {wl.name}")
    p = params(wl)
    inp = inputs(wl)
    ref = oracle_forward(wl)
    t = upload(wl)
    G, N, m, d = p.G, p.N, p.m, p.d
    CK = _r32(np.asarray(ref["CK"]).reshape(G, N, m))
    CQ = _r32(np.asarray(ref["CQ"]).reshape(G, N, m))
    X = _r32(np.asarray(ref["X"]).reshape(G, m, m))
    V = inp["V"].reshape(G, N, d)
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    S = torch.empty(G * m * d, device="cuda")
    lf.lf_ckv_reduce(p, _f32(CK.transpose(0, 2, 1)), t["V"], S, ws)
    Sref = np.einsum("gil,gic->glc", CK, V)
    P = torch.empty(G * m * d, device="cuda")
    lf.lf_landmark_mix(p, _f32(X), _f32(Sref), None, P)
    Pref = np.einsum("glk,gkc->glc", X, _r32(Sref))
    Y = torch.empty_like(t["Q"])
    lf.lf_out_gemm_dwc(p, _f32(CQ.transpose(0, 2, 1)), _f32(Pref), None, t["V"], t["w"], Y)
    torch.cuda.synchronize()
    assert relF(host(S).reshape(G, m, d), Sref) <= 1e-5
    assert relF(host(P).reshape(G, m, d), Pref) <= 1e-5
    P32 = _r32(Pref)
    w = inp["w64"]
    Yref = np.stack([CQ[g] @ P32[g] + O.dwc(V[g], w[(g % wl.heads) * d:(g % wl.heads + 1) * d], wl.H, wl.W)
                     for g in range(G)])
    bar = 1e-5 if wl.dtype == WL.F32 else tol(wl)
    assert relF(host(Y).reshape(G, N, d), Yref) <= bar


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16, EDGE[1], EDGE[2]], ids=lambda w: w.name)
def test_stage_out_fused(wl):
    """Output stage with C_Q recomputed per tile from Q and L: against the oracle's C_Q P + DWC(V)."""
    note(f"[gpu] stage out_gemm_dwc_fused {wl.name}")
    p = params(wl)
    inp = inputs(wl)
    ref = oracle_forward(wl)
    t = upload(wl)
    G, N, m, d = p.G, p.N, p.m, p.d
    Lr = _r32(np.asarray(ref["L"]).reshape(G, m, d))
    P32 = _r32(np.asarray(ref["P"]).reshape(G, m, d))
    Y = torch.empty_like(t["Q"])
    lf.lf_out_gemm_dwc_fused(p, t["Q"], _f32(Lr), _f32(P32), t["V"], t["w"], Y)
    Ya = torch.empty_like(t["Q"])
    lf.lf_out_gemm_dwc_fused(p, t["Q"], _f32(Lr), _f32(P32), t["V"], None, Ya)
    torch.cuda.synchronize()
    Qg, V = inp["Q"].reshape(G, N, d), inp["V"].reshape(G, N, d)
    w = inp["w64"]
    Yattn = np.stack([O.laplacian_kernel(Qg[g], Lr[g], wl.lam) @ P32[g] for g in range(G)])
    Yref = Yattn + np.stack([O.dwc(V[g], w[(g % wl.heads) * d:(g % wl.heads + 1) * d], wl.H, wl.W) for g in range(G)])
    bar = 1e-5 if wl.dtype == WL.F32 else tol(wl)
    e_a, e_f = relF(host(Ya).reshape(G, N, d), Yattn), relF(host(Y).reshape(G, N, d), Yref)
    note(f"    relF attn={e_a:.3e} full={e_f:.3e}")
    assert e_a <= bar
    assert e_f <= bar


def test_stage_whiten_stats_and_folded_output():
    wl = WL.TRAIN_S1
    note(f"[gpu] stages whiten {wl.name}")
    p = params(wl)
    ref = oracle_forward(wl)
    G, N, m, d = p.G, p.N, p.m, p.d
    CQ = _r32(np.asarray(ref["CQ"]).reshape(G, N, m))
    mu = torch.empty(G * m, device="cuda")
    rstd = torch.empty(G * m, device="cuda")
    lf.lf_whiten_stats(p, _f32(CQ.transpose(0, 2, 1)), mu, rstd)
    torch.cuda.synchronize()
    A, muref, rsref = zip(*[O.whiten_columns(CQ[g], wl.whiten_eps) for g in range(G)])
    assert relF(host(mu).reshape(G, m), np.stack(muref)) <= 1e-6
    assert relF(host(rstd).reshape(G, m), np.stack(rsref)) <= 1e-6


# --------------------------------------------------------------------------------------------------- invariants
def _permuted(wl, pb, ph, seed=0):
    """The workload's inputs with batch entries reordered by pb and heads by ph (each head's DWC filters with it)."""
    inp = inputs(wl, seed)
    out = {k: np.ascontiguousarray(inp[k + "_raw"][pb][:, ph]) for k in ("Q", "K", "V", "dY") if k + "_raw" in inp}
    d = wl.d
    out["w"] = np.ascontiguousarray(np.concatenate([inp["w"][h * d:(h + 1) * d] for h in ph]))
    return out


@pytest.mark.parametrize("wl", [WL.PVT_S3.replace(name="s3_B4_h3", B=4, heads=3),
                                WL.PVT_S1.replace(name="s1_B4_bf16", B=4, dtype=WL.BF16),
                                WL.TINY.replace(name="m100_B3_h2", B=3, heads=2, H=20, W=20, r=2,
                                                qk_dist="student_t")],
                         ids=lambda w: w.name)
def test_forward_is_equivariant_under_slice_permutation(wl):
    """The (batch, head) slices are independent: reordering the batch entries and the heads (with each head's DWC
    filters) reorders the outputs bit for bit, whatever CU or XCD each slice lands on."""
    note(f"[gpu] slice permutation {wl.name}")
    rng = np.random.default_rng(3)
    pb, ph = rng.permutation(wl.B), rng.permutation(wl.heads)
    p = params(wl)
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    inp = inputs(wl)
    outs = []
    for src in ({k: inp[k + "_raw"] for k in ("Q", "K", "V")} | {"w": inp["w"]}, _permuted(wl, pb, ph)):
        t = {k: dev(src[k]) for k in ("Q", "K", "V", "w")}
        Y = torch.empty_like(t["Q"])
        lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, None, ws)
        torch.cuda.synchronize()
        outs.append(Y.cpu())
    Y0, Yp = outs
    assert torch.equal(Yp, Y0[torch.as_tensor(pb)][:, torch.as_tensor(ph)])
