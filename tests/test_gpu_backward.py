"""GPU parity of the backward pass (lf_attn_bwd) against the fp64 oracle's gradients, which are themselves pinned to
finite differences of the whole block (tests/test_oracle_pins.py). Bar: relative Frobenius error <= 1e-4 (float32)
and <= 2e-2 (bf16) for each of dQ, dK, dV.

Every case runs with the DWC weights and without them. With them, dV is dominated by the adjoint stencil of dY
(the attention part C_K dS is ~1e-2 of it at the training shape and ~1e-4 without whitening), so only the run
without DWC gates the attention branch of dV."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import dev, host, inputs, note, oparams, params, relF, tol, upload
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

pytestmark = pytest.mark.gpu

CASES = [
    WL.TRAIN_S1,
    WL.TRAIN_S1.replace(name="train_s1_nowhiten_B2", B=2, whiten=False),
    WL.TINY.replace(name="train_tiny_whiten_h2", B=2, heads=2, whiten=True, backward=True),
    WL.TINY.replace(name="train_ragged_10x6_d32", H=10, W=6, d=32, r=2, whiten=True, backward=True),
    WL.TINY.replace(name="train_r1_m64", r=1, whiten=False, backward=True),
    WL.TRAIN_S1.replace(name="train_s1_bf16_B2", B=2, dtype=WL.BF16),
    # 26 Newton-Schulz steps: the forward's saved iterates come from three runs of coupled steps, each started from
    # T = W X formed afresh, and the reverse chain walks back through all of them.
    WL.TINY.replace(name="train_12x12_K26", B=2, H=12, W=12, r=2, ns_iters=26, whiten=True, backward=True,
                    qk_dist="student_t"),
] + [
    # Short reverse chains: no step, and step counts below the depth (four steps) at which the chain prefetches
    # its operands, or that end on each remainder of its three-step unrolled loop.
    WL.TINY.replace(name=f"train_tiny_K{k}", B=2, ns_iters=k, whiten=True, backward=True) for k in (0, 2, 3, 4, 5)
]


def _gpu_backward(wl, dwc=True):
    p = params(wl)
    t = upload(wl)
    w = t["w"] if dwc else None
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], w, Y, saved, ws)
    dQ, dK, dV = torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])
    lf.lf_attn_bwd(p, t["Q"], t["K"], t["V"], w, saved, t["dY"], dQ, dK, dV, ws)
    torch.cuda.synchronize()
    return host(dQ), host(dK), host(dV)


@pytest.mark.parametrize("dwc", [True, False], ids=["dwc", "attn_only"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(wl, dwc):
    note(f"[gpu] backward {wl.name} dwc={dwc}")
    inp = inputs(wl)
    ref = O.backward(inp["Q"], inp["K"], inp["V"], inp["w64"] if dwc else None, inp["dY"], oparams(wl))
    dQ, dK, dV = _gpu_backward(wl, dwc)
    errs = {n: relF(a, ref[n]) for n, a in (("dQ", dQ), ("dK", dK), ("dV", dV))}
    note("    " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= tol(wl), (n, e)


def test_backward_on_fd_crop():
    """The 4x4 crop (r=2, m=4, d=64, whitening on) on which the oracle's gradient is checked by finite differences,
    with and without the DWC weights."""
    wl = WL.TRAIN_S1
    inp = inputs(wl)
    idx = np.array([y * wl.W + x for y in range(4) for x in range(4)])
    crop = wl.replace(name="crop4x4", B=1, H=4, W=4, r=2)
    arrs = {k: inp[k][0:1, :, idx] for k in ("Q", "K", "V", "dY")}
    note("[gpu] backward crop4x4")
    p = params(crop)
    tt = {k: dev(np.ascontiguousarray(inp[k + "_raw"][0:1, :, idx])) for k in ("Q", "K", "V", "dY")}
    w = dev(inp["w"])
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    for ww, w64 in ((w, inp["w64"]), (None, None)):
        Y = torch.empty_like(tt["Q"])
        lf.lf_attn_fwd(p, tt["Q"], tt["K"], tt["V"], ww, Y, saved, ws)
        dQ, dK, dV = (torch.empty_like(tt["Q"]) for _ in range(3))
        lf.lf_attn_bwd(p, tt["Q"], tt["K"], tt["V"], ww, saved, tt["dY"], dQ, dK, dV, ws)
        torch.cuda.synchronize()
        ref = O.backward(arrs["Q"], arrs["K"], arrs["V"], w64, arrs["dY"], oparams(crop))
        for n, a in (("dQ", dQ), ("dK", dK), ("dV", dV)):
            assert relF(host(a), ref[n]) <= 1e-4, (n, ww is None)


def test_backward_is_deterministic():
    wl = WL.TRAIN_S1.replace(B=2)
    note("[gpu] backward determinism")
    a = _gpu_backward(wl)
    b = _gpu_backward(wl)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------------------------- the training op's other gradients
def _gpu_backward_ex(wl, flags):
    p = params(wl)
    t = upload(wl)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, saved, ws)
    dQ, dK, dV = torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])
    dw = torch.empty(p.heads * p.d * 9, device="cuda")
    dl = torch.empty(1, device="cuda")
    lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, t["dY"], dQ, dK, dV, dw, dl, flags, ws)
    torch.cuda.synchronize()
    return dict(dQ=host(dQ), dK=host(dK), dV=host(dV), d_dwc=host(dw).reshape(p.heads * p.d, 3, 3),
                dlam=float(host(dl)[0]))


PARAM_CASES = [
    WL.TRAIN_S1.replace(name="train_s1_B2", B=2),
    # m N = 729, not a multiple of 4: the lambda reduction takes its entry-by-entry path throughout
    WL.TINY.replace(name="train_9x9_r3", B=2, H=9, W=9, r=3, whiten=True, backward=True),
    WL.TINY.replace(name="train_tiny_whiten_h2", B=2, heads=2, whiten=True, backward=True),
    WL.TINY.replace(name="train_ragged_10x6_d32", H=10, W=6, d=32, r=2, whiten=True, backward=True),
    WL.TRAIN_S1.replace(name="train_s1_bf16_B2", B=2, dtype=WL.BF16),
    # 26 Newton-Schulz steps: the forward's saved iterates come from three runs of coupled steps, each started from
    # T = W X formed afresh, and the reverse chain walks back through all of them.
    WL.TINY.replace(name="train_12x12_K26", B=2, H=12, W=12, r=2, ns_iters=26, whiten=True, backward=True,
                    qk_dist="student_t"),
]


@pytest.mark.parametrize("wl", PARAM_CASES, ids=lambda w: w.name)
def test_param_grads_match_oracle(wl):
    """DWC weight gradient (summed over the batch per head) and lambda gradient, alpha held constant; dQ, dK and
    dV of the extended call are bitwise those of lf_attn_bwd."""
    note(f"[gpu] parameter gradients {wl.name}")
    inp = inputs(wl)
    ref = O.backward(inp["Q"], inp["K"], inp["V"], inp["w64"], inp["dY"], oparams(wl))
    g = _gpu_backward_ex(wl, 0)
    e_w = relF(g["d_dwc"], ref["d_dwc"])
    e_l = abs(g["dlam"] - ref["dlam"]) / abs(ref["dlam"])
    note(f"    d_dwc={e_w:.3e} dlambda={e_l:.3e} ({g['dlam']:.6e} vs {ref['dlam']:.6e})")
    assert e_w <= tol(wl)
    assert e_l <= tol(wl)
    dQ, dK, dV = _gpu_backward(wl)
    assert np.array_equal(dQ, g["dQ"]) and np.array_equal(dK, g["dK"]) and np.array_equal(dV, g["dV"])


def test_exact_alpha_matches_oracle():
    """One Newton-Schulz step and lambda = 16 (a landmark kernel matrix far from diagonal), so X_K depends on alpha:
    the exact gradients match the oracle's, and they differ from the constant-alpha ones by more than the bar."""
    wl = WL.TINY.replace(name="tiny_exact_alpha", B=2, lam=16.0, ns_iters=1, whiten=True, backward=True)
    note(f"[gpu] exact alpha {wl.name}")
    inp = inputs(wl)
    ref = O.backward(inp["Q"], inp["K"], inp["V"], inp["w64"], inp["dY"], oparams(wl), exact_alpha=True)
    ref0 = O.backward(inp["Q"], inp["K"], inp["V"], inp["w64"], inp["dY"], oparams(wl))
    g = _gpu_backward_ex(wl, lf.LF_BWD_EXACT_ALPHA)
    errs = {n: relF(g[n], ref[n]) for n in ("dQ", "dK", "dV")}
    errs["dlam"] = abs(g["dlam"] - ref["dlam"]) / abs(ref["dlam"])
    note("    " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= tol(wl), (n, e)
    assert relF(ref0["dQ"], ref["dQ"]) > 10 * tol(wl)
    assert abs(ref0["dlam"] - ref["dlam"]) > 10 * tol(wl) * abs(ref["dlam"])


def test_backward_on_a_user_stream_is_ordered_and_bitwise_stable():
    """On a user stream, two calls in a row (the second with other dY and a workspace filled with garbage) give the
    gradients of calls on the current stream bit for bit, and each output is complete when the user stream's next
    work (a copy) runs: lf_attn_bwd on the one stream, and lf_attn_bwd_ex with a lent second stream (its fork and
    join events are the caller's)."""
    note("[gpu] backward on a user stream")
    wl = WL.TRAIN_S1.replace(name="train_s1_B2", B=2)
    p = params(wl)
    t = upload(wl)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, saved, ws)
    dY2 = torch.flip(t["dY"], dims=[0]).contiguous()
    outs_ref = []
    for dy in (t["dY"], dY2):
        g = [torch.empty_like(t["Q"]) for _ in range(3)] + [torch.empty(p.heads * p.d * 9, device="cuda"),
                                                            torch.empty(1, device="cuda")]
        lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, dy, *g, 0, ws)
        outs_ref.append(g)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    aux = lf.AuxStream()
    s.wait_stream(torch.cuda.current_stream())
    single, lent = [], []
    with torch.cuda.stream(s):
        ws.fill_(0xA5)
        for dy in (t["dY"], dY2):
            dQ, dK, dV = torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])
            lf.lf_attn_bwd(p, t["Q"], t["K"], t["V"], t["w"], saved, dy, dQ, dK, dV, ws, stream=s)
            single.append(tuple(x.clone() for x in (dQ, dK, dV)))  # runs on s right after the call's work
        ws.fill_(0x5A)
        for dy in (t["dY"], dY2):
            g = [torch.empty_like(t["Q"]) for _ in range(3)] + [torch.empty(p.heads * p.d * 9, device="cuda"),
                                                                torch.empty(1, device="cuda")]
            lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, dy, *g, 0, ws, stream=s, aux=aux)
            lent.append(tuple(x.clone() for x in g))
    s.synchronize()
    for got, ref in zip(single, outs_ref):
        for a, b in zip(got, ref[:3]):
            assert torch.equal(a, b)
    for got, ref in zip(lent, outs_ref):
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


def test_training_op_is_equivariant_under_slice_permutation():
    """Reordering the batch entries and the heads (with each head's DWC filters) reorders dQ, dK and dV bit for bit
    and the per-head DWC weight gradient with the heads; the batch sums (DWC weights, lambda) change only by the
    order of their additions."""
    wl = WL.TRAIN_S1.replace(name="train_B4_h2_14x14", B=4, heads=2, H=14, W=14, r=2)
    note(f"[gpu] training op slice permutation {wl.name}")
    rng = np.random.default_rng(4)
    pb, ph = rng.permutation(wl.B), rng.permutation(wl.heads)
    inp = inputs(wl)
    d = wl.d
    sets = [{k: inp[k + "_raw"] for k in ("Q", "K", "V", "dY")} | {"w": inp["w"]},
            {k: np.ascontiguousarray(inp[k + "_raw"][pb][:, ph]) for k in ("Q", "K", "V", "dY")}
            | {"w": np.ascontiguousarray(np.concatenate([inp["w"][h * d:(h + 1) * d] for h in ph]))}]
    p = params(wl)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    res = []
    for s in sets:
        t = {k: dev(v) for k, v in s.items()}
        Y = torch.empty_like(t["Q"])
        lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, saved, ws)
        g = [torch.empty_like(t["Q"]) for _ in range(3)]
        dw = torch.empty(wl.heads * d * 9, device="cuda")
        dl = torch.empty(1, device="cuda")
        lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, t["dY"], *g, dw, dl, 0, ws)
        torch.cuda.synchronize()
        res.append(([x.cpu() for x in g], dw.cpu().view(wl.heads, d * 9), float(dl.cpu()[0])))
    (g0, dw0, dl0), (g1, dw1, dl1) = res
    ib, ih = torch.as_tensor(pb), torch.as_tensor(ph)
    for a, b in zip(g1, g0):
        assert torch.equal(a, b[ib][:, ih])
    assert relF(dw1.numpy(), dw0[ih].numpy()) <= 1e-6
    assert abs(dl1 - dl0) <= 1e-6 * abs(dl0)
