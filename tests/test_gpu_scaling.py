"""Exact linearity under power-of-two scaling. Y is linear in V, and every gradient of <dY, Y> is linear in dY. The
products that run on the fp16 MFMA in split form (x = hi + lo) scale each operand tile by a power of two taken from
its own largest entry, and everything else is fp32 arithmetic. So scaling V (or dY) by 2^k must scale every output
by exactly 2^k, bit for bit, for k far beyond the fp16 range: a conversion to fp16 with a fixed scale would
overflow or flush there and break the equality. Also: the C_K^T V stage on a signed C of large entries (the stage
entry point takes any C, not only kernel values in [0, 1]) against its plain definition."""

import numpy as np
import pytest
import torch

from gpu_util import host, note, params, relF, upload
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

pytestmark = pytest.mark.gpu

FWD = [WL.PVT_S1, WL.PVT_S3, WL.HIRES_BF16, WL.TINY.replace(name="tiny_r1_m64", r=1),
       WL.TINY.replace(name="ragged_18x14_m63", H=18, W=14, r=2, d=32)]
BWD = [WL.TRAIN_S1, WL.TRAIN_S1.replace(name="train_s1_bf16_B2", B=2, dtype=WL.BF16),
       WL.TINY.replace(name="train_tiny_whiten_h2", B=2, heads=2, whiten=True, backward=True)]


def _pow2(k):
    return float(2.0 ** k)


@pytest.mark.parametrize("k", [-24, 24])
@pytest.mark.parametrize("wl", FWD, ids=lambda w: w.name)
def test_forward_is_exactly_linear_in_v(wl, k):
    note(f"[gpu] forward scaling {wl.name} k={k}")
    p = params(wl)
    t = upload(wl)
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    Y1, Y2 = torch.empty_like(t["Q"]), torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y1, None, ws)
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"] * _pow2(k), t["w"], Y2, None, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(Y2).all()
    assert torch.equal(Y2, Y1 * _pow2(k))


@pytest.mark.parametrize("k", [-20, 20])
@pytest.mark.parametrize("wl", BWD, ids=lambda w: w.name)
def test_gradients_are_exactly_linear_in_dy(wl, k):
    note(f"[gpu] backward scaling {wl.name} k={k}")
    p = params(wl)
    t = upload(wl)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, saved, ws)

    def grads(dY):
        out = [torch.empty_like(t["Q"]) for _ in range(3)]
        dw = torch.empty(wl.heads * wl.d * 9, device="cuda")
        dlam = torch.empty(1, device="cuda")
        lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, dY, *out, dw, dlam, 0, ws)
        return out + [dw, dlam]

    g1 = grads(t["dY"])
    g2 = grads(t["dY"] * _pow2(k))
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "d_dwc_w", "d_lambda"), g1, g2):
        assert torch.isfinite(b).all(), name
        assert torch.equal(b, a * _pow2(k)), name


@pytest.mark.parametrize("wl", [WL.TINY, WL.PVT_S1, WL.HIRES_BF16], ids=lambda w: w.name)
def test_ckv_stage_on_signed_large_c(wl):
    # C with entries of both signs up to about 3e5 and V down to about 1e-5: S = C^T V against its fp64 definition
    note(f"[gpu] ckv stage, signed C {wl.name}")
    p = params(wl)
    G, N, m, d = p.G, p.N, p.m, p.d
    rng = np.random.default_rng(7)
    C = (rng.standard_normal((G, N, m)) * 2.0 ** 16).astype(np.float32)
    C[:, : min(N, 64), :] = 0.0  # a whole chunk of zeros
    t = upload(wl)
    V = t["V"] * _pow2(-16)
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    S = torch.empty(G * m * d, device="cuda")
    lf.lf_ckv_reduce(p, torch.from_numpy(np.ascontiguousarray(C.transpose(0, 2, 1))).cuda(), V, S, ws)
    torch.cuda.synchronize()
    Vh = host(V).reshape(G, N, d)
    Sref = np.einsum("gil,gic->glc", C.astype(np.float64), Vh)
    assert relF(host(S).reshape(G, m, d), Sref) <= 1e-5
