"""Capture of whole calls in a HIP graph. The library enqueues only kernels and, for lf_attn_bwd_ex with a lent side
stream, event records and waits; it allocates, copies, clears and synchronises nothing. So a caller may capture a
forward, or a whole training step, and replay it. Each replay here runs with the outputs first set to NaN and an
eager call between replays, and must reproduce the eager call's outputs bit for bit."""

import pytest
import torch

from gpu_util import note, params, upload
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

pytestmark = pytest.mark.gpu

CASES = [
    WL.PVT_S1,                                  # inference forward (no saved buffer)
    WL.HIRES_BF16,                              # m > 64: the batched solver's launches
    WL.TRAIN_S1,                                # forward with saved buffer + full backward on two streams
    WL.TINY.replace(name="train_tiny_whiten_h2", B=2, heads=2, whiten=True, backward=True),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_graph_replay_is_bitwise_eager(wl):
    note(f"[gpu] graph capture {wl.name}")
    train = bool(wl.whiten) or getattr(wl, "backward", False)
    p = params(wl)
    t = upload(wl)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    ws = torch.empty(max(fwd_b, bwd_b if train else 0), dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda") if train else None
    Y = torch.empty_like(t["Q"])
    outs = [Y]
    if train:
        dQ, dK, dV = (torch.empty_like(t["Q"]) for _ in range(3))
        dw = torch.empty(wl.heads * wl.d * 9, device="cuda")
        dlam = torch.empty(1, device="cuda")
        outs += [dQ, dK, dV, dw, dlam]
        aux = lf.AuxStream()

    def step():
        st = torch.cuda.current_stream()
        lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y, saved, ws, st)
        if train:
            lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], saved, t["dY"], dQ, dK, dV, dw, dlam, 0, ws, st,
                              aux=aux)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call on the capture's stream kind, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager call"
        step()  # eager work between replays
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("wl", [WL.PVT_S1, WL.HIRES_BF16], ids=lambda w: w.name)
def test_graph_replay_of_the_noalloc_forward(wl):
    # the entry point for callers that cannot allocate, captured as such a caller would: every replay must match
    # the workspace forward's output bit for bit
    note(f"[gpu] graph capture of lf_attn_fwd_noalloc {wl.name}")
    p = params(wl)
    t = upload(wl)
    fwd_b, _, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    Y_ref = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y_ref, None, ws)
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd_noalloc(p, t["Q"], t["K"], t["V"], t["w"], Y, torch.cuda.current_stream())  # device set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lf.lf_attn_fwd_noalloc(p, t["Q"], t["K"], t["V"], t["w"], Y, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref), f"replay {rep} differs from the workspace forward"
        lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], Y_ref, None, ws)  # eager work between replays
        torch.cuda.synchronize()
    del g
