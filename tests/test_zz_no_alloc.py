"""The allocation-free forward (lf_attn_fwd_noalloc) against lf_attn_fwd through the C ABI.

It launches the same kernels on the library's static scratch array instead of a caller workspace, so its output must
be bitwise lf_attn_fwd's; it is also checked against the fp64 oracle at the contract's bar. Two calls in a row, the
second on a smaller input, so that the second one runs on what the first left in the array."""

import pytest
import torch

from gpu_util import gpu_forward, host, note, oracle_forward, params, relF, tol, upload
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

pytestmark = pytest.mark.gpu

PAIRS = [
    (WL.PVT_S1, WL.TINY),
    (WL.HIRES_BF16, WL.PVT_S3.replace(name="s3_B2_h5", B=2)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda pr: f"{pr[0].name}-then-{pr[1].name}")
def test_noalloc_forward_matches_workspace_forward(pair):
    results = []
    for wl in pair:
        note(f"[gpu] noalloc forward {wl.name}")
        p = params(wl)
        t = upload(wl)
        Y = torch.empty_like(t["Q"])
        Ya = torch.empty_like(t["Q"])
        lf.lf_attn_fwd_noalloc(p, t["Q"], t["K"], t["V"], t["w"], Y)
        lf.lf_attn_fwd_noalloc(p, t["Q"], t["K"], t["V"], None, Ya)
        torch.cuda.synchronize()
        results.append((wl, Y, Ya))
    for wl, Y, Ya in results:
        Yref, _, _ = gpu_forward(wl, dwc=True, save=False)
        Yaref, _, _ = gpu_forward(wl, dwc=False, save=False)
        assert torch.equal(Y, Yref), wl.name
        assert torch.equal(Ya, Yaref), wl.name
        ref = oracle_forward(wl)
        e_full, e_attn = relF(host(Y), ref["Y"]), relF(host(Ya), ref["Yattn"])
        note(f"    {wl.name}: relF full={e_full:.3e} attn={e_attn:.3e}")
        assert e_full <= tol(wl) and e_attn <= tol(wl)


def test_noalloc_forward_on_a_user_stream():
    """On a user stream the output is complete when the stream's next work runs, and equal to the current-stream
    result."""
    wl = WL.PVT_S1.replace(name="s1_B2", B=2)
    note(f"[gpu] noalloc forward on a user stream {wl.name}")
    p = params(wl)
    t = upload(wl)
    Yref, _, _ = gpu_forward(wl, dwc=True, save=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        Y = torch.empty_like(t["Q"])
        lf.lf_attn_fwd_noalloc(p, t["Q"], t["K"], t["V"], t["w"], Y, stream=s)
        Yc = Y.clone()
    s.synchronize()
    assert torch.equal(Yc, Yref)


def test_noalloc_rejects_a_shape_beyond_its_array():
    """A shape whose forward workspace exceeds the static array is refused on the host (LF_EWORKSPACE). The call gets
    small placeholder tensors, which no launch may read: the library must refuse before launching anything."""
    import ctypes

    wl = WL.HIRES_BF16.replace(name="hires_B4", B=4)
    p = params(wl)
    fwd, _, _ = lf.lf_attn_query(p)
    assert fwd > lf.LF_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(64, device="cuda")
    y = torch.zeros(64, device="cuda")
    rc = lf.load_library().lf_attn_fwd_noalloc(ctypes.byref(p), x.data_ptr(), x.data_ptr(), x.data_ptr(), None,
                                                y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == lf.LF_EWORKSPACE
    assert torch.count_nonzero(y) == 0
