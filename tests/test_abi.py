"""C ABI contract checks that need no GPU: the library loads, exports every symbol include/lf_attn.h declares, and
rejects bad parameters on the host before anything is launched."""

import ctypes
import os
import re

import pytest
import torch

from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lf_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lf.LIB_PATH):
        from laplacian_nystr_vit_amd import build
        build.build()
    return lf.load_library()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lf_\w+)\s*\(", src, flags=re.M)))


def test_header_declarations_match_binding():
    assert sorted(lf.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {lf.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def _p(wl, **kw):
    p = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, wl.ns_iters, wl.whiten,
                       wl.whiten_eps, torch.bfloat16 if wl.dtype == WL.BF16 else torch.float32, wl.kernel)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("wl", list(WL.ALL.values()), ids=lambda w: w.name)
def test_query_sizes_and_saved_layout(lib, wl):
    p = _p(wl)
    fwd, saved, bwd = lf.lf_attn_query(p)
    G, N, m, d, K = p.G, p.N, p.m, p.d, p.ns_iters
    assert fwd >= 4 * G * (2 * N * m + m * d + m * m)
    lay = lf.lf_attn_saved_layout(p)
    sizes = {"L": G * m * d, "CQ": G * N * m, "CK": G * N * m, "We": G * m * m, "xs": G * (K + 1) * m * m,
             "mu": G * m, "rstd": G * m, "S": G * m * d, "P": G * m * d, "alpha": G}
    spans = sorted((lay[k], lay[k] + 4 * n) for k, n in sizes.items())
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert all(lay[k] % 256 == 0 for k in sizes)
    assert lay["total"] == saved >= spans[-1][1]
    if m <= 64 and d <= 64:
        assert bwd > 0
    else:
        assert bwd == 0


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, lf.LF_EINVAL), ("heads", -1, lf.LF_EINVAL), ("r", 3, lf.LF_EINVAL), ("r", 0, lf.LF_EINVAL),
    ("lambda_", 0.0, lf.LF_EINVAL), ("lambda_", float("nan"), lf.LF_EINVAL), ("eps", -1e-3, lf.LF_EINVAL),
    ("ns_iters", -1, lf.LF_EINVAL), ("ns_iters", 65, lf.LF_EINVAL), ("whiten", 2, lf.LF_EINVAL),
    ("dtype", 7, lf.LF_EINVAL), ("d", 48, lf.LF_EUNSUPPORTED), ("r", 1, lf.LF_EUNSUPPORTED),
    ("kernel", 2, lf.LF_EINVAL), ("kernel", -1, lf.LF_EINVAL),
])
def test_query_rejects_bad_params(lib, field, value, code):
    p = _p(WL.PVT_S1)  # 56x56 grid: r=1 gives m=3136 > LF_M_MAX, r=3 does not divide 56
    setattr(p, field, value)
    with pytest.raises(lf.LfError) as e:
        lf.lf_attn_query(p)
    assert e.value.code == code


def test_whiten_eps_must_be_positive_when_whitening(lib):
    p = _p(WL.TRAIN_S1, whiten_eps=0.0)
    with pytest.raises(lf.LfError) as e:
        lf.lf_attn_query(p)
    assert e.value.code == lf.LF_EINVAL


def test_null_params_and_strerror(lib):
    assert lib.lf_attn_query(None, None, None, None) == lf.LF_EINVAL
    for code in (lf.LF_OK, lf.LF_EINVAL, lf.LF_EWORKSPACE, lf.LF_EUNSUPPORTED, lf.LF_EHIP):
        assert len(lf.lf_strerror(code)) > 0


def test_fwd_rejects_null_pointers_and_small_workspace_without_launching(lib):
    p = _p(WL.TINY)
    fwd, _, _ = lf.lf_attn_query(p)
    # distinct fake device addresses; never dereferenced because validation fails before any launch
    q, k, v, y, ws = (ctypes.c_void_p(a << 20) for a in (1, 2, 3, 4, 5))
    assert lib.lf_attn_fwd(ctypes.byref(p), None, k, v, None, y, None, ws, fwd, None) == lf.LF_EINVAL
    assert lib.lf_attn_fwd(ctypes.byref(p), q, k, v, None, y, None, ws, fwd - 1, None) == lf.LF_EWORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 4)
    assert lib.lf_attn_fwd(ctypes.byref(p), misaligned, k, v, None, y, None, ws, fwd, None) == lf.LF_EINVAL
    assert lib.lf_attn_fwd(ctypes.byref(p), q, k, v, None, q, None, ws, fwd, None) == lf.LF_EINVAL  # Y aliases Q


def test_bwd_rejects_unsupported_shapes_on_host(lib):
    p = _p(WL.HIRES_BF16)  # m = 256
    fake = ctypes.c_void_p(0x100000)
    rc = lib.lf_attn_bwd(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert rc == lf.LF_EUNSUPPORTED


def test_binding_rejects_host_tensors(lib):
    p = _p(WL.TINY)
    q = torch.zeros(p.G * p.N * p.d)
    with pytest.raises(TypeError):
        lf.lf_landmark_pool(p, q, torch.zeros(p.G * p.m * p.d))


def test_bwd_ex_validates_flags_and_alignment_on_host(lib):
    p = _p(WL.TRAIN_S1)
    _, _, bwd = lf.lf_attn_query(p)
    fake = ctypes.c_void_p(0x100000)
    misaligned = ctypes.c_void_p(0x100004)
    # unknown flag bits, then a misaligned d_dwc_w: both rejected before anything is launched
    assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, None, None, 2,
                              fake, bwd, None, None) == lf.LF_EINVAL
    assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, misaligned,
                              None, 0, fake, bwd, None, None) == lf.LF_EINVAL
    assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, None, None,
                              lf.LF_BWD_EXACT_ALPHA, fake, bwd - 1, None, None) == lf.LF_EWORKSPACE


def test_bwd_ex_validates_the_lent_stream_on_host(lib):
    """A lent second stream with a missing handle, one event for both roles, or the call's own stream is rejected
    before anything is launched."""
    p = _p(WL.TRAIN_S1)
    _, _, bwd = lf.lf_attn_query(p)
    fake = ctypes.c_void_p(0x100000)
    st, ev1, ev2 = 0x200000, 0x300000, 0x400000
    bad = [lf.LfAuxStream(None, ev1, ev2), lf.LfAuxStream(st, None, ev2), lf.LfAuxStream(st, ev1, None),
           lf.LfAuxStream(st, ev1, ev1)]
    for aux in bad:
        assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, None, None,
                                  0, fake, bwd, None, ctypes.byref(aux)) == lf.LF_EINVAL
    same = lf.LfAuxStream(st, ev1, ev2)
    assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, None, None, 0,
                              fake, bwd, ctypes.c_void_p(st), ctypes.byref(same)) == lf.LF_EINVAL


def test_cg_validates_on_host(lib):
    """lf_cg_pinv rejects a step count outside 0..LF_CG_ITERS_MAX, misaligned pointers and m > 64 before launching."""
    p = _p(WL.PVT_S1)
    fake = ctypes.c_void_p(0x100000)
    misaligned = ctypes.c_void_p(0x100004)
    assert lib.lf_cg_pinv(ctypes.byref(p), fake, fake, None, -1, None) == lf.LF_EINVAL
    assert lib.lf_cg_pinv(ctypes.byref(p), fake, fake, None, lf.LF_CG_ITERS_MAX + 1, None) == lf.LF_EINVAL
    assert lib.lf_cg_pinv(ctypes.byref(p), fake, misaligned, None, 4, None) == lf.LF_EINVAL
    assert lib.lf_cg_pinv(ctypes.byref(p), None, fake, None, 4, None) == lf.LF_EINVAL
    assert lib.lf_cg_pinv(ctypes.byref(p), fake, fake, misaligned, 4, None) == lf.LF_EINVAL
    assert lib.lf_cg_pinv(ctypes.byref(_p(WL.HIRES_BF16)), fake, fake, None, 4, None) == lf.LF_EUNSUPPORTED


def test_gaussian_variant_is_forward_only_on_host(lib):
    """The Gaussian-kernel parameter set is valid for the forward pass and its stage call, and the backward pass and
    the fused (Laplacian) output stage reject it with LF_EUNSUPPORTED before launching."""
    p = _p(WL.GAUSS_S1)
    assert p.kernel == lf.LF_KERNEL_GAUSS
    fwd, saved, bwd = lf.lf_attn_query(p)
    assert fwd > 0 and saved > 0
    fake = ctypes.c_void_p(0x100000)
    assert lib.lf_attn_bwd(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, fake, bwd,
                           None) == lf.LF_EUNSUPPORTED
    assert lib.lf_attn_bwd_ex(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake, fake, None, None, 0,
                              fake, bwd, None, None) == lf.LF_EUNSUPPORTED
    assert lib.lf_out_gemm_dwc_fused(ctypes.byref(p), fake, fake, fake, fake, None, fake, None) == lf.LF_EUNSUPPORTED
    # the stage call validates its pointers before launching
    misaligned = ctypes.c_void_p(0x100004)
    assert lib.lf_gauss_l2_exp(ctypes.byref(p), fake, fake, fake, fake, misaligned, fake, None) == lf.LF_EINVAL
    assert lib.lf_gauss_l2_exp(ctypes.byref(p), fake, None, fake, fake, fake, fake, None) == lf.LF_EINVAL
    with pytest.raises(ValueError):
        lf.make_params(1, 1, 8, 8, 16, 2, kernel="cosine")


def test_fwd_noalloc_rejects_on_host(lib):
    """The allocation-free forward rejects, before touching the device, a shape whose forward workspace exceeds its
    static scratch array (LF_EWORKSPACE), and bad pointers or parameters (LF_EINVAL), like lf_attn_fwd."""
    m = re.search(r"#define LF_NOALLOC_SCRATCH_BYTES \(([0-9 *]+)\)", open(HEADER).read())
    assert m and eval(m.group(1), {"__builtins__": {}}) == lf.LF_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x100000)
    misaligned = ctypes.c_void_p(0x100004)
    big = _p(WL.HIRES_BF16.replace(B=4))
    fwd, _, _ = lf.lf_attn_query(big)
    assert fwd > lf.LF_NOALLOC_SCRATCH_BYTES
    assert lib.lf_attn_fwd_noalloc(ctypes.byref(big), fake, fake, fake, None, ctypes.c_void_p(0x200000),
                                   None) == lf.LF_EWORKSPACE
    p = _p(WL.PVT_S1)
    fwd, _, _ = lf.lf_attn_query(p)
    assert fwd <= lf.LF_NOALLOC_SCRATCH_BYTES
    assert lib.lf_attn_fwd_noalloc(ctypes.byref(p), misaligned, fake, fake, None, ctypes.c_void_p(0x200000),
                                   None) == lf.LF_EINVAL
    assert lib.lf_attn_fwd_noalloc(ctypes.byref(p), fake, fake, fake, None, fake, None) == lf.LF_EINVAL  # Y == Q
    assert lib.lf_attn_fwd_noalloc(ctypes.byref(p), fake, fake, fake, None, None, None) == lf.LF_EINVAL
    bad = _p(WL.PVT_S1)
    bad.r = 5  # 56 % 5 != 0
    assert lib.lf_attn_fwd_noalloc(ctypes.byref(bad), fake, fake, fake, None, ctypes.c_void_p(0x200000),
                                   None) == lf.LF_EINVAL
