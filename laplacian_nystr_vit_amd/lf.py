"""Thin ctypes binding of liblf_attn.so (include/lf_attn.h): argument marshalling only.

Every function here has the name of the C entry point it wraps and forwards to it. It accepts torch tensors
(device memory) and checks that they are CUDA tensors and contiguous, of the expected dtype and large enough.
It then passes their pointers and the current HIP stream. All computation happens in the library's HIP kernels;
there is no fallback. If the library has not been built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblf_attn.so")

LF_OK, LF_EINVAL, LF_EWORKSPACE, LF_EUNSUPPORTED, LF_EHIP = 0, -1, -2, -3, -4
LF_F32, LF_BF16 = 0, 1
LF_KERNEL_LAPLACE, LF_KERNEL_GAUSS = 0, 1
LF_M_MAX = 256
LF_NS_ITERS_MAX = 64

# Every symbol include/lf_attn.h declares.
EXPORTS = (
    "lf_attn_query", "lf_attn_saved_layout", "lf_attn_fwd", "lf_attn_bwd", "lf_strerror", "lf_landmark_pool",
    "lf_laplace_l1_exp", "lf_ns_pinv", "lf_ckv_reduce", "lf_whiten_stats", "lf_landmark_mix", "lf_out_gemm_dwc",
    "lf_out_gemm_dwc_fused", "lf_attn_bwd_ex", "lf_cg_pinv", "lf_gauss_l2_exp", "lf_attn_fwd_noalloc",
)
LF_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
LF_BWD_EXACT_ALPHA = 1
LF_CG_ITERS_MAX = 256


class LfAttnParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("heads", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("lambda_", ctypes.c_float), ("eps", ctypes.c_float),
        ("ns_iters", ctypes.c_int32), ("whiten", ctypes.c_int32), ("whiten_eps", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("kernel", ctypes.c_int32),
    ]

    @property
    def G(self) -> int:
        return self.B * self.heads

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def m(self) -> int:
        return (self.H // self.r) * (self.W // self.r)


class LfSavedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("L", "CQ", "CK", "We", "xs", "mu", "rstd", "S", "P", "alpha", "total")]


class LfAuxStream(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("fork", ctypes.c_void_p), ("join", ctypes.c_void_p)]


class AuxStream:
    """A second stream and two events the caller lends to lf_attn_bwd_ex (the library keeps no stream or event of
    its own). Owned by this object; torch creates them (default priority, events without timing)."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.fork = torch.cuda.Event(enable_timing=False)
        self.join = torch.cuda.Event(enable_timing=False)
        # torch creates an event's HIP handle on its first record
        self.fork.record(self.stream)
        self.join.record(self.stream)
        self.stream.synchronize()

    def as_c(self) -> LfAuxStream:
        return LfAuxStream(self.stream.cuda_stream, self.fork.cuda_event, self.join.cuda_event)


class LfError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {lf_strerror(code)} (status {code})")


_lib = None
_P = ctypes.POINTER(LfAttnParams)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads liblf_attn.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python laplacian_nystr_vit_amd/build.py`")
    lib = ctypes.CDLL(path)
    sig = {
        "lf_attn_query": (ctypes.c_int, [_P, ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "lf_attn_saved_layout": (ctypes.c_int, [_P, ctypes.POINTER(LfSavedLayout)]),
        "lf_attn_fwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "lf_attn_fwd_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp]),
        "lf_attn_bwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "lf_attn_bwd_ex": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int,
                                          _vp, _sz, _vp, ctypes.POINTER(LfAuxStream)]),
        "lf_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "lf_landmark_pool": (ctypes.c_int, [_P, _vp, _vp, _vp]),
        "lf_laplace_l1_exp": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "lf_gauss_l2_exp": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "lf_ns_pinv": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "lf_ckv_reduce": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _sz, _vp]),
        "lf_whiten_stats": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp]),
        "lf_landmark_mix": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp]),
        "lf_out_gemm_dwc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "lf_out_gemm_dwc_fused": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "lf_cg_pinv": (ctypes.c_int, [_P, _vp, _vp, _vp, ctypes.c_int32, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def make_params(B: int, heads: int, H: int, W: int, d: int, r: int, lam: float = 4.0, eps: float = 1e-3,
                ns_iters: int = 12, whiten: bool = False, whiten_eps: float = 1e-5,
                dtype: torch.dtype = torch.float32, kernel: str = "laplace") -> LfAttnParams:
    """kernel: "laplace" (exp(-||x-y||_1/lambda), the method) or "gauss" (exp(-||x-y||_2^2/lambda))."""
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be torch.float32 or torch.bfloat16")
    kernels = {"laplace": LF_KERNEL_LAPLACE, "gauss": LF_KERNEL_GAUSS}
    if kernel not in kernels:
        raise ValueError('kernel must be "laplace" or "gauss"')
    return LfAttnParams(B, heads, H, W, d, r, lam, eps, ns_iters, 1 if whiten else 0, whiten_eps,
                        LF_BF16 if dtype == torch.bfloat16 else LF_F32, kernels[kernel])


def io_dtype(p: LfAttnParams) -> torch.dtype:
    return torch.bfloat16 if p.dtype == LF_BF16 else torch.float32


def _check(rc: int, where: str) -> None:
    if rc != LF_OK:
        raise LfError(rc, where)


def _ptr(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None,
         numel: Optional[int] = None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def lf_strerror(code: int) -> str:
    return load_library().lf_strerror(code).decode()


def lf_attn_query(p: LfAttnParams) -> Tuple[int, int, int]:
    f, s, b = _sz(), _sz(), _sz()
    _check(load_library().lf_attn_query(ctypes.byref(p), ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)),
           "lf_attn_query")
    return f.value, s.value, b.value


def lf_attn_saved_layout(p: LfAttnParams) -> dict:
    lay = LfSavedLayout()
    _check(load_library().lf_attn_saved_layout(ctypes.byref(p), ctypes.byref(lay)), "lf_attn_saved_layout")
    return {n: getattr(lay, n) for n, _ in LfSavedLayout._fields_}


def lf_attn_fwd(p, Q, K, V, dwc_w, Y, saved, ws, stream=None) -> None:
    dt, n = io_dtype(p), p.G * p.N * p.d
    args = [_ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(V, "V", dt, n),
            _ptr(dwc_w, "dwc_w", torch.float32, p.heads * p.d * 9), _ptr(Y, "Y", dt, n)]
    fwd_b, saved_b, _ = lf_attn_query(p)
    if saved is not None and _nbytes(saved) < saved_b:
        raise ValueError(f"saved needs {saved_b} bytes")
    _check(load_library().lf_attn_fwd(ctypes.byref(p), *args, _ptr(saved, "saved"), _ptr(ws, "ws"), _nbytes(ws),
                                      _stream(stream)), "lf_attn_fwd")


def lf_attn_fwd_noalloc(p, Q, K, V, dwc_w, Y, stream=None) -> None:
    """The forward pass on the library's static device scratch array (no workspace argument, nothing allocated)."""
    dt, n = io_dtype(p), p.G * p.N * p.d
    _check(load_library().lf_attn_fwd_noalloc(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(V, "V", dt, n),
        _ptr(dwc_w, "dwc_w", torch.float32, p.heads * p.d * 9), _ptr(Y, "Y", dt, n), _stream(stream)),
        "lf_attn_fwd_noalloc")


def lf_attn_bwd(p, Q, K, V, dwc_w, saved, dY, dQ, dK, dV, ws, stream=None) -> None:
    dt, n = io_dtype(p), p.G * p.N * p.d
    _, saved_b, _ = lf_attn_query(p)
    if _nbytes(saved) < saved_b:
        raise ValueError(f"saved needs {saved_b} bytes")
    _check(load_library().lf_attn_bwd(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(V, "V", dt, n),
        _ptr(dwc_w, "dwc_w", torch.float32, p.heads * p.d * 9), _ptr(saved, "saved"), _ptr(dY, "dY", dt, n),
        _ptr(dQ, "dQ", dt, n), _ptr(dK, "dK", dt, n), _ptr(dV, "dV", dt, n), _ptr(ws, "ws"), _nbytes(ws),
        _stream(stream)), "lf_attn_bwd")


def lf_attn_bwd_ex(p, Q, K, V, dwc_w, saved, dY, dQ, dK, dV, d_dwc_w, d_lambda, flags, ws, stream=None,
                   aux: Optional[AuxStream] = None) -> None:
    """aux: None (every launch on `stream`) or an AuxStream lent for the independent parts of the work."""
    dt, n = io_dtype(p), p.G * p.N * p.d
    _, saved_b, _ = lf_attn_query(p)
    if _nbytes(saved) < saved_b:
        raise ValueError(f"saved needs {saved_b} bytes")
    ca = ctypes.byref(aux.as_c()) if aux is not None else None
    _check(load_library().lf_attn_bwd_ex(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(V, "V", dt, n),
        _ptr(dwc_w, "dwc_w", torch.float32, p.heads * p.d * 9), _ptr(saved, "saved"), _ptr(dY, "dY", dt, n),
        _ptr(dQ, "dQ", dt, n), _ptr(dK, "dK", dt, n), _ptr(dV, "dV", dt, n),
        _ptr(d_dwc_w, "d_dwc_w", torch.float32, p.heads * p.d * 9), _ptr(d_lambda, "d_lambda", torch.float32, 1),
        int(flags), _ptr(ws, "ws"), _nbytes(ws), _stream(stream), ca), "lf_attn_bwd_ex")


def lf_landmark_pool(p, Q, L, stream=None) -> None:
    _check(load_library().lf_landmark_pool(ctypes.byref(p), _ptr(Q, "Q", io_dtype(p), p.G * p.N * p.d),
                                           _ptr(L, "L", torch.float32, p.G * p.m * p.d), _stream(stream)),
           "lf_landmark_pool")


def lf_laplace_l1_exp(p, Q, K, L, CQ, CK, We, stream=None) -> None:
    dt, n = io_dtype(p), p.G * p.N * p.d
    f32, nm = torch.float32, p.G * p.N * p.m
    _check(load_library().lf_laplace_l1_exp(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(L, "L", f32, p.G * p.m * p.d),
        _ptr(CQ, "CQ", f32, nm), _ptr(CK, "CK", f32, nm), _ptr(We, "We", f32, p.G * p.m * p.m), _stream(stream)),
        "lf_laplace_l1_exp")


def lf_gauss_l2_exp(p, Q, K, L, CQ, CK, We, stream=None) -> None:
    dt, n = io_dtype(p), p.G * p.N * p.d
    f32, nm = torch.float32, p.G * p.N * p.m
    _check(load_library().lf_gauss_l2_exp(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(K, "K", dt, n), _ptr(L, "L", f32, p.G * p.m * p.d),
        _ptr(CQ, "CQ", f32, nm), _ptr(CK, "CK", f32, nm), _ptr(We, "We", f32, p.G * p.m * p.m), _stream(stream)),
        "lf_gauss_l2_exp")


def lf_ns_pinv(p, We, X, xs, alpha, resid, ws, stream=None) -> None:
    f32, mm = torch.float32, p.G * p.m * p.m
    _check(load_library().lf_ns_pinv(
        ctypes.byref(p), _ptr(We, "We", f32, mm), _ptr(X, "X", f32, mm),
        _ptr(xs, "xs", f32, mm * (p.ns_iters + 1)), _ptr(alpha, "alpha", f32, p.G), _ptr(resid, "resid", f32, p.G),
        _ptr(ws, "ws"), _nbytes(ws), _stream(stream)), "lf_ns_pinv")


def lf_cg_pinv(p, We, X, resid, iters, stream=None) -> None:
    f32, mm = torch.float32, p.G * p.m * p.m
    _check(load_library().lf_cg_pinv(
        ctypes.byref(p), _ptr(We, "We", f32, mm), _ptr(X, "X", f32, mm),
        _ptr(resid, "resid", f32, p.G * max(int(iters), 0)), int(iters), _stream(stream)), "lf_cg_pinv")


def lf_ckv_reduce(p, CK, V, S, ws, stream=None) -> None:
    _check(load_library().lf_ckv_reduce(
        ctypes.byref(p), _ptr(CK, "CK", torch.float32, p.G * p.N * p.m), _ptr(V, "V", io_dtype(p), p.G * p.N * p.d),
        _ptr(S, "S", torch.float32, p.G * p.m * p.d), _ptr(ws, "ws"), _nbytes(ws), _stream(stream)),
        "lf_ckv_reduce")


def lf_whiten_stats(p, CQ, mu, rstd, stream=None) -> None:
    f32 = torch.float32
    _check(load_library().lf_whiten_stats(
        ctypes.byref(p), _ptr(CQ, "CQ", f32, p.G * p.N * p.m), _ptr(mu, "mu", f32, p.G * p.m),
        _ptr(rstd, "rstd", f32, p.G * p.m), _stream(stream)), "lf_whiten_stats")


def lf_landmark_mix(p, X, S, rstd, P, stream=None) -> None:
    f32 = torch.float32
    _check(load_library().lf_landmark_mix(
        ctypes.byref(p), _ptr(X, "X", f32, p.G * p.m * p.m), _ptr(S, "S", f32, p.G * p.m * p.d),
        _ptr(rstd, "rstd", f32, p.G * p.m), _ptr(P, "P", f32, p.G * p.m * p.d), _stream(stream)), "lf_landmark_mix")


def lf_out_gemm_dwc(p, CQ, P, mu, V, dwc_w, Y, stream=None) -> None:
    f32, dt, n = torch.float32, io_dtype(p), p.G * p.N * p.d
    _check(load_library().lf_out_gemm_dwc(
        ctypes.byref(p), _ptr(CQ, "CQ", f32, p.G * p.N * p.m), _ptr(P, "P", f32, p.G * p.m * p.d),
        _ptr(mu, "mu", f32, p.G * p.m), _ptr(V, "V", dt, n), _ptr(dwc_w, "dwc_w", f32, p.heads * p.d * 9),
        _ptr(Y, "Y", dt, n), _stream(stream)), "lf_out_gemm_dwc")


def lf_out_gemm_dwc_fused(p, Q, L, P, V, dwc_w, Y, stream=None) -> None:
    """Y = C_Q P + DWC(V) with C_Q recomputed per tile from Q and the landmarks L (no whitening)."""
    f32, dt, n = torch.float32, io_dtype(p), p.G * p.N * p.d
    _check(load_library().lf_out_gemm_dwc_fused(
        ctypes.byref(p), _ptr(Q, "Q", dt, n), _ptr(L, "L", f32, p.G * p.m * p.d), _ptr(P, "P", f32, p.G * p.m * p.d),
        _ptr(V, "V", dt, n), _ptr(dwc_w, "dwc_w", f32, p.heads * p.d * 9), _ptr(Y, "Y", dt, n), _stream(stream)),
        "lf_out_gemm_dwc_fused")


# ------------------------------------------------------------------------------------------------------------
# Conveniences built only from the calls above plus torch allocation.
# ------------------------------------------------------------------------------------------------------------
def saved_views(p: LfAttnParams, saved: torch.Tensor) -> dict:
    """float32 views of the intermediates inside a `saved` buffer, shaped per slice (C_Q, C_K landmark-major)."""
    lay = lf_attn_saved_layout(p)
    G, N, m, d, K = p.G, p.N, p.m, p.d, p.ns_iters
    shapes = {"L": (G, m, d), "CQ": (G, m, N), "CK": (G, m, N), "We": (G, m, m), "xs": (G, K + 1, m, m),
              "mu": (G, m), "rstd": (G, m), "S": (G, m, d), "P": (G, m, d), "alpha": (G,)}
    out = {}
    for k, shp in shapes.items():
        n = 1
        for s in shp:
            n *= s
        out[k] = saved[lay[k]:lay[k] + 4 * n].view(torch.float32).view(shp)
    return out


class LaplacianAttention:
    """Owns the workspace and saved buffers for one parameter set and calls lf_attn_fwd / lf_attn_bwd."""

    def __init__(self, p: LfAttnParams, device="cuda"):
        self.p = p
        self.device = torch.device(device)
        self.fwd_bytes, self.saved_bytes, self.bwd_bytes = lf_attn_query(p)
        self.ws = torch.empty(max(self.fwd_bytes, self.bwd_bytes, 256), dtype=torch.uint8, device=self.device)
        self.saved: Optional[torch.Tensor] = None

    def forward(self, Q, K, V, dwc_w=None, save: bool = False, Y: Optional[torch.Tensor] = None):
        if Y is None:
            Y = torch.empty_like(Q)
        if save and self.saved is None:
            self.saved = torch.empty(self.saved_bytes, dtype=torch.uint8, device=self.device)
        lf_attn_fwd(self.p, Q, K, V, dwc_w, Y, self.saved if save else None, self.ws)
        return Y

    def backward(self, Q, K, V, dwc_w, dY):
        if self.saved is None:
            raise RuntimeError("forward(save=True) must run before backward")
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        lf_attn_bwd(self.p, Q, K, V, dwc_w, self.saved, dY, dQ, dK, dV, self.ws)
        return dQ, dK, dV
