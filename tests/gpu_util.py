"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle as O
from laplacian_nystr_vit_amd import lf
from laplacian_nystr_vit_amd import workloads as WL

# Bars from the contract: relative Frobenius error of the GPU result against the fp64 oracle.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# Intermediates computed in float32 (L, the kernel matrices, X_K, S, P) are gated at the float32 bar whatever the
# input dtype: a bf16 input only changes the numbers they start from, which the oracle receives too.
TOL_STAGE = TOL_F32


def tol(wl) -> float:
    return TOL_BF16 if wl.dtype == WL.BF16 else TOL_F32


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def params(wl, **kw) -> lf.LfAttnParams:
    p = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, wl.ns_iters, wl.whiten,
                       wl.whiten_eps, torch.bfloat16 if wl.dtype == WL.BF16 else torch.float32, wl.kernel)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def oparams(wl) -> O.Params:
    return O.Params(B=wl.B, heads=wl.heads, H=wl.H, W=wl.W, d=wl.d, r=wl.r, lam=wl.lam, eps=wl.eps,
                    ns_iters=wl.ns_iters, whiten=wl.whiten, whiten_eps=wl.whiten_eps, kernel=wl.kernel)


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    """Host array -> device tensor. uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
        if dtype is not None:
            t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def relF(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


@functools.lru_cache(maxsize=None)
def inputs(wl, seed: int = 0):
    return WL.make_inputs(wl, seed=seed, with_dy=True)


@functools.lru_cache(maxsize=None)
def oracle_forward(wl, seed: int = 0):
    inp = inputs(wl, seed)
    return O.forward(inp["Q"], inp["K"], inp["V"], inp["w64"], oparams(wl))


def upload(wl, seed: int = 0):
    inp = inputs(wl, seed)
    return {"Q": dev(inp["Q_raw"]), "K": dev(inp["K_raw"]), "V": dev(inp["V_raw"]), "dY": dev(inp["dY_raw"]),
            "w": dev(inp["w"])}


def gpu_forward(wl, seed: int = 0, dwc: bool = True, save: bool = True):
    """Runs lf_attn_fwd through the C ABI. Returns (Y, saved views or None, params)."""
    p = params(wl)
    t = upload(wl, seed)
    fwd_b, saved_b, _ = lf.lf_attn_query(p)
    ws = torch.empty(fwd_b, dtype=torch.uint8, device="cuda")
    saved = torch.empty(saved_b, dtype=torch.uint8, device="cuda") if save else None
    Y = torch.empty_like(t["Q"])
    lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"] if dwc else None, Y, saved, ws)
    torch.cuda.synchronize()
    views = lf.saved_views(p, saved) if save else None
    return Y, views, p
