"""Synthetic workloads for the LaplacianFormer attention block: shapes plus a seeded input generator.

This module holds none of the method's arithmetic. It only names the problem sizes and draws the random
inputs (Q, K, V, depthwise-conv weights, upstream gradient) that both the GPU path and the fp64 CPU oracle
consume, so that the two sides see bit-identical inputs.

The shapes follow the PVT backbone the LaplacianFormer note builds on (papernotes.org ICLR 2026 reading note
"LaplacianFormer：用拉普拉斯核重新思考线性注意力", section "整体框架" / framework): stage-1 (56x56 tokens) and
stage-3 (14x14 tokens) grids, plus a 128x128 high-resolution grid. Q and K are heavy-tailed (Student-t, nu=3,
scaled by 0.5) because the same note (section "研究背景与动机" / motivation) reports heavy-tailed query-key
distance statistics on trained vision transformers; the trained activations themselves are not available, so
these seeded draws stand in for them.

Generator: numpy ``default_rng(seed)`` (PCG64). Draw order Q, K, V, w, dY. Every draw is made in float64, cast
to float32 with round-to-nearest-even, and for bf16 workloads cast again to bf16 with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    d: int
    r: int
    lam: float
    eps: float
    ns_iters: int
    dtype: str = F32
    qk_dist: str = "student_t"  # "student_t" (0.5 * t_3) or "normal"
    whiten: bool = False
    whiten_eps: float = 1e-5
    backward: bool = False
    dwc: bool = True
    kernel: str = "laplace"  # or "gauss": exp(-||x - y||_2^2 / lambda) in place of the Laplacian kernel

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def m(self) -> int:
        return (self.H // self.r) * (self.W // self.r)

    @property
    def G(self) -> int:
        return self.B * self.heads

    @property
    def tokens(self) -> int:
        return self.B * self.heads * self.N

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny fp32 instance: 8x8 grid, d=16, r=2 -> m=16 (and the r=1 variant, m=N=64).
TINY = Workload("tiny_8x8_d16", B=1, heads=1, H=8, W=8, d=16, r=2, lam=4.0, eps=1e-3, ns_iters=20,
                qk_dist="normal")
TINY_R1 = TINY.replace(name="tiny_8x8_d16_r1", r=1)
# PVT stage-1 shape, fp32: B=8, 56x56 grid, d=64, r=8 -> m=49.
PVT_S1 = Workload("pvt_s1_56x56_m49", B=8, heads=1, H=56, W=56, d=64, r=8, lam=4.0, eps=1e-3, ns_iters=12)
# PVT stage-3 batched shape, fp32: B=64, 5 heads, 14x14 grid, r=2 -> m=49.
PVT_S3 = Workload("pvt_s3_14x14_m49", B=64, heads=5, H=14, W=14, d=64, r=2, lam=4.0, eps=1e-3, ns_iters=12)
# High-resolution shape, bf16 inputs: B=2, 128x128 grid, r=8 -> m=256.
HIRES_BF16 = Workload("hires_128x128_m256_bf16", B=2, heads=1, H=128, W=128, d=64, r=8, lam=4.0, eps=1e-4,
                      ns_iters=16, dtype=BF16)
# Training step at the PVT stage-1 shape: diagonal whitening on, forward + backward.
TRAIN_S1 = PVT_S1.replace(name="train_pvt_s1_56x56_m49", whiten=True, backward=True)
# The Gaussian-kernel variant at the stage-1 shape. Its landmark matrix is far worse conditioned (kappa ~ 740
# against ~ 13 for the Laplacian one on these inputs), so Newton-Schulz needs 24 steps to converge instead of 12.
GAUSS_S1 = PVT_S1.replace(name="gauss_pvt_s1_56x56_m49", kernel="gauss", ns_iters=24)

ALL = {w.name: w for w in (TINY, TINY_R1, PVT_S1, PVT_S3, HIRES_BF16, TRAIN_S1, GAUSS_S1)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns to float64."""
    u = b.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _draw(rng: np.random.Generator, shape, dist: str, scale: float = 1.0) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(shape)
    elif dist == "student_t":
        x = 0.5 * rng.standard_t(3.0, size=shape)
    else:
        raise ValueError(dist)
    return (x * scale).astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0, with_dy: Optional[bool] = None) -> Dict[str, np.ndarray]:
    """Seeded synthetic inputs for a workload.

    Returns a dict with, for each tensor X in Q, K, V (and dY when requested):
      ``X``      the values as float64 (exactly the numbers the GPU receives),
      ``X_raw``  the array to upload: float32, or uint16 bf16 bit patterns for bf16 workloads.
    plus ``w`` (float32 depthwise-conv weights [heads*d, 3, 3]) and ``w64`` (same as float64).
    Layout of Q, K, V, dY: [B, heads, N, d], token n = y*W + x.
    """
    if with_dy is None:
        with_dy = wl.backward
    rng = np.random.default_rng(seed)
    shape = (wl.B, wl.heads, wl.N, wl.d)
    out: Dict[str, np.ndarray] = {}
    draws = [("Q", wl.qk_dist), ("K", wl.qk_dist), ("V", "normal")]
    for name, dist in draws:
        out[name + "_f32"] = _draw(rng, shape, dist)
    w = _draw(rng, (wl.heads * wl.d, 3, 3), "normal", scale=1.0 / 3.0)
    if with_dy:
        out["dY_f32"] = _draw(rng, shape, "normal")
    result: Dict[str, np.ndarray] = {}
    for name in ("Q", "K", "V", "dY"):
        key = name + "_f32"
        if key not in out:
            continue
        x32 = out[key]
        if wl.dtype == BF16:
            bits = f32_to_bf16_bits(x32)
            result[name + "_raw"] = bits
            result[name] = bf16_bits_to_f64(bits)
        else:
            result[name + "_raw"] = x32
            result[name] = x32.astype(np.float64)
    result["w"] = w
    result["w64"] = w.astype(np.float64)
    return result


def spd_matrix(m: int, kappa: float, seed: int) -> np.ndarray:
    """Seeded synthetic symmetric positive definite m x m matrix with condition number kappa, rounded to float32
    and returned as float64 (exactly the numbers the GPU receives): a random orthonormal basis (QR of a Gaussian
    matrix) with eigenvalues spaced geometrically from 1 to kappa, symmetrised after the product. The solver
    claim of the pages is stated at kappa = 50."""
    rng = np.random.default_rng(seed)
    basis, _ = np.linalg.qr(rng.standard_normal((m, m)))
    a = (basis * np.geomspace(1.0, kappa, m)) @ basis.T
    return (0.5 * (a + a.T)).astype(np.float32).astype(np.float64)
