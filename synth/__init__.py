"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and rounds them to the storage types the layer consumes
(bf16 by round-to-nearest-even, fp32 as drawn). It holds none of the method's
arithmetic: no codebook, no quantization, no matmul.

Weights stand in for trained LLaMA projections. The QLoRA paper (as reviewed on
the ai-papercheck page "QLoRA: Efficient Finetuning of Quantized LLMs", finding
on Appendix F) reports that trained weights are close to normal, so the
workloads draw them from N(0, sigma) with the shapes of the 7B and 65B layers.

bf16 tensors are carried on the host as ``numpy.uint16`` bit patterns; the
helper ``bf16_to_f32`` widens them exactly (a 16-bit shift).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "f32_to_bf16", "bf16_to_f32", "normal_f32", "normal_bf16", "Workload",
    "make_linear_workload", "WORKLOADS", "lora_scale",
]


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. Inputs must be finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the fp32 values they encode, exactly."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """fp32 samples of N(0, sigma^2): a standard normal draw scaled by sigma in fp32."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    return z


def normal_bf16(rng: np.random.Generator, shape, sigma: float,
                outlier_frac: float = 0.0, outlier_mult: float = 10.0) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma^2) samples.

    With ``outlier_frac`` > 0 a seeded Bernoulli mask picks that fraction of the
    entries and multiplies them by ``outlier_mult`` before the bf16 rounding
    (the "1% outliers at 10x scale" of the 65B workload).
    """
    z = normal_f32(rng, shape, sigma)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < np.float32(outlier_frac)
        z[mask] *= np.float32(outlier_mult)
    return f32_to_bf16(z)


def lora_scale(alpha: float, r: int) -> float:
    """LoRA scale s = alpha / r (the usual LoRA scaling; the pages leave it open)."""
    return float(alpha) / float(r) if r > 0 else 0.0


@dataclasses.dataclass
class Workload:
    """One QLoRA-linear problem instance.

    W is [N, K] (out_features x in_features), X is [M, K], Y and dY are [M, N],
    A is [r, K], B is [N, r]. ``w_dtype`` is "f32" or "bf16"; bf16 arrays hold
    uint16 bit patterns, f32 arrays hold float32.
    """
    name: str
    M: int
    N: int
    K: int
    r: int
    alpha: float
    w_dtype: str
    W: np.ndarray
    X: np.ndarray          # bf16 bits [M, K]
    A: Optional[np.ndarray]  # f32 [r, K]
    B: Optional[np.ndarray]  # f32 [N, r]
    dY: Optional[np.ndarray]  # bf16 bits [M, N]

    @property
    def s(self) -> float:
        return lora_scale(self.alpha, self.r)

    def W_f32(self) -> np.ndarray:
        return self.W if self.w_dtype == "f32" else bf16_to_f32(self.W)


def make_linear_workload(name: str, M: int, N: int, K: int, r: int, alpha: float,
                         seed: int, w_dtype: str = "bf16", w_sigma: float = 0.02,
                         outlier_frac: float = 0.0, with_dy: bool = True,
                         lora_sigma: float = 0.01) -> Workload:
    """Draw a seeded workload. Every tensor comes from one PCG64 stream in a
    fixed order (W, X, A, B, dY), so a (name, seed) pair fixes every byte."""
    rng = np.random.default_rng(seed)
    if w_dtype == "f32":
        W = normal_f32(rng, (N, K), w_sigma)
        if outlier_frac > 0.0:
            mask = rng.random(size=(N, K), dtype=np.float32) < np.float32(outlier_frac)
            W[mask] *= np.float32(10.0)
    elif w_dtype == "bf16":
        W = normal_bf16(rng, (N, K), w_sigma, outlier_frac=outlier_frac)
    else:
        raise ValueError(w_dtype)
    X = normal_bf16(rng, (M, K), 1.0)
    A = normal_f32(rng, (r, K), lora_sigma) if r > 0 else None
    B = normal_f32(rng, (N, r), lora_sigma) if r > 0 else None
    dY = normal_bf16(rng, (M, N), 1.0) if with_dy else None
    return Workload(name, M, N, K, r, alpha, w_dtype, W, X, A, B, dY)


# The workloads of the benchmark table, by name. Each entry gives the keyword
# arguments of make_linear_workload (seed included).
WORKLOADS: Dict[str, dict] = {
    # Tiny QLoRA linear: W fp32 256x256, X 16x256, r=8, alpha=16.
    "tiny": dict(M=16, N=256, K=256, r=8, alpha=16.0, seed=1, w_dtype="f32"),
    # Llama-7B attention projection, 4 x 1024 tokens, r=64, alpha=16.
    "attn7b": dict(M=4096, N=4096, K=4096, r=64, alpha=16.0, seed=7, w_dtype="bf16"),
    # Llama-7B MLP decode shapes (forward only), M in {1, 4, 16}.
    "gate7b_m1": dict(M=1, N=11008, K=4096, r=64, alpha=16.0, seed=11, with_dy=False),
    "gate7b_m4": dict(M=4, N=11008, K=4096, r=64, alpha=16.0, seed=12, with_dy=False),
    "gate7b_m16": dict(M=16, N=11008, K=4096, r=64, alpha=16.0, seed=13, with_dy=False),
    "down7b_m1": dict(M=1, N=4096, K=11008, r=64, alpha=16.0, seed=21, with_dy=False),
    "down7b_m4": dict(M=4, N=4096, K=11008, r=64, alpha=16.0, seed=22, with_dy=False),
    "down7b_m16": dict(M=16, N=4096, K=11008, r=64, alpha=16.0, seed=23, with_dy=False),
    # Llama-65B MLP, 2048 tokens, 1% outliers at 10x in W.
    "up65b": dict(M=2048, N=22016, K=8192, r=64, alpha=16.0, seed=65, outlier_frac=0.01),
    "down65b": dict(M=2048, N=8192, K=22016, r=64, alpha=16.0, seed=66, outlier_frac=0.01),
}


def workload(name: str, **overrides) -> Workload:
    """Build a named workload from WORKLOADS (keyword overrides allowed)."""
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return make_linear_workload(name, **kw)


# Whole-model stack of a 65B-shaped decoder: per layer four 8192x8192
# attention projections and three MLP matrices (two 22016x8192, one 8192x22016).
STACK65B_LAYERS = 80
STACK65B_SHAPES = [(8192, 8192)] * 4 + [(22016, 8192), (22016, 8192), (8192, 22016)]
