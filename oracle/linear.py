"""Oracle: the QLoRA linear layer, forward and backward, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer (QLoRA vs ChatGPT page, capability rows "LoRA on the quantized
base" and "training pipeline"): the base weight is frozen and stored in NF4 +
DQ, it is dequantized block by block for the matmul, and a full-precision
low-rank adapter is added. With W-hat the dequantized weight [N, K],
A [r, K], B [N, r] and the LoRA scale s:

    Y  = X W-hat^T + s (X A^T) B^T                      (forward)

Gradients flow only to the adapter and to the input; the base gets none
(the same page: gradients are computed only for the LoRA parameters). With
upstream gradient dY [M, N]:

    dH = s dY B                     [M, r]
    dX = dY W-hat + dH A            [M, K]
    dA = dH^T X                     [r, K]
    dB = s dY^T (X A^T)             [N, r]

All products are fp64 matmuls of the exact inputs (bf16 X and dY widened
exactly, fp32 W-hat, A and B). No rounding is applied to the results.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def forward(X, W_hat, A, B, s):
    """Y = X W-hat^T + s (X A^T) B^T in fp64. A and B may be None (no adapter)."""
    X, W_hat, A, B = _f64(X), _f64(W_hat), _f64(A), _f64(B)
    Y = X @ W_hat.T
    if A is not None and B is not None and A.shape[0] > 0:
        H = X @ A.T
        Y = Y + float(s) * (H @ B.T)
    return Y


def lora_down(X, A):
    """H = X A^T in fp64 (the adapter's down projection)."""
    return _f64(X) @ _f64(A).T


def backward(dY, X, W_hat, A, B, s):
    """Returns (dX, dA, dB) in fp64; dA and dB are None without an adapter."""
    dY, X, W_hat, A, B = _f64(dY), _f64(X), _f64(W_hat), _f64(A), _f64(B)
    dX = dY @ W_hat
    if A is None or B is None or A.shape[0] == 0:
        return dX, None, None
    dH = float(s) * (dY @ B)
    dX = dX + dH @ A
    dA = dH.T @ X
    H = X @ A.T
    dB = float(s) * (dY.T @ H)
    return dX, dA, dB


def rel_fro(got, ref) -> float:
    """Relative Frobenius error ||got - ref||_F / ||ref||_F (0 if both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


__all__ = ["forward", "lora_down", "backward", "rel_fro"]
