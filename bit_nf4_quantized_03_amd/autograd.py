"""torch.autograd wrapper of the QLoRA linear layer.

Marshalling only: the forward is one ``qlora_linear_fwd_save`` call, which
also keeps the adapter activations bf16(scale X A^T) [M, r], and the backward
one ``qlora_linear_bwd_saved`` call that takes them instead of forming them
again (``qlora_linear_fwd`` / ``qlora_linear_bwd`` without an adapter)
(QLoRA vs ChatGPT page, capability
"training pipeline": the 4-bit base is frozen and dequantized on the fly,
gradients go to the low-rank adapter and the input). It lets a caller compose
projections into a larger model with autograd, recompute them under
``torch.utils.checkpoint``, and gives the base weight no gradient.

Tensors: X bf16 [M, K] (any leading shape, flattened to M rows), A fp32
[r, K], B fp32 [N, r], on the weight's device. The output is bf16 [..., N].
"""
from __future__ import annotations

import torch

from . import NF4Weight, qlora_linear_bwd, qlora_linear_bwd_saved, qlora_linear_fwd, qlora_linear_fwd_save


class QLoRALinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, A, B, W: NF4Weight, scale: float):
        lead = X.shape[:-1]
        X2 = X.reshape(-1, X.shape[-1]).contiguous()
        if A is not None:
            Y, Hs = qlora_linear_fwd_save(X2, W, A, B, scale)
        else:
            Y, Hs = qlora_linear_fwd(X2, W, A, B, scale), None
        ctx.save_for_backward(X2, A, B, Hs)
        ctx.W, ctx.scale, ctx.lead = W, scale, lead
        return Y.reshape(*lead, W.rows)

    @staticmethod
    def backward(ctx, dY):
        X2, A, B, Hs = ctx.saved_tensors
        dY2 = dY.reshape(-1, ctx.W.rows).to(torch.bfloat16).contiguous()
        if Hs is not None:
            dX, dA, dB = qlora_linear_bwd_saved(dY2, X2, Hs, ctx.W, A, B, ctx.scale)
        else:
            dX, dA, dB = qlora_linear_bwd(dY2, X2, ctx.W, A, B, ctx.scale)
        return dX.reshape(*ctx.lead, ctx.W.cols), dA, dB, None, None


def qlora_linear(X, W: NF4Weight, A=None, B=None, scale: float = 0.0):
    """Y = X W-hat^T + scale (X A^T) B^T with autograd to X, A and B."""
    return QLoRALinearFn.apply(X, A, B, W, float(scale))
