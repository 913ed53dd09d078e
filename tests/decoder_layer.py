"""A LLaMA-style decoder layer built from seven QLoRA projections, for the
composed-layer parity test and the layer benchmark.

The projections (q, k, v, o of attention; gate, up, down of the SwiGLU MLP)
are the QLoRA linear layer of the pages (QLoRA vs ChatGPT page, capability
"training pipeline": a frozen 4-bit base dequantized on the fly plus a
trainable low-rank adapter, applied to every linear layer of the
transformer). The glue between them (RMSNorm, causal softmax attention,
SiLU gating, residual adds) is the standard decoder layer the pages'
models use; the pages do not define it further, so it is written here with
plain torch operations and serves only to compose the projections:

    h1 = rmsnorm(x) g1
    q, k, v = h1 Wq^T, h1 Wk^T, h1 Wv^T          (each with its adapter)
    o  = softmax(q k^T / sqrt(dh) + causal mask) v   per head
    x2 = x + o Wo^T
    h2 = rmsnorm(x2) g2
    y  = x2 + (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T

`layer_forward` takes the projection as a callable, so the same composition
runs on the GPU kernels (bf16 operands, fp32 glue) and on the fp64 oracle.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

import synth

NAMES = ("q", "k", "v", "o", "gate", "up", "down")


@dataclasses.dataclass
class LayerSpec:
    d: int          # hidden width
    f: int          # MLP width
    heads: int
    r: int          # adapter rank
    alpha: float

    def shape(self, name):
        """(out_features, in_features) of projection `name`."""
        if name in ("q", "k", "v", "o"):
            return self.d, self.d
        if name in ("gate", "up"):
            return self.f, self.d
        return self.d, self.f

    @property
    def scale(self) -> float:
        return synth.lora_scale(self.alpha, self.r)


def make_params(spec: LayerSpec, seed: int):
    """Seeded fp32 host arrays: base weights W ~ N(0, 0.02) rounded to bf16 (the
    stored base the quantizer reads), adapters A, B ~ N(0, 0.01), RMSNorm gains
    near 1."""
    rng = np.random.default_rng(seed)
    p = {}
    for name in NAMES:
        n, k = spec.shape(name)
        w = synth.bf16_to_f32(synth.f32_to_bf16(synth.normal_f32(rng, (n, k), 0.02)))
        p[name] = (w, synth.normal_f32(rng, (spec.r, k), 0.01), synth.normal_f32(rng, (n, spec.r), 0.01))
    p["g1"] = (1.0 + synth.normal_f32(rng, (spec.d,), 0.1)).astype(np.float32)
    p["g2"] = (1.0 + synth.normal_f32(rng, (spec.d,), 0.1)).astype(np.float32)
    return p


def rmsnorm(x, g, eps: float = 1e-6):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g


def layer_forward(x, lin, g1, g2, heads: int):
    """x [b, T, d]; lin(name, h) applies projection `name` to h [b, T, in]."""
    b, T, d = x.shape
    dh = d // heads
    h1 = rmsnorm(x, g1)

    def split(t):
        return t.reshape(b, T, heads, dh).transpose(1, 2).contiguous()

    q, k, v = split(lin("q", h1)), split(lin("k", h1)), split(lin("v", h1))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(dh)
    mask = torch.ones(T, T, dtype=torch.bool, device=x.device).triu(1)
    s = s.masked_fill(mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), v).transpose(1, 2).reshape(b, T, d)
    x2 = x + lin("o", o)
    h2 = rmsnorm(x2, g2)
    m = torch.nn.functional.silu(lin("gate", h2)) * lin("up", h2)
    return x2 + lin("down", m)


class GpuLayer:
    """The layer on the GPU kernels: NF4 + DQ base weights quantized by the
    library, fp32 adapters as autograd leaves, bf16 projection operands and
    fp32 glue."""

    def __init__(self, qb, spec: LayerSpec, params, device):
        from bit_nf4_quantized_03_amd.autograd import qlora_linear
        self._lin = qlora_linear
        self.spec = spec
        self.W, self.A, self.B = {}, {}, {}
        for name in NAMES:
            w, a, bb = params[name]
            wd = torch.from_numpy(synth.f32_to_bf16(w).view(np.int16)).to(device).view(torch.bfloat16)
            self.W[name] = qb.qlora_nf4_quantize(wd)
            self.A[name] = torch.from_numpy(a).to(device).requires_grad_(True)
            self.B[name] = torch.from_numpy(bb).to(device).requires_grad_(True)
        self.g1 = torch.from_numpy(params["g1"]).to(device)
        self.g2 = torch.from_numpy(params["g2"]).to(device)

    def lin(self, name, h):
        y = self._lin(h.to(torch.bfloat16), self.W[name], self.A[name], self.B[name], self.spec.scale)
        return y.float()

    def forward(self, x):
        return layer_forward(x, self.lin, self.g1, self.g2, self.spec.heads)

    def zero_grad(self):
        for t in list(self.A.values()) + list(self.B.values()):
            t.grad = None
