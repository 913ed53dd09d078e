"""Oracle: one AdamW step for the LoRA parameters, with optimizer state that
may be paged to host memory.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix, and the reading taken where they are silent:

* Only the adapter parameters are trained, in full precision, with their
  gradients from the backward pass; the optimizer state (momentum and
  variance) is paged between GPU and CPU memory so that memory spikes do not
  end the run (Guanaco topic page, "Technical Innovations: Paged
  Optimizers"; QLoRA vs ChatGPT page, capability on paged optimizers).
* The pages do not give the optimizer's formula. Reading: AdamW (Adam with
  decoupled weight decay, Loshchilov and Hutter), fp32 state, every step an
  fp32 operation rounded to nearest even with no fused multiply-add:
      c1 = fp32(1 - beta1), c2 = fp32(1 - beta2)
      m' = fp32(fp32(beta1 m) + fp32(c1 g))
      v' = fp32(fp32(beta2 v) + fp32(c2 fp32(g g)))
      mh = fp32(m' / bc1), vh = fp32(v' / bc2)
      u  = fp32(mh / fp32(sqrt(vh) + eps))       (sqrt correctly rounded)
      p' = fp32(p - fp32(lr fp32(u + fp32(wd p))))
  with the bias corrections bc1 = 1 - beta1^t and bc2 = 1 - beta2^t given by
  the caller as fp32 numbers (t >= 1 the step count).
* Paging moves the state, not the arithmetic: the result is the same whether
  the state lives in device or host memory.
"""
from __future__ import annotations

import numpy as np


def bias_corrections(beta1: float, beta2: float, t: int):
    """fp32(1 - beta^t) for both moments, with beta the fp32 value the step
    uses (fp64 arithmetic, then one rounding)."""
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    return np.float32(1.0 - b1 ** t), np.float32(1.0 - b2 ** t)


def adamw_step(p, g, m, v, lr, beta1, beta2, eps, wd, bc1, bc2):
    """Returns (p', m', v') as fp32 arrays, by the op order in the module docstring."""
    f = np.float32
    p, g, m, v = (np.asarray(a, dtype=np.float32) for a in (p, g, m, v))
    b1, b2 = f(beta1), f(beta2)
    c1, c2 = f(f(1.0) - b1), f(f(1.0) - b2)
    m2 = (b1 * m).astype(np.float32) + (c1 * g).astype(np.float32)
    m2 = m2.astype(np.float32)
    gg = (g * g).astype(np.float32)
    v2 = ((b2 * v).astype(np.float32) + (c2 * gg).astype(np.float32)).astype(np.float32)
    mh = (m2 / f(bc1)).astype(np.float32)
    vh = (v2 / f(bc2)).astype(np.float32)
    den = (np.sqrt(vh).astype(np.float32) + f(eps)).astype(np.float32)
    u = (mh / den).astype(np.float32)
    step = (f(lr) * (u + (f(wd) * p).astype(np.float32)).astype(np.float32)).astype(np.float32)
    p2 = (p - step).astype(np.float32)
    return p2, m2, v2


__all__ = ["bias_corrections", "adamw_step"]
