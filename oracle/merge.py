"""Oracle: merging a LoRA adapter into the quantized base, then requantizing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix, and the reading taken where they are silent:

* Adapters trained on the quantized base can be merged into its weights to
  give a standalone model; weighted ensembles of adapters are merged the same
  way, and full-precision adapters meet a quantized base, so the merge must
  handle the precision (QLoRA vs ChatGPT page, capability on adapter
  composition and merging).
* Reading of the merge: W' = W-hat + s * B A, with W-hat the dequantized base
  (fp32, as the dequantizer gives it), A [r, K] and B [N, r] in fp32. The sum
  over the rank runs in fp64 with j ascending; every product B[n, j] A[j, k]
  of two fp32 values is exact in fp64. Then t = fp64(s * sum), u =
  fp64(w-hat + t), and w' = fp32(u) (round to nearest even). A weighted
  ensemble of adapters is one merge with the adapters concatenated along the
  rank, each weight folded into its B.
* The merged fp32 weight is quantized again with the quantizer of ``nf4``, in
  any of the formats (so r = 0 converts a weight from one format to another).
"""
from __future__ import annotations

import numpy as np

from . import nf4


def merged_weight(t: nf4.NF4Tensor, codebook, A, B, s) -> np.ndarray:
    """fp32 W' = fp32(w-hat + fp64(s * sum_j B[:, j] A[j, :])) with the sum in
    fp64, j ascending (rank r = 0: W' = w-hat)."""
    w = nf4.dequantize(t, codebook).astype(np.float64)
    N, K = w.shape
    acc = np.zeros((N, K), dtype=np.float64)
    if A is not None and B is not None:
        A64 = np.asarray(A, dtype=np.float32).astype(np.float64)
        B64 = np.asarray(B, dtype=np.float32).astype(np.float64)
        for j in range(A64.shape[0]):
            acc += B64[:, j, None] * A64[None, j, :]
    u = w + np.float64(np.float32(s)) * acc
    return u.astype(np.float32)


def merge_requantize(t: nf4.NF4Tensor, codebook, A, B, s, out_codebook=None,
                     out_double_quant: bool = True) -> nf4.NF4Tensor:
    """Merge the adapter into the base and quantize the result again (in the
    output codebook and DQ setting, by default NF4 + DQ)."""
    w = merged_weight(t, codebook, A, B, s)
    if out_codebook is None:
        out_codebook = nf4.nf4_codebook()
    return nf4.quantize(w, out_codebook, double_quant=out_double_quant)


__all__ = ["merged_weight", "merge_requantize"]
