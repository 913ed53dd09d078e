"""Plain CPU oracle for QLoRA's NF4 + double-quantization format and its linear layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package. The product path
(the HIP library and its Python binding) never imports it, and this package
never imports the product: the two share no code, tables or constants.

The oracle is slow and obviously correct by design: vectorized NumPy on whole
arrays, fp64 for every matmul, and explicit fp32 operations (NumPy float32
``+ - * /`` are IEEE round-to-nearest-even with no fused multiply-add) where the
storage format fixes a float32 result bit for bit.

Modules
  nf4     codebook derivation (NF4, and the FP4 comparison levels), block-wise
          quantization, double quantization of the absmax constants (or fp32
          constants without it), dequantization, storage size.
  linear  QLoRA linear forward and backward in fp64.
  merge   merging an adapter into the dequantized base (fp64 rank sum,
          one rounding to fp32) and requantizing it.
  adamw   one AdamW step of the adapter parameters in fp32, op by op.

Sources (the pages the method is taken from):
  * Guanaco topic page (chipfoundryservices.com), "Technical Innovations":
    NF4 is optimal for normally distributed data and finer near zero; and
    "Core Architecture & Training": double quantization saves about 0.4 bit per
    parameter.
  * ai-papercheck review "QLoRA: Efficient Finetuning of Quantized LLMs",
    finding on paper p.5 Section 3: the k-bit type has an exact zero point and
    uses all 2^k values; findings on paper p.8 Table 4: the NFloat4,
    NFloat4 + DQ and Float4 rows (the comparison formats: no DQ, FP4 levels).
  * unfragile.ai "QLoRA vs ChatGPT", capability rows on 4-bit NF4 quantization
    (block-wise absmax scaling, LoRA in full precision), double quantization
    (8-bit constants with their own scales), LoRA on the frozen base (rank 8-64)
    and the training pipeline (block-wise on-the-fly dequantization, gradients
    for the LoRA parameters only), and adapter composition (adapters merged
    into the base weights for a standalone model).

Every function whose result is pinned only by its own self-consistency says
"parity unpinned" in its docstring; at present none does.
"""
from . import nf4, linear, merge, adamw  # noqa: F401
