"""Oracle: NF4 codebook, block-wise NF4 quantization, double quantization, dequantization.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

What the pages fix, and the reading taken where they are silent:

* Data type. NF4 is built for normally distributed weights and is finer near
  zero (Guanaco topic page, "Technical Innovations: NormalFloat4"); the k-bit
  type has an exact zero and uses all 2^k = 16 values (QLoRA review,
  finding on paper p.5 Section 3). Reading: equal-probability-mass quantiles
  of N(0, 1), 8 on the positive side and 7 on the negative side plus an exact
  0, taken at the centres of equal-mass bins whose outermost centre is
  p_max = 1 - (1/(2*16) + 1/(2*15))/2, divided by the largest quantile so the
  ends are exactly -1 and +1. Values are computed with 50-digit arithmetic and
  rounded once to fp32.
* Blocks and scaling. Block-wise quantization with absmax scaling (QLoRA vs
  ChatGPT page, capability "NF4 4-bit quantization"). Blocks are 64
  consecutive elements of the row-major flattened weight; the last block may
  be partial. Each element is scaled as y = fp32(x / absmax) (true division)
  and coded as the nearest codebook value, ties to the lower index. A block of
  zeros stores absmax 0 and code 7 (the 0.0 level) everywhere.
* Packing. Two codes per byte, element 2j in the high nibble; an odd element
  count leaves a zero low nibble in the last byte.
* Double quantization. The absmax constants are themselves quantized to 8 bits
  with their own scales (QLoRA vs ChatGPT page, capability "double
  quantization"; about 0.4 bit per parameter saved, Guanaco topic page,
  "Core Architecture & Training"). Reading: one mean per tensor is subtracted
  (the "zero-point" the page mentions), then symmetric linear int8 codes in
  blocks of 256 constants, each block with an fp32 scale equal to its largest
  |absmax - mean|. The mean is an fp64 sum over a perfect binary tree with
  adjacent pairing (leaves in index order, zero padded to a power of two),
  divided by the count in fp64 and rounded once to fp32.
* Dequantization (block-wise, on the fly: QLoRA vs ChatGPT page, capability
  "training pipeline"). Reading of the reconstruction order, all fp32 with
  round-to-nearest-even and no fused multiply-add:
      k_d  = fp32(scale_d / 127)
      c'_b = fp32(fp32(q_b * k_d) + mean)
      w    = fp32(codebook[code] * c'_b)
  and a bf16 output is the round-to-nearest-even of that fp32 value.
* Comparison formats. The paper's Table 4 (QLoRA review, findings on paper
  p.8 Table 4: rows NFloat4, NFloat4 + DQ and Float4, and the caption that has
  FP4 about one point behind) compares NF4 with and without double
  quantization and a 4-bit float. Without DQ the fp32 absmax constants are
  stored as they are and w = fp32(codebook[code] * absmax_b). The pages do not
  define the 4-bit float. Reading: the float with one sign bit, two exponent
  bits (bias 1, subnormals at exponent 0, no infinities) and one mantissa bit,
  whose 15 distinct values are +-{0, 1/2, 1, 3/2, 2, 3, 4, 6}; they are divided
  by 6 so that a block's absmax maps to the largest magnitude, as NF4's levels
  span [-1, 1]. The table lists the values in ascending order with the zero at
  index 7, as NF4 does, and repeats +1 at index 15, so the nearest-level rule
  (ties to the lower index) never yields code 15. Quantization, packing and
  dequantization are otherwise those of NF4.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction

import mpmath
import numpy as np

NF4_BLOCK = 64
DQ_BLOCK = 256
N_LEVELS = 16
ZERO_CODE = 7

# ---------------------------------------------------------------------------
# Codebook
# ---------------------------------------------------------------------------


def nf4_p_max():
    """Outermost equal-mass bin centre: average of the 16-level and the 15-level
    view of the asymmetric type, 1 - (1/32 + 1/30)/2 (an mpmath number)."""
    return 1 - (mpmath.mpf(1) / (2 * 16) + mpmath.mpf(1) / (2 * 15)) / 2


def _normal_quantile(p):
    """Inverse standard-normal CDF via the inverse error function (mpmath)."""
    return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)


def nf4_levels_mp(dps: int = 50):
    """The 16 NF4 levels as mpmath numbers, sorted ascending.

    Positive side: quantiles at 8 equally spaced probabilities from p_max down
    to (not including) 1/2. Negative side: the mirror of 7 equally spaced
    probabilities from p_max to 1/2. Plus an exact zero. All divided by the
    quantile at p_max.
    """
    with mpmath.workdps(dps):
        p_max = nf4_p_max()
        half = mpmath.mpf(1) / 2
        pos_p = [p_max + (half - p_max) * i / 8 for i in range(8)]
        neg_p = [p_max + (half - p_max) * i / 7 for i in range(7)]
        z_max = _normal_quantile(p_max)
        pos = [_normal_quantile(p) / z_max for p in pos_p]
        neg = [-_normal_quantile(p) / z_max for p in neg_p]
        levels = sorted(neg + [mpmath.mpf(0)] + pos)
        return levels


def round_to_f32(v) -> np.float32:
    """Round a real (mpmath or Python number) to the nearest fp32, ties to even.

    Avoids double rounding through fp64 by comparing the fp32 neighbours of a
    first guess in exact mpmath arithmetic.
    """
    with mpmath.workdps(60):
        v = mpmath.mpf(v)
        g = np.float32(float(v))
        cands = {float(g), float(np.nextafter(g, np.float32(np.inf))),
                 float(np.nextafter(g, np.float32(-np.inf)))}
        best = None
        for c in sorted(cands):
            d = abs(mpmath.mpf(c) - v)
            if best is None or d < best[0]:
                best = (d, c)
            elif d == best[0]:
                # tie: keep the candidate with an even fp32 mantissa
                if np.float32(c).view(np.uint32) % 2 == 0:
                    best = (d, c)
        return np.float32(best[1])


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels as fp32, ascending; index = 4-bit code."""
    return np.array([round_to_f32(v) for v in nf4_levels_mp()], dtype=np.float32)


def e2m1_values():
    """Every value of the 4-bit float (1 sign, 2 exponent bits with bias 1,
    1 mantissa bit; exponent field 0 is subnormal), as exact fractions,
    ascending and without the duplicate zero: 15 values."""
    vals = set()
    for sign in (1, -1):
        for e in range(4):
            for m in range(2):
                if e == 0:
                    mag = Fraction(m, 2)                       # 2^(1 - bias) * (m / 2)
                else:
                    mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
                vals.add(sign * mag)
    return sorted(vals)


def fp4_codebook() -> np.ndarray:
    """The 16 FP4 levels as fp32: the 15 values of ``e2m1_values`` divided by
    the largest one (each rounded once to fp32), ascending, with +1 repeated
    at index 15 (a code the nearest-level rule never chooses)."""
    vals = e2m1_values()
    top = vals[-1]
    levels = [v / top for v in vals] + [Fraction(1)]
    with mpmath.workdps(50):
        return np.array([round_to_f32(mpmath.mpf(v.numerator) / v.denominator) for v in levels],
                        dtype=np.float32)


# ---------------------------------------------------------------------------
# First level: block absmax and nearest code
# ---------------------------------------------------------------------------


def nearest_code(y: np.ndarray, codebook: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """Index of the codebook value nearest to each fp32 y, ties to the lower index.

    Distances are |y - c_j| in fp64; for fp32 operands of magnitude <= 1 whose
    distance matters (away from the tiny values that are far from every
    midpoint) these differences are exact in fp64, so this is the exact argmin.
    ``np.argmin`` returns the first minimum, which is the lower-index tie rule.
    """
    y = np.asarray(y, dtype=np.float32).reshape(-1)
    cb = codebook.astype(np.float64)
    out = np.empty(y.size, dtype=np.uint8)
    for s in range(0, y.size, chunk):
        yy = y[s:s + chunk].astype(np.float64)
        d = np.abs(yy[:, None] - cb[None, :])
        out[s:s + chunk] = np.argmin(d, axis=1).astype(np.uint8)
    return out


def block_absmax(x: np.ndarray, block: int = NF4_BLOCK) -> np.ndarray:
    """fp32 max |x| over consecutive blocks of the flattened input (last block may be partial)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    nb = -(-n // block)
    pad = np.zeros(nb * block, dtype=np.float32)
    pad[:n] = np.abs(x)
    return pad.reshape(nb, block).max(axis=1)


def nf4_codes(x: np.ndarray, codebook: np.ndarray):
    """Per-element NF4 codes and per-block absmax of the flattened fp32 input.

    y = fp32(x / absmax) (IEEE division); zero blocks give y = 0 and hence the
    0.0 level, code 7.
    """
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    a = block_absmax(x)
    a_el = np.repeat(a, NF4_BLOCK)[:n]
    y = np.zeros(n, dtype=np.float32)
    nz = a_el > 0
    y[nz] = x[nz] / a_el[nz]
    return nearest_code(y, codebook), a


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2j in the high nibble, 2j+1 in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    c = np.empty(p.size * 2, dtype=np.uint8)
    c[0::2] = p >> 4
    c[1::2] = p & 0x0F
    return c[:n]


# ---------------------------------------------------------------------------
# Second level: double quantization of the absmax constants
# ---------------------------------------------------------------------------


def tree_sum_f64(v: np.ndarray) -> float:
    """fp64 sum over a perfect binary tree: leaves in index order, zero padded
    to the next power of two, adjacent pairs added level by level."""
    v = np.asarray(v, dtype=np.float64).reshape(-1)
    if v.size == 0:
        return 0.0
    p = 1
    while p < v.size:
        p *= 2
    t = np.zeros(p, dtype=np.float64)
    t[:v.size] = v
    while t.size > 1:
        t = t[0::2] + t[1::2]
    return float(t[0])


def dq_mean(absmax: np.ndarray) -> np.float32:
    """Per-tensor mean of the absmax constants: fp32(tree_sum_fp64 / count)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    return np.float32(np.float64(tree_sum_f64(a)) / np.float64(a.size))


def double_quantize(absmax: np.ndarray):
    """Quantize fp32 absmax constants to int8 with per-256 fp32 scales and one mean.

    d = fp32(a - mean); scale = max |d| over the block; t = fp32(d / scale);
    u = fp32(t * 127); q = round-half-even(u) clamped to [-127, 127]. A block
    whose scale is 0 stores q = 0.
    Returns (q int8 [nb], scale f32 [nd], mean f32).
    """
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    mu = dq_mean(a)
    d = (a - mu).astype(np.float32)
    nd = -(-nb // DQ_BLOCK)
    dpad = np.zeros(nd * DQ_BLOCK, dtype=np.float32)
    dpad[:nb] = d
    scale = np.abs(dpad).reshape(nd, DQ_BLOCK).max(axis=1).astype(np.float32)
    s_el = np.repeat(scale, DQ_BLOCK)[:nb]
    t = np.zeros(nb, dtype=np.float32)
    nz = s_el > 0
    t[nz] = d[nz] / s_el[nz]
    u = (t * np.float32(127.0)).astype(np.float32)
    q = np.clip(np.rint(u), -127, 127).astype(np.int8)
    return q, scale, mu


def dq_reconstruct(q: np.ndarray, scale: np.ndarray, mu) -> np.ndarray:
    """Per-block scale c' = fp32(fp32(q * fp32(scale / 127)) + mean)."""
    q = np.asarray(q, dtype=np.int8).reshape(-1)
    k = (np.asarray(scale, dtype=np.float32) / np.float32(127.0)).astype(np.float32)
    k_el = np.repeat(k, DQ_BLOCK)[:q.size]
    return ((q.astype(np.float32) * k_el).astype(np.float32) + np.float32(mu)).astype(np.float32)


# ---------------------------------------------------------------------------
# The stored format
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class NF4Tensor:
    """4-bit weight of ``shape`` (row-major). With ``dq`` the absmax constants
    are stored double-quantized (absmax_q, dq_scale, dq_mean) and ``absmax``
    holds the first-level constants for tests only; without it absmax_q,
    dq_scale and dq_mean are None and ``absmax`` is the stored fp32 constant."""
    shape: tuple
    codes: np.ndarray      # uint8 [ceil(n/2)]
    absmax_q: np.ndarray   # int8  [nb], or None without DQ
    dq_scale: np.ndarray   # f32   [nd], or None without DQ
    dq_mean: np.float32    # f32 scalar, or None without DQ
    absmax: np.ndarray     # f32 [nb], first-level constants
    dq: bool = True

    @property
    def n(self) -> int:
        return int(np.prod(self.shape))


def quantize(w: np.ndarray, codebook: np.ndarray = None, double_quant: bool = True) -> NF4Tensor:
    """Quantize an fp32-valued weight (bf16 inputs widened exactly) to 4-bit
    codes of ``codebook`` (NF4 by default), with or without DQ.

    The two levels are sequential: codes are chosen with the true fp32 absmax,
    then (with DQ) the absmax constants are double-quantized; so the codes do
    not depend on ``double_quant``.
    """
    if codebook is None:
        codebook = nf4_codebook()
    w = np.asarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("oracle quantize: inputs must be finite")
    codes, a = nf4_codes(w, codebook)
    if not double_quant:
        return NF4Tensor(tuple(w.shape), pack_codes(codes), None, None, None, a, dq=False)
    q, scale, mu = double_quantize(a)
    return NF4Tensor(tuple(w.shape), pack_codes(codes), q, scale, mu, a)


def dequantize(t: NF4Tensor, codebook: np.ndarray = None) -> np.ndarray:
    """fp32 reconstruction w = fp32(codebook[code] * c'_block), in ``t.shape``;
    c' is the double-quantized constant, or the stored fp32 absmax without DQ."""
    if codebook is None:
        codebook = nf4_codebook()
    n = t.n
    codes = unpack_codes(t.codes, n)
    cprime = dq_reconstruct(t.absmax_q, t.dq_scale, t.dq_mean) if t.dq else np.asarray(t.absmax, np.float32)
    c_el = np.repeat(cprime, NF4_BLOCK)[:n]
    w = (codebook[codes] * c_el).astype(np.float32)
    return w.reshape(t.shape)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of finite fp32 values, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def storage_bytes(n: int, double_quant: bool = True) -> int:
    """Bytes of the stored format: codes n/2 (rounded up) + int8 per block +
    fp32 scale per DQ block + one fp32 mean; without DQ, codes + fp32 per block."""
    nb = -(-n // NF4_BLOCK)
    if not double_quant:
        return -(-n // 2) + 4 * nb
    nd = -(-nb // DQ_BLOCK)
    return -(-n // 2) + nb + 4 * nd + 4


def bits_per_param(n: int, double_quant: bool = True) -> float:
    return 8.0 * storage_bytes(n, double_quant) / n


__all__ = [
    "NF4_BLOCK", "DQ_BLOCK", "ZERO_CODE", "nf4_codebook", "nf4_levels_mp", "round_to_f32",
    "e2m1_values", "fp4_codebook",
    "nearest_code", "block_absmax", "nf4_codes", "pack_codes", "unpack_codes",
    "tree_sum_f64", "dq_mean", "double_quantize", "dq_reconstruct", "NF4Tensor",
    "quantize", "dequantize", "f32_to_bf16_rne", "storage_bytes", "bits_per_param",
]

