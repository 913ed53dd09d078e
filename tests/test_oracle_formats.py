"""Pins of the oracle's comparison formats: NF4 without double quantization and
the 4-bit float (FP4) codebook.

The paper's Table 4 compares NFloat4, NFloat4 + DQ and Float4 (QLoRA review,
findings on paper p.8 Table 4; the caption has FP4 about one point behind).
The checks rest on exact rational arithmetic, on the published value grid of
the 4-bit float with one mantissa bit (+-{0, 1/2, 1, 3/2, 2, 3, 4, 6}), on
identities of any block-wise absmax quantizer, on the claim that NF4 suits
normally distributed weights best (Guanaco topic page, "Technical Innovations:
NormalFloat4") and on the storage figures the pages print.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "storage_claims.json")

# The 4-bit float with 2 exponent bits and 1 mantissa bit, as published for
# the OCP microscaling formats: its non-negative values.
E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


@pytest.fixture(scope="module")
def fp4():
    return nf4.fp4_codebook()


@pytest.fixture(scope="module")
def nf():
    return nf4.nf4_codebook()


def exact_nearest(y, cb):
    """argmin_j |y - c_j| in exact rational arithmetic, ties to the lower index."""
    fy = Fraction(float(y))
    best, bi = None, None
    for j, c in enumerate(cb):
        d = abs(fy - Fraction(float(c)))
        if best is None or d < best:
            best, bi = d, j
    return bi


def is_nearest_f32(f, v):
    """fp32 f is a correctly rounded value of the exact rational v."""
    f = np.float32(f)
    d = abs(Fraction(float(f)) - v)
    for nb in (np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
        if abs(Fraction(float(nb)) - v) < d:
            return False
    return True


def test_e2m1_values_are_the_published_grid():
    vals = nf4.e2m1_values()
    assert len(vals) == 15
    assert sorted(v for v in vals if v >= 0) == E2M1_GRID
    assert sorted(-v for v in vals if v <= 0) == E2M1_GRID


def test_fp4_codebook_layout(fp4):
    assert fp4.dtype == np.float32 and fp4.shape == (16,)
    assert np.all(np.diff(fp4[:15]) > 0), "15 distinct ascending values"
    assert fp4[15] == fp4[14] == 1.0 and fp4[0] == -1.0
    assert fp4[nf4.ZERO_CODE] == 0.0
    assert np.array_equal(fp4[:15], -fp4[:15][::-1])
    for i, g in enumerate(sorted(E2M1_GRID[1:] + [-v for v in E2M1_GRID])):
        assert is_nearest_f32(fp4[i], g / 6)


def test_fp4_nearest_code_exact_near_midpoints_and_random(fp4):
    ys = []
    for i in range(15):
        m = (Fraction(float(fp4[i])) + Fraction(float(fp4[i + 1]))) / 2
        v = np.float32(float(m))
        for _ in range(5):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(11):
            ys.append(v)
            v = np.nextafter(v, np.float32(2))
    rng = np.random.default_rng(31)
    ys = np.concatenate([np.array(ys, np.float32), rng.uniform(-1, 1, 2000).astype(np.float32), fp4,
                         np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45], np.float32)])
    got = nf4.nearest_code(ys, fp4)
    want = np.array([exact_nearest(y, fp4) for y in ys])
    assert np.array_equal(got, want)


def _e2m1_round(t):
    """Round-to-nearest onto the 4-bit float grid, done the floating-point way:
    spacing 1/2 below 2 (subnormals and the first binade), then 2^(e-1) in
    binade [2^e, 2^(e+1)); saturate at 6. t is a float away from midpoints."""
    m = abs(t)
    if m >= 6:
        q = 6.0
    else:
        step = 0.5 if m < 2 else 2.0 ** (np.floor(np.log2(m)) - 1)
        q = min(round(m / step) * step, 6.0)
    return q if t >= 0 else -q


def test_fp4_codes_match_float_rounding(fp4):
    rng = np.random.default_rng(32)
    x = rng.standard_normal(64 * 300).astype(np.float32)
    codes, a = nf4.nf4_codes(x, fp4)
    y = x / np.repeat(a, 64)
    mids = np.array([(float(fp4[i]) + float(fp4[i + 1])) / 2 for i in range(14)])
    checked = 0
    for yi, ci in zip(y, codes):
        if np.min(np.abs(mids - yi)) < 1e-5:
            continue
        assert float(fp4[ci]) * 6 == pytest.approx(_e2m1_round(6 * float(yi)), abs=1e-6)
        checked += 1
    assert checked > 0.99 * y.size


def test_fp4_uses_fifteen_codes_never_fifteen(fp4):
    rng = np.random.default_rng(33)
    x = rng.standard_normal(64 * 2000).astype(np.float32)
    codes, _ = nf4.nf4_codes(x, fp4)
    assert codes.max() == 14
    assert set(np.unique(codes).tolist()) == set(range(15))


@pytest.mark.parametrize("which", ["nf4", "fp4"])
def test_codes_do_not_depend_on_double_quantization(which, nf, fp4):
    cb = nf if which == "nf4" else fp4
    rng = np.random.default_rng(34)
    x = (rng.standard_normal((40, 257)) * 0.03).astype(np.float32)
    t1 = nf4.quantize(x, cb)
    t0 = nf4.quantize(x, cb, double_quant=False)
    assert np.array_equal(t0.codes, t1.codes)
    assert np.array_equal(t0.absmax, t1.absmax)
    assert t0.absmax_q is None and t0.dq_scale is None and t0.dq_mean is None and not t0.dq


@pytest.mark.parametrize("which", ["nf4", "fp4"])
def test_no_dq_reconstruction(which, nf, fp4):
    """Without DQ the block maximum comes back exactly (it takes an end level,
    +-1) and every element lies within half the widest level gap times absmax."""
    cb = nf if which == "nf4" else fp4
    rng = np.random.default_rng(35)
    x = (rng.standard_normal(64 * 500 + 37) * 0.05).astype(np.float32)
    x[64 * 3:64 * 4] = 0.0
    t = nf4.quantize(x, cb, double_quant=False)
    w = nf4.dequantize(t, cb)
    a = t.absmax
    blocks = -(-x.size // 64)
    xp = np.zeros(blocks * 64, np.float32)
    xp[:x.size] = x
    wp = np.zeros(blocks * 64, np.float32)
    wp[:x.size] = w
    xp, wp = xp.reshape(blocks, 64), wp.reshape(blocks, 64)
    i = np.argmax(np.abs(xp), axis=1)
    assert np.array_equal(np.abs(wp[np.arange(blocks), i]), a)
    assert np.all(wp[3] == 0.0)
    half_gap = np.max(np.diff(cb.astype(np.float64))) / 2
    err = np.abs(wp.astype(np.float64) - xp) / np.maximum(a[:, None].astype(np.float64), 1e-30)
    assert err.max() <= half_gap * (1 + 1e-6)


def test_no_dq_error_is_not_above_dq_error(nf):
    rng = np.random.default_rng(36)
    x = (rng.standard_normal(64 * 4096) * 0.02).astype(np.float32)
    e1 = np.mean((nf4.dequantize(nf4.quantize(x, nf), nf) - x).astype(np.float64) ** 2)
    e0 = np.mean((nf4.dequantize(nf4.quantize(x, nf, double_quant=False), nf) - x).astype(np.float64) ** 2)
    assert e0 <= e1
    assert e1 <= 1.05 * e0   # DQ costs little (the paper's NFloat4 and NFloat4 + DQ rows agree)


def test_nf4_beats_fp4_on_normal_weights(nf, fp4):
    rng = np.random.default_rng(37)
    x = rng.standard_normal(64 * 8192).astype(np.float32)
    e_nf = np.mean((nf4.dequantize(nf4.quantize(x, nf, double_quant=False), nf) - x).astype(np.float64) ** 2)
    e_fp = np.mean((nf4.dequantize(nf4.quantize(x, fp4, double_quant=False), fp4) - x).astype(np.float64) ** 2)
    assert e_nf < e_fp


def test_storage_without_dq_against_page_figures():
    with open(GOLDEN) as f:
        g = json.load(f)
    n = 4096 * 4096
    assert nf4.bits_per_param(n, double_quant=False) == 4.5    # 32-bit constant per 64 weights
    saving = nf4.bits_per_param(n, double_quant=False) - nf4.bits_per_param(n)
    assert abs(saving - g["dq_saving_bits_per_param"]["value"]) < 0.05
    assert nf4.storage_bytes(65, double_quant=False) == 33 + 8


def test_planted_format_mistakes_are_caught(monkeypatch, nf):
    """A wrong exponent bias, or a dequantizer that ignores the fp32 constants
    without DQ, fails the pins above."""
    real = nf4.e2m1_values

    def bias0():
        return [2 * v for v in real()]
    monkeypatch.setattr(nf4, "e2m1_values", bias0)
    with pytest.raises(AssertionError):
        test_e2m1_values_are_the_published_grid()
    monkeypatch.setattr(nf4, "e2m1_values", real)

    real_deq = nf4.dequantize

    def deq_wrong(t, codebook=None):
        t2 = nf4.NF4Tensor(t.shape, t.codes, *nf4.double_quantize(t.absmax), t.absmax)
        return real_deq(t2, codebook)
    monkeypatch.setattr(nf4, "dequantize", deq_wrong)
    with pytest.raises(AssertionError):
        test_no_dq_reconstruction("nf4", nf, None)
