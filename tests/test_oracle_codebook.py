"""Pins of the oracle's NF4 codebook against what the pages and mathematics fix.

* 16 values, an exact zero (ai-papercheck QLoRA review, finding on paper p.5
  Section 3: all 2^k values of a k-bit type with a discrete zero point).
* Range [-1, 1] under absmax scaling (QLoRA vs ChatGPT page, capability "NF4
  4-bit quantization").
* Built for normally distributed weights, finer near zero (Guanaco topic page,
  "Technical Innovations: NormalFloat4"): the levels are normal quantiles at
  equally spaced probabilities. Checked with the forward CDF (scipy ``ndtr``),
  a function the oracle does not use, and with a second inverse (scipy
  ``ndtri``) instead of mpmath's ``erfinv``.
"""
import json
import os

import numpy as np
import pytest
import scipy.special as sps

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "storage_claims.json")


@pytest.fixture(scope="module")
def cb():
    return nf4.nf4_codebook()


def test_sixteen_strictly_increasing(cb):
    claims = json.load(open(GOLDEN))
    assert cb.dtype == np.float32
    assert cb.size == claims["levels"]["value"] == 16
    assert np.all(np.diff(cb.astype(np.float64)) > 0)


def test_exact_zero_and_unit_ends(cb):
    bits = cb.view(np.uint32)
    assert bits[nf4.ZERO_CODE] == 0x00000000          # +0.0 exactly
    assert bits[0] == np.float32(-1.0).view(np.uint32)
    assert bits[15] == np.float32(1.0).view(np.uint32)
    # the zero level splits the type 7 negative / 8 positive
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8


def test_denser_near_zero(cb):
    c = cb.astype(np.float64)
    pos_gaps = np.diff(c[7:])            # 0 -> c8 -> ... -> 1
    neg_gaps = np.diff(c[:8])[::-1]      # 0 -> c6 -> ... -> -1, as magnitudes
    assert np.all(np.diff(pos_gaps) > 0), pos_gaps
    assert np.all(np.diff(neg_gaps) > 0), neg_gaps


def test_levels_are_normal_quantiles_forward_cdf(cb):
    """Phi(c_i * z_max) must land on the equally spaced probability grid."""
    p_max = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    z_max = sps.ndtri(p_max)
    c = cb.astype(np.float64)
    pos_grid = p_max + (0.5 - p_max) * np.arange(8) / 8.0      # c15 ... c8
    neg_grid = p_max + (0.5 - p_max) * np.arange(7) / 7.0      # -c0 ... -c6
    got_pos = sps.ndtr(c[15:7:-1] * z_max)
    got_neg = sps.ndtr(-c[0:7] * z_max)
    # fp32 rounding of a level moves Phi by at most pdf * ulp * z_max < 1e-7
    assert np.max(np.abs(got_pos - pos_grid)) < 2e-7
    assert np.max(np.abs(got_neg - neg_grid)) < 2e-7


def test_second_inverse_gives_same_fp32_table(cb):
    """An independent fp64 derivation with scipy's ndtri rounds to the same bits."""
    p_max = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    z_max = sps.ndtri(p_max)
    pos = sps.ndtri(p_max + (0.5 - p_max) * np.arange(8) / 8.0) / z_max
    neg = -sps.ndtri(p_max + (0.5 - p_max) * np.arange(7) / 7.0) / z_max
    alt = np.sort(np.concatenate([neg, [0.0], pos])).astype(np.float32)
    assert np.array_equal(alt.view(np.uint32), cb.view(np.uint32))


def test_all_sixteen_codes_used_on_normal_data(cb):
    rng = np.random.default_rng(0)
    x = rng.standard_normal(64 * 512).astype(np.float32)
    codes, _ = nf4.nf4_codes(x, cb)
    assert set(np.unique(codes).tolist()) == set(range(16))


def test_round_to_f32_is_correct_rounding():
    # exact midpoint between 1 and the next float rounds to even (1.0)
    one_up = float(np.nextafter(np.float32(1), np.float32(2)))
    mid = (1.0 + one_up) / 2.0
    assert nf4.round_to_f32(mid) == np.float32(1.0)
    # a value just above the midpoint rounds up
    assert nf4.round_to_f32(np.nextafter(mid, 2.0)) == np.float32(one_up)
