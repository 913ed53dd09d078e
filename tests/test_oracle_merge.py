"""Pins of the oracle's adapter merge (W' = W-hat + s B A, then requantize).

The checks rest on exact rational arithmetic for the merged fp32 weight, on
the identity that a merged weight reproduces the LoRA forward pass (the
oracle's linear layer computes (X A^T) B^T on its own), and on the zero
adapter leaving the base unchanged.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import synth
from oracle import linear, merge, nf4


@pytest.fixture(scope="module")
def cb():
    return nf4.nf4_codebook()


def _case(N, K, r, seed, cb, fmt_dq=True, codebook=None):
    rng = np.random.default_rng(seed)
    w = synth.normal_f32(rng, (N, K), 0.02)
    t = nf4.quantize(w, codebook if codebook is not None else cb, double_quant=fmt_dq)
    A = (rng.standard_normal((r, K)) * 0.01).astype(np.float32) if r else None
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32) if r else None
    return t, A, B


def test_merged_weight_is_the_rounded_exact_value(cb):
    N, K, r, s = 3, 70, 5, np.float32(0.37)
    t, A, B = _case(N, K, r, 11, cb)
    got = merge.merged_weight(t, cb, A, B, s)
    w = nf4.dequantize(t, cb)
    for n in range(N):
        for k in range(K):
            exact = Fraction(float(w[n, k])) + Fraction(float(s)) * sum(
                Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r))
            with mpmath.workdps(80):
                want = nf4.round_to_f32(mpmath.mpf(exact.numerator) / exact.denominator)
            assert got[n, k] == want, (n, k)


@pytest.mark.parametrize("fmt_dq", [True, False])
def test_zero_adapter_keeps_the_base(cb, fmt_dq):
    t, A, B = _case(40, 192, 8, 12, cb, fmt_dq)
    w = nf4.dequantize(t, cb)
    for (a, b, s) in ((None, None, 0.5), (A, B, 0.0)):
        got = merge.merged_weight(t, cb, a, b, s)
        assert np.array_equal(got.view(np.uint32), w.view(np.uint32))
    t2 = merge.merge_requantize(t, cb, None, None, 1.0, cb, fmt_dq)
    assert np.array_equal(t2.codes, t.codes)


def test_merged_weight_reproduces_the_lora_forward(cb):
    """X W'^T equals X W-hat^T + s (X A^T) B^T up to the fp32 rounding of W'."""
    N, K, r, s = 96, 128, 16, 0.5
    t, A, B = _case(N, K, r, 13, cb)
    rng = np.random.default_rng(14)
    X = rng.standard_normal((33, K)).astype(np.float32)
    Wm = merge.merged_weight(t, cb, A, B, s)
    y_merged = X.astype(np.float64) @ Wm.astype(np.float64).T
    y_lora = linear.forward(X, nf4.dequantize(t, cb), A, B, s)
    assert np.abs(y_merged - y_lora).max() <= 1e-6 * np.abs(y_lora).max()
    # the adapter term is not negligible at this scale
    y_base = linear.forward(X, nf4.dequantize(t, cb), None, None, 0.0)
    assert np.abs(y_lora - y_base).max() > 1e-3 * np.abs(y_lora).max()


def test_requantized_merge_is_the_quantized_merged_weight(cb):
    fp4 = nf4.fp4_codebook()
    t, A, B = _case(8, 320, 4, 15, cb)
    for ocb, odq in ((cb, True), (fp4, False)):
        q = merge.merge_requantize(t, cb, A, B, 0.25, ocb, odq)
        ref = nf4.quantize(merge.merged_weight(t, cb, A, B, 0.25), ocb, double_quant=odq)
        assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.absmax, ref.absmax)


def test_planted_merge_mistakes_are_caught(monkeypatch, cb):
    """A sign error or a transposed product fails the pins above."""
    real = merge.merged_weight

    def wrong_sign(t, codebook, A, B, s):
        return real(t, codebook, A, B, -s)
    monkeypatch.setattr(merge, "merged_weight", wrong_sign)
    with pytest.raises(AssertionError):
        test_merged_weight_reproduces_the_lora_forward(cb)
    with pytest.raises(AssertionError):
        test_merged_weight_is_the_rounded_exact_value(cb)
    monkeypatch.setattr(merge, "merged_weight", real)

    def order_swapped(t, codebook, A, B, s):
        # the adapter product taken the other way round (A^T B^T), square case
        return real(t, codebook, B.T.copy() if B is not None else None,
                    A.T.copy() if A is not None else None, s)
    monkeypatch.setattr(merge, "merged_weight", order_swapped)
    with pytest.raises(Exception):
        test_merged_weight_reproduces_the_lora_forward(cb)
