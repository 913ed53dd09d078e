"""Pins of the oracle's quantizer, double quantizer and dequantizer.

Each check rests on something other than the oracle's own formula:
exact rational arithmetic (``fractions.Fraction``) for the nearest-code and
int8 decisions, ``math.fsum`` for the mean, identities that hold for any
correct block-wise absmax quantizer, and the storage figures the pages print
(tests/golden/storage_claims.json).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "storage_claims.json")


@pytest.fixture(scope="module")
def cb():
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


def near_midpoint_values(cb, ulps=4):
    out = []
    for i in range(15):
        m = (Fraction(float(cb[i])) + Fraction(float(cb[i + 1]))) / 2
        f = np.float32(float(m))
        lo = f
        for _ in range(ulps):
            lo = np.nextafter(lo, np.float32(-2))
        v = lo
        for _ in range(2 * ulps + 1):
            out.append(v)
            v = np.nextafter(v, np.float32(2))
    return np.array(out, dtype=np.float32)


def test_nearest_code_exact_near_every_midpoint(cb):
    ys = near_midpoint_values(cb, ulps=6)
    got = nf4.nearest_code(ys, cb)
    want = np.array([exact_nearest(y, cb) for y in ys])
    assert np.array_equal(got, want)


def test_nearest_code_exact_random_and_special(cb):
    rng = np.random.default_rng(3)
    ys = np.concatenate([
        rng.uniform(-1, 1, 3000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-38, 0.5, -0.5], dtype=np.float32),
        cb,
    ])
    got = nf4.nearest_code(ys, cb)
    want = np.array([exact_nearest(y, cb) for y in ys])
    assert np.array_equal(got, want)
    assert np.array_equal(nf4.nearest_code(cb, cb), np.arange(16))


def test_tie_goes_to_lower_index():
    toy = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32)
    got = nf4.nearest_code(np.array([0.25, -0.25, 0.75, -0.75], dtype=np.float32), toy)
    assert got.tolist() == [2, 1, 3, 0]


def test_absmax_element_gets_an_end_code(cb):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((37, 64)) * 0.02).astype(np.float32)
    codes, a = nf4.nf4_codes(x, cb)
    codes = codes.reshape(37, 64)
    idx = np.argmax(np.abs(x), axis=1)
    for b in range(37):
        v = x[b, idx[b]]
        assert a[b] == abs(v)
        assert codes[b, idx[b]] == (15 if v > 0 else 0)


def test_zero_block_and_negative_zero(cb):
    x = np.zeros(130, dtype=np.float32)
    x[64] = -0.0
    x[100] = 0.25
    x[128] = -0.0
    t = nf4.quantize(x, cb)
    codes = nf4.unpack_codes(t.codes, x.size)
    assert t.absmax[0] == 0.0 and t.absmax[2] == 0.0
    assert np.all(codes[:64] == 7) and np.all(codes[128:] == 7)
    assert codes[64] == 7 and codes[100] == 15
    w = nf4.dequantize(t, cb)
    assert np.all(w[:64] == 0.0) and np.all(w[128:] == 0.0)


def test_blocks_are_independent_and_tail_is_zero_padding(cb):
    """Permuting whole blocks permutes codes; a partial tail block equals the
    same data zero-padded to a full block (zeros never change an absmax)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(64 * 9 + 23) * 0.02).astype(np.float32)
    c1, a1 = nf4.nf4_codes(x, cb)
    xp = np.concatenate([x, np.zeros(64 - 23, dtype=np.float32)])
    c2, a2 = nf4.nf4_codes(xp, cb)
    assert np.array_equal(c1, c2[:x.size]) and np.array_equal(a1, a2)
    perm = rng.permutation(10)
    xb = xp.reshape(10, 64)[perm].reshape(-1)
    c3, a3 = nf4.nf4_codes(xb, cb)
    assert np.array_equal(c3.reshape(10, 64), c2.reshape(10, 64)[perm])
    assert np.array_equal(a3, a2[perm])


def test_scaling_by_power_of_two_keeps_codes(cb):
    """y = x / absmax is invariant under x -> 2^e x (exact in fp32)."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(64 * 20) * 0.02).astype(np.float32)
    c1, _ = nf4.nf4_codes(x, cb)
    for e in (-20, -3, 5, 30):
        c2, _ = nf4.nf4_codes((x * np.float32(2.0 ** e)).astype(np.float32), cb)
        assert np.array_equal(c1, c2)


def test_pack_high_nibble_first_and_odd_tail():
    codes = np.array([1, 2, 3, 4, 5], dtype=np.uint8)
    p = nf4.pack_codes(codes)
    assert p.tolist() == [0x12, 0x34, 0x50]
    assert nf4.unpack_codes(p, 5).tolist() == [1, 2, 3, 4, 5]


def test_tree_sum_matches_fsum_and_all_equal_is_exact():
    rng = np.random.default_rng(7)
    for n in (1, 2, 3, 255, 256, 257, 1000, 4097):
        a = rng.uniform(0.01, 0.2, n).astype(np.float32)
        mu = nf4.dq_mean(a)
        exact = math.fsum(float(v) for v in a) / n
        assert abs(float(mu) - exact) <= float(np.spacing(np.float32(exact)))
    a = np.full(1000, np.float32(0.0375), dtype=np.float32)
    assert nf4.dq_mean(a) == np.float32(0.0375)


def test_dq_codes_are_nearest_int8_levels():
    rng = np.random.default_rng(8)
    a = np.abs(rng.standard_normal(256 * 5 + 77) * 0.05).astype(np.float32)
    q, scale, mu = nf4.double_quantize(a)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    d = (a - mu).astype(np.float32)
    checked = 0
    for i in range(a.size):
        s2 = Fraction(float(scale[i // 256]))
        v = Fraction(127) * Fraction(float(d[i])) / s2
        fl = math.floor(v)
        frac = v - fl
        exact = fl + (1 if frac > Fraction(1, 2) else 0)
        if frac == Fraction(1, 2):
            exact = fl if fl % 2 == 0 else fl + 1
        if abs(float(frac) - 0.5) < 1e-4:
            assert abs(int(q[i]) - exact) <= 1
        else:
            assert int(q[i]) == exact
            checked += 1
    assert checked > 0.99 * a.size
    # each block's largest |a - mean| maps to +-127
    for b in range(scale.size):
        blk = d[b * 256:(b + 1) * 256]
        j = np.argmax(np.abs(blk))
        assert abs(int(q[b * 256 + j])) == 127


def test_dq_reconstruction_error_bound():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_normal(256 * 12) * 0.05).astype(np.float32)
    q, scale, mu = nf4.double_quantize(a)
    cp = nf4.dq_reconstruct(q, scale, mu)
    s_el = np.repeat(scale, 256)[:a.size].astype(np.float64)
    err = np.abs(cp.astype(np.float64) - a.astype(np.float64))
    slack = 1e-6 * (np.abs(a) + abs(float(mu)) + s_el)
    assert np.all(err <= s_el / 254.0 + slack)


def test_dq_zero_scale_block():
    a = np.full(300, np.float32(0.125), dtype=np.float32)
    q, scale, mu = nf4.double_quantize(a)
    assert mu == np.float32(0.125) and np.all(scale == 0) and np.all(q == 0)
    assert np.all(nf4.dq_reconstruct(q, scale, mu) == np.float32(0.125))


def test_roundtrip_codebook_valued_blocks_is_exact(cb):
    """Blocks built as fp32(c[code] * a) with a common a and an end code in
    every block: mean = a, scale = 0, c' = a, so dequantize returns the input
    bit for bit and the codes come back."""
    rng = np.random.default_rng(10)
    a = np.float32(0.0371)
    nblk = 300
    codes = rng.integers(0, 16, size=(nblk, 64)).astype(np.uint8)
    codes[:, 5] = rng.choice([0, 15], size=nblk)
    x = (cb[codes] * a).astype(np.float32).reshape(-1)
    t = nf4.quantize(x, cb)
    assert np.all(t.absmax == a) and t.dq_mean == a
    assert np.all(t.absmax_q == 0) and np.all(t.dq_scale == 0)
    assert np.array_equal(nf4.unpack_codes(t.codes, x.size), codes.reshape(-1))
    w = nf4.dequantize(t, cb)
    assert np.array_equal(w.view(np.uint32), x.view(np.uint32))


def test_requantize_is_idempotent_on_codes(cb):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    t = nf4.quantize(x, cb)
    assert np.all(nf4.dq_reconstruct(t.absmax_q, t.dq_scale, t.dq_mean) > 0)
    w = nf4.dequantize(t, cb)
    t2 = nf4.quantize(w, cb)
    assert np.array_equal(t2.codes, t.codes)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5], dtype=np.float32)
    got = nf4.f32_to_bf16_rne(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even is 1.0; 1+3*2^-8 ties up to 1+2^-6
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020]


def test_storage_closed_form_against_page_figures():
    claims = json.load(open(GOLDEN))
    n = 4096 * 4096
    nb, nd = n // 64, n // 64 // 256
    assert nf4.storage_bytes(n) == n // 2 + nb + 4 * nd + 4
    assert nf4.storage_bytes(65536) == 33812
    assert nf4.storage_bytes(4096 * 11008) == 23259908
    assert nf4.storage_bytes(8192 * 22016) == 93039620
    bits_dq = nf4.bits_per_param(n)
    bits_no_dq = 4.0 + 32.0 / 64.0                        # fp32 absmax per block
    saving = bits_no_dq - bits_dq
    assert abs(saving - claims["dq_saving_bits_per_param"]["value"]) < 0.05
    const_no_dq = 32.0 / 64.0
    const_dq = 8.0 / 64.0 + 32.0 / (64.0 * 256.0)
    factor = const_no_dq / const_dq
    assert claims["dq_constant_reduction_factor"]["min"] <= factor <= claims["dq_constant_reduction_factor"]["max"]
    share = const_dq / bits_dq
    assert claims["constants_share_of_model"]["min"] <= share <= claims["constants_share_of_model"]["max"]
    assert abs(16.0 / bits_dq - claims["nf4_compression_vs_16bit"]["value"]) < 0.2
    assert claims["dq_constant_bits"]["value"] == 8


# --- planted mistakes: each broken copy of the oracle must fail some pin ---

def _ties_upper(y, codebook, chunk=1 << 20):
    y = np.asarray(y, dtype=np.float32).reshape(-1).astype(np.float64)
    d = np.abs(y[:, None] - codebook.astype(np.float64)[None, ::-1])
    return (codebook.size - 1 - np.argmin(d, axis=1)).astype(np.uint8)


def _absmax_no_abs(x, block=nf4.NF4_BLOCK):
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    nb = -(-x.size // block)
    pad = np.zeros(nb * block, dtype=np.float32)
    pad[:x.size] = x
    return pad.reshape(nb, block).max(axis=1)


def _pack_low_first(codes):
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return ((c[1::2] << 4) | c[0::2]).astype(np.uint8)


def _dq_no_mean(absmax):
    a = np.asarray(absmax, dtype=np.float32)
    nd = -(-a.size // 256)
    pad = np.zeros(nd * 256, dtype=np.float32); pad[:a.size] = a
    scale = np.abs(pad).reshape(nd, 256).max(axis=1).astype(np.float32)
    t = (a / np.repeat(scale, 256)[:a.size]).astype(np.float32)
    q = np.clip(np.rint(t * np.float32(127)), -127, 127).astype(np.int8)
    return q, scale, nf4.dq_mean(a)


_MUTANTS = [
    ("nearest_code", _ties_upper, ["test_tie_goes_to_lower_index"]),
    ("block_absmax", _absmax_no_abs, ["test_absmax_element_gets_an_end_code"]),
    ("pack_codes", _pack_low_first, ["test_pack_high_nibble_first_and_odd_tail"]),
    ("double_quantize", _dq_no_mean, ["test_dq_reconstruction_error_bound"]),
]


@pytest.mark.parametrize("fname,mut,pins", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_planted_quantizer_mistakes_are_caught(monkeypatch, fname, mut, pins):
    monkeypatch.setattr(nf4, fname, mut)
    cbk = nf4.nf4_codebook()
    caught = False
    for pin in pins:
        fn = globals()[pin]
        try:
            if "cb" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                fn(cbk)
            else:
                fn()
        except AssertionError:
            caught = True
    assert caught
