"""GPU parity of qlora_nf4_merge (adapter merged into the quantized base, then
quantized again) against the oracle.

Bar: the requantized result bit-exact (packed codes and the stored constants:
fp32 absmax, or the int8 DQ codes, DQ scales and mean). The merged fp32
weight is defined with the rank sum in fp64 and one rounding, so both sides
reach the same fp32 values and hence the same codes.
"""
import numpy as np
import pytest

import synth
from oracle import merge, nf4
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_nf4_quantized_03_amd as m
    return m


def codebook(fmt):
    return nf4.fp4_codebook() if fmt & 2 else nf4.nf4_codebook()


def check_same(q, ref, label):
    codes = gu.host(q.codes)
    assert np.array_equal(codes, ref.codes), f"{label}: codes differ at {np.flatnonzero(codes != ref.codes)[:10]}"
    if ref.dq:
        assert np.array_equal(gu.host(q.absmax_q), ref.absmax_q), f"{label}: DQ codes differ"
        assert np.array_equal(gu.host(q.dq_scale).view(np.uint32), ref.dq_scale.view(np.uint32)), label
        assert gu.host(q.dq_mean).view(np.uint32)[0] == np.float32(ref.dq_mean).view(np.uint32), label
    else:
        assert np.array_equal(gu.host(q.absmax).view(np.uint32), ref.absmax.view(np.uint32)), \
            f"{label}: fp32 constants differ"


def run_case(qb, N, K, r, s, fin, fout, seed, label):
    rng = np.random.default_rng(seed)
    w = synth.normal_f32(rng, (N, K), 0.02)
    A = (rng.standard_normal((r, K)) * 0.01).astype(np.float32) if r else None
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32) if r else None
    gu.announce(f"merge {label} N={N} K={K} r={r} fmt {fin}->{fout}")
    W = qb.qlora_nf4_quantize(gu.dev_f32(w), fmt=fin)
    q = qb.qlora_nf4_merge(W, gu.dev_f32(A) if r else None, gu.dev_f32(B) if r else None, s, fmt=fout)
    base = nf4.quantize(w, codebook(fin), double_quant=not fin & 1)
    ref = merge.merge_requantize(base, codebook(fin), A, B, s, codebook(fout), not fout & 1)
    check_same(q, ref, label)
    return W, q


@pytest.mark.parametrize("fin,fout", [(0, 0), (1, 1), (0, 3), (3, 0), (2, 2)])
@pytest.mark.parametrize("N,K,r", [(3, 333, 5), (70, 300, 8), (256, 512, 64), (64, 1024, 256), (33, 4160, 1)])
def test_merge_matches_oracle(qb, fin, fout, N, K, r):
    run_case(qb, N, K, r, 0.37, fin, fout, seed=N * 31 + K + r + 7 * fin + fout, label="ragged")


@pytest.mark.parametrize("fin,fout", [(0, 0), (0, 1), (1, 2), (3, 0)])
def test_rank_zero_requantizes(qb, fin, fout):
    """r = 0: the base is dequantized and quantized again (a format change)."""
    run_case(qb, 48, 320, 0, 0.0, fin, fout, seed=90 + fin * 4 + fout, label="rank 0")


def test_merge_in_place(qb):
    """out = W: the base is read completely before the output is written."""
    rng = np.random.default_rng(5)
    N, K, r = 96, 448, 16
    w = synth.normal_f32(rng, (N, K), 0.02)
    A = gu.dev_f32((rng.standard_normal((r, K)) * 0.01).astype(np.float32))
    B = gu.dev_f32((rng.standard_normal((N, r)) * 0.01).astype(np.float32))
    gu.announce("merge in place")
    W1 = qb.qlora_nf4_quantize(gu.dev_f32(w))
    W2 = qb.qlora_nf4_quantize(gu.dev_f32(w))
    q = qb.qlora_nf4_merge(W1, A, B, 0.5)
    qb.qlora_nf4_merge(W2, A, B, 0.5, out=W2)
    for a, b in ((q.codes, W2.codes), (q.absmax_q, W2.absmax_q), (q.dq_scale, W2.dq_scale), (q.dq_mean, W2.dq_mean)):
        assert np.array_equal(gu.host(a), gu.host(b))


def test_attn7b_merge_full(qb):
    """The 7B attention projection (4096 x 4096, r = 64, s = 0.25) at full size."""
    wl = synth.workload("attn7b")
    w32 = synth.bf16_to_f32(wl.W)
    gu.announce("merge attn7b 4096x4096 r=64")
    W = qb.qlora_nf4_quantize(gu.dev_bf16(wl.W))
    q = qb.qlora_nf4_merge(W, gu.dev_f32(wl.A), gu.dev_f32(wl.B), wl.s)
    cb = nf4.nf4_codebook()
    ref = merge.merge_requantize(nf4.quantize(w32, cb), cb, wl.A, wl.B, wl.s, cb, True)
    check_same(q, ref, "attn7b")
