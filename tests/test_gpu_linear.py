"""GPU parity of qlora_linear_fwd / qlora_linear_bwd (and the variants that
keep and reuse the adapter activations) against the fp64 oracle.

Bar (relative Frobenius error against the oracle evaluated on the exact
inputs: bf16 X and dY, the oracle's fp32 dequantized weight, fp32 A and B):
2e-2 for Y, dX, dA and dB. A tighter regression bound (5e-3) is asserted too,
since bf16 operand rounding gives about 1e-3. The same 2e-2 bar holds on every
256 x 256 tile of each result (gpu_util.max_tile_rel), so a wrong tile, strip
or tile edge cannot hide in the whole tensor's norm. With X = I and no adapter the
output must be bf16(W-hat^T) bit for bit (one nonzero product per output);
the same holds for dX with dY = I.
"""
import numpy as np
import pytest

import synth
from oracle import linear, nf4
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = 2e-2
REG = 5e-3


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_nf4_quantized_03_amd as m
    return m


@pytest.fixture(scope="module")
def cb():
    return nf4.nf4_codebook()


class Case:
    """Device copies plus oracle inputs of one workload."""

    def __init__(self, qb, wl, cb):
        self.wl = wl
        w32 = wl.W_f32()
        self.W_dev = gu.dev_f32(w32) if wl.w_dtype == "f32" else gu.dev_bf16(wl.W)
        gu.announce(f"quantize {wl.name} N={wl.N} K={wl.K}")
        self.q = qb.qlora_nf4_quantize(self.W_dev)
        self.ref_q = nf4.quantize(w32, cb)
        self.What = nf4.dequantize(self.ref_q, cb)
        self.X = gu.dev_bf16(wl.X)
        self.X32 = synth.bf16_to_f32(wl.X)
        self.A = gu.dev_f32(wl.A) if wl.A is not None else None
        self.B = gu.dev_f32(wl.B) if wl.B is not None else None
        self.dY = gu.dev_bf16(wl.dY) if wl.dY is not None else None
        self.dY32 = synth.bf16_to_f32(wl.dY) if wl.dY is not None else None


def _fwd(qb, c, label):
    wl = c.wl
    gu.announce(f"fwd {label} M={wl.M} N={wl.N} K={wl.K} r={wl.r}")
    Y = qb.qlora_linear_fwd(c.X, c.q, c.A, c.B, wl.s)
    Yg = gu.host_bf16_f32(Y)
    Yr = linear.forward(c.X32, c.What, wl.A, wl.B, wl.s)
    e = gu.rel_fro(Yg, Yr)
    assert e <= TOL, f"{label}: fwd rel err {e}"
    assert e <= REG, f"{label}: fwd rel err {e} above regression bound"
    et = gu.max_tile_rel(Yg, Yr)
    assert et <= TOL, f"{label}: fwd worst tile rel err {et}"
    return e


def _bwd(qb, c, label):
    wl = c.wl
    gu.announce(f"bwd {label} M={wl.M} N={wl.N} K={wl.K} r={wl.r}")
    dX, dA, dB = qb.qlora_linear_bwd(c.dY, c.X, c.q, c.A, c.B, wl.s)
    rX, rA, rB = linear.backward(c.dY32, c.X32, c.What, wl.A, wl.B, wl.s)
    pairs = {"dX": (gu.host_bf16_f32(dX), rX)}
    if wl.r > 0:
        pairs["dA"] = (gu.host(dA), rA)
        pairs["dB"] = (gu.host(dB), rB)
    errs = {}
    for k, (got, ref) in pairs.items():
        e = errs[k] = gu.rel_fro(got, ref)
        assert e <= TOL, f"{label}: {k} rel err {e}"
        assert e <= REG, f"{label}: {k} rel err {e} above regression bound"
        et = gu.max_tile_rel(got, ref)
        assert et <= TOL, f"{label}: {k} worst tile rel err {et}"
    return errs


def test_tiny_fwd_bwd(qb, cb):
    c = Case(qb, synth.workload("tiny"), cb)
    _fwd(qb, c, "tiny")
    _bwd(qb, c, "tiny")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16, 17, 33, 130, 300])
@pytest.mark.parametrize("r", [0, 8, 64, 72])
def test_ragged_m_and_rank(qb, cb, M, r):
    wl = synth.make_linear_workload("ragged", M=M, N=320, K=448, r=r, alpha=16.0,
                                    seed=M * 100 + r, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"ragged M={M} r={r}")
    _bwd(qb, c, f"ragged M={M} r={r}")


@pytest.mark.parametrize("M", [1, 130, 300])
def test_max_rank(qb, cb, M):
    """r = 256, the largest rank the boundary accepts: four 64-column adapter
    tiles in the down-projection, the gradient tiles and the GEMMs' adapter
    steps, with ragged M, N = 320 and K = 448 (reduction lengths of 5 and 7
    steps of 64)."""
    wl = synth.make_linear_workload("maxrank", M=M, N=320, K=448, r=256, alpha=16.0,
                                    seed=7000 + M, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"max rank M={M}")
    _bwd(qb, c, f"max rank M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 16, 23, 32])
@pytest.mark.parametrize("r", [0, 8, 72])
def test_decode_split_k_ragged(qb, cb, M, r):
    """Skinny-M forward with several K splits, a short last split, K not a
    multiple of 256 (absmax bytes not dword aligned) and a partial column strip."""
    wl = synth.make_linear_workload("decode-ragged", M=M, N=320, K=2240, r=r, alpha=16.0,
                                    seed=7000 + M * 10 + r, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"decode-ragged M={M} r={r}")


@pytest.mark.parametrize("K", [4160, 11072])
@pytest.mark.parametrize("r", [1, 3, 9])
def test_decode_one_row_odd_rank(qb, cb, K, r):
    """One row of X with a rank that is not a multiple of 4 (the row-stream
    kernel then reads the B rows with single-word loads), and workgroups whose
    rows hold a block count that is not a multiple of 4, so the last word of
    their int8 constants is partial: N = 64 with K = 4160 (65 blocks a row, 5
    rows a workgroup) and K = 11072 (173 blocks a row, 2 rows a workgroup)."""
    wl = synth.make_linear_workload("decode-odd-rank", M=1, N=64, K=K, r=r, alpha=16.0,
                                    seed=7200 + K + r, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"decode-odd-rank K={K} r={r}")


@pytest.mark.parametrize("M", [1, 3])
def test_decode_long_rows(qb, cb, M):
    """K = 16448 (514 chunks of 32 elements per row, past what the row-stream
    decode keeps in registers): the matrix-core decode path at M <= 4, with
    r = 9."""
    wl = synth.make_linear_workload("decode-long", M=M, N=128, K=16448, r=9, alpha=16.0,
                                    seed=7100 + M, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"decode-long M={M}")


def test_identity_input_gives_exact_weight(qb, cb):
    """X = I (M = K), no adapter: Y[m, n] = bf16(w-hat[n, m]) exactly.
    dY = I (M = N): dX = bf16(w-hat) exactly."""
    import torch
    N, K = 192, 256
    rng = np.random.default_rng(3)
    w = synth.normal_f32(rng, (N, K), 0.02)
    q = qb.qlora_nf4_quantize(gu.dev_f32(w))
    What = nf4.dequantize(nf4.quantize(w, cb), cb)
    gu.announce("identity fwd")
    X = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    Y = qb.qlora_linear_fwd(X, q)
    assert np.array_equal(gu.host_bf16_bits(Y), nf4.f32_to_bf16_rne(What.T.copy()))
    gu.announce("identity bwd")
    dY = torch.eye(N, dtype=torch.bfloat16, device="cuda")
    X2 = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    dX, _, _ = qb.qlora_linear_bwd(dY, X2, q)
    assert np.array_equal(gu.host_bf16_bits(dX), nf4.f32_to_bf16_rne(What))


@pytest.mark.parametrize("M,N,K,r", [(33, 512, 2048, 64), (100, 832, 2048, 0), (256, 768, 1024, 8),
                                     (300, 512, 2048, 72), (128, 4096, 4096, 64)])
def test_mid_m_split_reduction(qb, cb, M, N, K, r):
    """33 <= M <= 300: few 256 x 256 output tiles, so the large-tile GEMMs
    split their reduction (forward over K, dX over N) into up to 16 ranges of
    at least four 64-deep steps, write fp32 partials and sum them in split
    order into bf16. Splits here: forward 8, 8, 4, 8, 16; dX 2, 3, 3, 2, 16
    (N = 832 is 13 steps: dX splits of 5, 5 and 3 steps)."""
    wl = synth.make_linear_workload("midm", M=M, N=N, K=K, r=r, alpha=16.0,
                                    seed=7300 + M + r, w_dtype="bf16")
    c = Case(qb, wl, cb)
    _fwd(qb, c, f"mid-M M={M} N={N} K={K} r={r}")
    _bwd(qb, c, f"mid-M M={M} N={N} K={K} r={r}")


def test_identity_input_exact_with_split_reduction(qb, cb):
    """X = I (M = K = 512, N = 256) and dY = I (M = N = 512, K = 256): two
    output tiles, so both GEMMs split their reduction in two; the partial
    without the nonzero product adds +0, so Y = bf16(W-hat^T) and
    dX = bf16(W-hat) still hold bit for bit."""
    import torch
    rng = np.random.default_rng(5)
    for N, K in ((256, 512), (512, 256)):
        w = synth.normal_f32(rng, (N, K), 0.02)
        q = qb.qlora_nf4_quantize(gu.dev_f32(w))
        What = nf4.dequantize(nf4.quantize(w, cb), cb)
        if K == 512:
            gu.announce("identity fwd, split reduction")
            Y = qb.qlora_linear_fwd(torch.eye(K, dtype=torch.bfloat16, device="cuda"), q)
            assert np.array_equal(gu.host_bf16_bits(Y), nf4.f32_to_bf16_rne(What.T.copy()))
        else:
            gu.announce("identity bwd, split reduction")
            dY = torch.eye(N, dtype=torch.bfloat16, device="cuda")
            dX, _, _ = qb.qlora_linear_bwd(dY, torch.zeros((N, K), dtype=torch.bfloat16, device="cuda"), q)
            assert np.array_equal(gu.host_bf16_bits(dX), nf4.f32_to_bf16_rne(What))


def _saved(qb, c, label):
    """qlora_linear_fwd_save / qlora_linear_bwd_saved: Y bit-identical to
    qlora_linear_fwd's; Hs = bf16(s X A^T) against the oracle's fp64 down
    projection (bf16 rounding only: regression bound); the backward from Hs
    against the oracle like qlora_linear_bwd, and repeatable bit for bit.
    With fewer than 64 values of H (M r < 64) dA and dB are scaled copies of
    a few dot products, whose relative error can exceed the regression bound
    by chance; the 2e-2 bar still holds there."""
    wl = c.wl
    reg = REG if wl.M * wl.r >= 64 else TOL
    gu.announce(f"fwd_save/bwd_saved {label} M={wl.M} N={wl.N} K={wl.K} r={wl.r}")
    Y0 = qb.qlora_linear_fwd(c.X, c.q, c.A, c.B, wl.s)
    Y, Hs = qb.qlora_linear_fwd_save(c.X, c.q, c.A, c.B, wl.s)
    assert np.array_equal(gu.host_bf16_bits(Y), gu.host_bf16_bits(Y0)), f"{label}: Y differs from qlora_linear_fwd"
    Hr = wl.s * linear.lora_down(c.X32, wl.A)
    e = gu.rel_fro(gu.host_bf16_f32(Hs), Hr)
    assert e <= reg, f"{label}: Hs rel err {e}"
    rX, rA, rB = linear.backward(c.dY32, c.X32, c.What, wl.A, wl.B, wl.s)
    outs = []
    for _ in range(2):
        dX, dA, dB = qb.qlora_linear_bwd_saved(c.dY, c.X, Hs, c.q, c.A, c.B, wl.s)
        outs.append((gu.host_bf16_bits(dX), gu.host(dA), gu.host(dB)))
        for k, got, ref in (("dX", gu.host_bf16_f32(dX), rX), ("dA", gu.host(dA), rA), ("dB", gu.host(dB), rB)):
            e = gu.rel_fro(got, ref)
            assert e <= (REG if k == "dX" else reg), f"{label}: saved {k} rel err {e}"
            et = gu.max_tile_rel(got, ref)
            assert et <= TOL, f"{label}: saved {k} worst tile rel err {et}"
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{label}: saved backward not repeatable"


@pytest.mark.parametrize("M", [1, 17, 33, 300])
@pytest.mark.parametrize("r", [1, 8, 64, 72, 256])
def test_saved_activations_ragged(qb, cb, M, r):
    """The saved-activation forward and backward with ragged M (the decode
    path for M <= 32, the large-tile path above), ranks below, at and above
    one 64-column adapter tile (r not a multiple of 64: the caller's [M, r]
    is padded to the kernels' width and back) up to the largest accepted
    rank."""
    wl = synth.make_linear_workload("saved", M=M, N=320, K=448, r=r, alpha=16.0,
                                    seed=9000 + M * 10 + r, w_dtype="bf16")
    _saved(qb, Case(qb, wl, cb), f"saved M={M} r={r}")


@pytest.mark.parametrize("M,N,K,r", [(128, 512, 2048, 72), (100, 832, 2048, 64)])
def test_saved_activations_with_split_reduction(qb, cb, M, N, K, r):
    """The saved pair where the forward and dX GEMMs split their reduction
    (few output tiles): the caller's Hs feeds split 0's adapter steps."""
    wl = synth.make_linear_workload("saved-split", M=M, N=N, K=K, r=r, alpha=16.0, seed=9500 + M + r,
                                    w_dtype="bf16")
    _saved(qb, Case(qb, wl, cb), f"saved split M={M} N={N} K={K} r={r}")


def test_saved_activations_attn7b(qb, cb):
    """The 7B attention projection at full size (M = 4096, r = 64: the caller's
    Hs is used in place by the GEMMs)."""
    _saved(qb, Case(qb, synth.workload("attn7b"), cb), "attn7b")


def test_zero_scale_and_zero_adapter(qb, cb):
    wl = synth.make_linear_workload("zs", M=64, N=256, K=256, r=8, alpha=0.0, seed=9)
    c = Case(qb, wl, cb)
    dX, dA, dB = qb.qlora_linear_bwd(c.dY, c.X, c.q, c.A, c.B, 0.0)
    assert np.all(gu.host(dA) == 0) and np.all(gu.host(dB) == 0)
    import torch
    Y0 = qb.qlora_linear_fwd(c.X, c.q, torch.zeros_like(c.A), c.B, 2.0)
    Yn = qb.qlora_linear_fwd(c.X, c.q)
    assert torch.equal(Y0, Yn)


@pytest.mark.parametrize("name", ["gate7b_m1", "gate7b_m4", "gate7b_m16",
                                  "down7b_m1", "down7b_m4", "down7b_m16"])
def test_decode_shapes_full(qb, cb, name):
    c = Case(qb, synth.workload(name), cb)
    _fwd(qb, c, name)


def test_attn7b_full(qb, cb):
    c = Case(qb, synth.workload("attn7b"), cb)
    _fwd(qb, c, "attn7b")
    _bwd(qb, c, "attn7b")


@pytest.mark.parametrize("name", ["up65b", "down65b"])
def test_mlp65b_sampled(qb, cb, name):
    """65B MLP shapes at full size: Y and dX checked on 64 sampled rows (each
    row of the oracle needs only that row of X / dY); dA and dB in full."""
    wl = synth.workload(name)
    w32 = wl.W_f32()
    W_dev = gu.dev_bf16(wl.W)
    gu.announce(f"quantize {name}")
    q = qb.qlora_nf4_quantize(W_dev)
    del W_dev
    What = nf4.dequantize(nf4.quantize(w32, cb), cb)
    X, A, B, dY = gu.dev_bf16(wl.X), gu.dev_f32(wl.A), gu.dev_f32(wl.B), gu.dev_bf16(wl.dY)
    X32, dY32 = synth.bf16_to_f32(wl.X), synth.bf16_to_f32(wl.dY)
    rows = np.sort(np.random.default_rng(1).choice(wl.M, 64, replace=False))
    gu.announce(f"fwd {name}")
    Y = gu.host_bf16_f32(qb.qlora_linear_fwd(X, q, A, B, wl.s))
    Yr = linear.forward(X32[rows], What, wl.A, wl.B, wl.s)
    e = gu.rel_fro(Y[rows], Yr)
    assert e <= REG, f"{name}: fwd {e}"
    assert gu.max_tile_rel(Y[rows], Yr) <= TOL, f"{name}: fwd worst tile"
    gu.announce(f"bwd {name}")
    dX, dA, dB = qb.qlora_linear_bwd(dY, X, q, A, B, wl.s)
    dH = wl.s * (dY32.astype(np.float64) @ wl.B.astype(np.float64))
    rX = dY32[rows].astype(np.float64) @ What.astype(np.float64) + dH[rows] @ wl.A.astype(np.float64)
    rA = dH.T @ X32.astype(np.float64)
    rB = wl.s * (dY32.T.astype(np.float64) @ (X32.astype(np.float64) @ wl.A.T.astype(np.float64)))
    for k, got, ref in (("dX", gu.host_bf16_f32(dX)[rows], rX), ("dA", gu.host(dA), rA),
                        ("dB", gu.host(dB), rB)):
        e = gu.rel_fro(got, ref)
        assert e <= REG, f"{name}: {k} {e}"
        assert gu.max_tile_rel(got, ref) <= TOL, f"{name}: {k} worst tile"


@pytest.mark.parametrize("M", [16, 300])
@pytest.mark.parametrize("saved", [False, True])
def test_graph_replays_match_eager(qb, cb, M, saved):
    """The whole path captured as one HIP graph (quantize, dequantize, forward,
    backward; M = 16 takes the decode kernels, M = 300 the large-tile ones;
    with `saved` the forward keeps the adapter activations and the backward
    takes them) and replayed three times, with the outputs cleared and eager
    work on the same stream between replays: every replay reproduces the eager
    results bit for bit (the library allocates and clears nothing inside a
    call)."""
    import torch
    wl = synth.make_linear_workload("graph", M=M, N=320, K=448, r=72, alpha=16.0, seed=4000 + M, w_dtype="bf16")
    dev = torch.device("cuda:0")
    W = gu.dev_bf16(wl.W)
    X, dY = gu.dev_bf16(wl.X), gu.dev_bf16(wl.dY)
    A, B = gu.dev_f32(wl.A), gu.dev_f32(wl.B)
    q = qb.NF4Weight.empty(wl.N, wl.K, dev)
    ws_q = torch.empty(qb.qlora_nf4_quantize_workspace_bytes(wl.N, wl.K), dtype=torch.uint8, device=dev)
    ws_l = qb.linear_workspace(M, wl.N, wl.K, wl.r, dev)
    Wd = torch.empty((wl.N, wl.K), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, wl.K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((wl.r, wl.K), dtype=torch.float32, device=dev)
    dB = torch.empty((wl.N, wl.r), dtype=torch.float32, device=dev)
    Hs = torch.zeros((M, wl.r), dtype=torch.bfloat16, device=dev)   # untouched unless saved

    def step():
        qb.qlora_nf4_quantize(W, out=q, ws=ws_q)
        qb.qlora_nf4_dequantize(q, torch.bfloat16, out=Wd)
        if saved:
            qb.qlora_linear_fwd_save(X, q, A, B, wl.s, ws=ws_l, out=Y, hs=Hs)
            qb.qlora_linear_bwd_saved(dY, X, Hs, q, A, B, wl.s, ws=ws_l, outs=(dX, dA, dB))
        else:
            qb.qlora_linear_fwd(X, q, A, B, wl.s, ws=ws_l, out=Y)
            qb.qlora_linear_bwd(dY, X, q, A, B, wl.s, ws=ws_l, outs=(dX, dA, dB))

    gu.announce(f"graph capture M={M} saved={saved}")
    outs = (q.codes, q.absmax_q, q.dq_scale, q.dq_mean, Wd, Y, Hs, dX, dA, dB)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        _ = (X.float() * 2.0).sum()   # unrelated eager work on the stream between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("codes", "absmax_q", "dq_scale", "dq_mean", "Wd", "Y", "Hs", "dX", "dA", "dB"), outs,
                              eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"


def test_binding_rejects_mismatched_tensors(qb, cb):
    """Wrong shapes, dtypes or a missing factor are refused by the binding
    with an exception before anything is launched: the C ABI takes bare
    pointers and could not tell a short tensor from a long one."""
    import torch
    wl = synth.make_linear_workload("guard", M=8, N=128, K=192, r=8, alpha=16.0, seed=5)
    c = Case(qb, wl, cb)
    bad_X = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        qb.qlora_linear_fwd(bad_X, c.q, c.A, c.B, wl.s)
    with pytest.raises(ValueError):
        qb.qlora_linear_fwd(c.X, c.q, c.A[:, :64].contiguous(), c.B, wl.s)
    with pytest.raises(ValueError):
        qb.qlora_linear_fwd(c.X, c.q, c.A, None, wl.s)
    with pytest.raises(TypeError):
        qb.qlora_linear_fwd(c.X, c.q, c.A.double(), c.B, wl.s)
    with pytest.raises(ValueError):
        qb.qlora_linear_fwd(c.X, c.q, c.A, c.B, wl.s, out=torch.empty((8, 64), dtype=torch.bfloat16,
                                                                      device="cuda"))
    with pytest.raises(ValueError):
        qb.qlora_linear_bwd(c.dY[:, :64].contiguous(), c.X, c.q, c.A, c.B, wl.s)
    with pytest.raises(ValueError):
        qb.qlora_linear_bwd(c.dY, c.X, c.q, c.A, c.B, wl.s,
                            outs=(torch.empty((8, 192), dtype=torch.bfloat16, device="cuda"),
                                  torch.empty((8, 100), device="cuda"), torch.empty((128, 8), device="cuda")))
    with pytest.raises(ValueError):
        qb.qlora_nf4_dequantize(c.q, torch.float32, out=torch.empty((64, 192), device="cuda"))
    torch.cuda.synchronize()


def test_decode_sync_words_return_to_zero_and_results_repeat(qb):
    """The single-launch decode forward exchanges partials between workgroups
    through the workspace's leading synchronization words. After every call
    they are all zero again (no wait timed out, every counter and flag was
    cleared), one workspace serves several shapes in turn (split and unsplit
    reductions, adapter ranks 0 to 256), and repeated calls give bit-identical
    outputs."""
    import torch
    dev = torch.device("cuda:0")
    shapes = [(1, 11008, 4096, 64), (16, 4096, 11008, 64), (4, 320, 2240, 72), (32, 320, 448, 256),
              (7, 1024, 576, 0), (1, 64, 64, 8)]
    need = max(qb.qlora_linear_workspace_bytes(*s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    for rep in range(2):
        for (M, N, K, r) in shapes:
            gu.announce(f"decode sync M={M} N={N} K={K} r={r} rep={rep}")
            W = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            q = qb.qlora_nf4_quantize(W)
            X = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
            A = torch.randn((r, K), generator=gen, device=dev) * 0.01 if r else None
            B = torch.randn((N, r), generator=gen, device=dev) * 0.01 if r else None
            outs = [qb.qlora_linear_fwd(X, q, A, B, 0.25, ws=ws) for _ in range(3)]
            torch.cuda.synchronize()
            assert torch.count_nonzero(ws[:qb.LINEAR_SYNC_BYTES]).item() == 0, \
                f"sync words not cleared after M={M} N={N} K={K} r={r}"
            for o in outs[1:]:
                assert torch.equal(o, outs[0]), f"M={M} N={N} K={K} r={r}: repeated calls differ"
            fresh = qb.qlora_linear_fwd(X, q, A, B, 0.25)
            assert torch.equal(fresh, outs[0]), f"M={M} N={N} K={K} r={r}: shared workspace differs"



def test_large_m_counters_return_to_zero_and_results_repeat(qb):
    """Large-M forward and backward (split partials of the adapter
    down-projection, summed in a fixed split order): the workspace's leading
    synchronization words stay zero, repeated calls give bit-identical
    outputs and gradients, and a fresh workspace gives the same results.
    Shapes: split and unsplit reductions, ragged M, r = 8, 9 (rows of B not
    16-byte aligned), 72 (two column tiles) and 256."""
    import torch
    dev = torch.device("cuda:0")
    shapes = [(4096, 4096, 4096, 64), (300, 320, 448, 72), (33, 320, 448, 9), (130, 320, 448, 256),
              (2048, 1024, 8192, 8)]
    need = max(qb.qlora_linear_workspace_bytes(*s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    for (M, N, K, r) in shapes:
        gu.announce(f"large-M counters M={M} N={N} K={K} r={r}")
        W = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        q = qb.qlora_nf4_quantize(W)
        X = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
        dY = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16)
        A = torch.randn((r, K), generator=gen, device=dev) * 0.01
        B = torch.randn((N, r), generator=gen, device=dev) * 0.01
        fw = [qb.qlora_linear_fwd(X, q, A, B, 0.25, ws=ws) for _ in range(2)]
        bw = [qb.qlora_linear_bwd(dY, X, q, A, B, 0.25, ws=ws) for _ in range(2)]
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:qb.LINEAR_SYNC_BYTES]).item() == 0, \
            f"counters not cleared after M={M} N={N} K={K} r={r}"
        assert torch.equal(fw[0], fw[1]), f"M={M} N={N} K={K} r={r}: repeated forwards differ"
        for a, b in zip(bw[0], bw[1]):
            assert torch.equal(a, b), f"M={M} N={N} K={K} r={r}: repeated backwards differ"
        assert torch.equal(qb.qlora_linear_fwd(X, q, A, B, 0.25), fw[0])
        for a, b in zip(qb.qlora_linear_bwd(dY, X, q, A, B, 0.25), bw[0]):
            assert torch.equal(a, b), f"M={M} N={N} K={K} r={r}: fresh workspace differs"