"""Pins of the oracle's QLoRA linear forward and backward.

The forward is pinned by identities any correct implementation satisfies:
X = I gives back W-hat^T; the output equals X times the merged weight
W-hat + s B A (the adapter merge of the QLoRA vs ChatGPT page, capability
"adapter composition and merging"); the adapter's contribution has rank <= r;
s = 0 or a zero adapter leaves the base product. The backward is pinned by
central finite differences of L = <dY, Y> in fp64, a different computation
from the closed-form gradients. A final test plants mistakes in copies of the
oracle and checks that some pin catches each one.
"""
import numpy as np
import pytest

from oracle import linear


def _case(M=6, N=7, K=7, r=3, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.1
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    return X, W, A, B, dY


def fwd_pins(fwd):
    """Return a list of failure strings for the forward identities."""
    fails = []
    X, W, A, B, _ = _case()          # square W, so a transposed W still fits
    s = 1.75
    K = W.shape[1]
    I = np.eye(K)
    if not np.array_equal(fwd(I, W, A, B, 0.0), W.T):
        fails.append("identity input with s=0")
    Y = fwd(X, W, A, B, s)
    merged = X @ (W + s * (B @ A)).T
    if not np.allclose(Y, merged, rtol=1e-12, atol=1e-12):
        fails.append("merged-weight identity")
    D = Y - fwd(X, W, A, B, 0.0)
    sv = np.linalg.svd(D, compute_uv=False)
    if not np.all(sv[A.shape[0]:] < 1e-10 * max(1.0, sv[0])):
        fails.append("adapter term rank <= r")
    if not np.allclose(fwd(X, W, np.zeros_like(A), B, s), X @ W.T, rtol=1e-14, atol=1e-14):
        fails.append("zero A")
    Y2 = fwd(2.0 * X, W, A, B, s)
    if not np.allclose(Y2, 2.0 * Y, rtol=1e-13, atol=1e-13):
        fails.append("linearity in X")
    return fails


def fd_grads(fwd, X, W, A, B, dY, s, h=1e-6, picks=12, seed=1):
    """Central differences of L = sum(dY * Y) at random entries of X, A, B."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("X", "A", "B"):
        P = {"X": X, "A": A, "B": B}[name]
        vals = []
        for _ in range(picks):
            idx = tuple(rng.integers(0, d) for d in P.shape)
            Pp = P.copy(); Pp[idx] += h
            Pm = P.copy(); Pm[idx] -= h
            args_p = dict(X=X, A=A, B=B); args_p[name] = Pp
            args_m = dict(X=X, A=A, B=B); args_m[name] = Pm
            Lp = np.sum(dY * fwd(args_p["X"], W, args_p["A"], args_p["B"], s))
            Lm = np.sum(dY * fwd(args_m["X"], W, args_m["A"], args_m["B"], s))
            vals.append((idx, (Lp - Lm) / (2 * h)))
        out[name] = vals
    return out


def bwd_pins(fwd, bwd):
    fails = []
    X, W, A, B, dY = _case(seed=2)
    s = 0.6
    dX, dA, dB = bwd(dY, X, W, A, B, s)
    fd = fd_grads(fwd, X, W, A, B, dY, s)
    for name, G in (("X", dX), ("A", dA), ("B", dB)):
        for idx, g in fd[name]:
            if not abs(G[idx] - g) <= 1e-6 * max(1.0, abs(g)):
                fails.append(f"finite difference d{name}")
                break
    dX0, dA0, dB0 = bwd(dY, X, W, A, B, 0.0)
    if not (np.all(dA0 == 0) and np.all(dB0 == 0) and np.allclose(dX0, dY @ W)):
        fails.append("s = 0")
    _, _, dBz = bwd(dY, X, W, np.zeros_like(A), B, s)
    if not np.all(dBz == 0):
        fails.append("A = 0 gives dB = 0")
    _, dAz, _ = bwd(dY, X, W, A, np.zeros_like(B), s)
    if not np.all(dAz == 0):
        fails.append("B = 0 gives dA = 0")
    return fails


def test_forward_pins():
    assert fwd_pins(linear.forward) == []


def test_backward_pins():
    assert bwd_pins(linear.forward, linear.backward) == []


def test_no_adapter_is_plain_dequant_matmul():
    X, W, A, B, dY = _case()
    assert np.array_equal(linear.forward(X, W, None, None, 2.0), X @ W.T)
    dX, dA, dB = linear.backward(dY, X, W, None, None, 2.0)
    assert dA is None and dB is None and np.array_equal(dX, dY @ W)


def test_rel_fro():
    a = np.ones((3, 3))
    assert linear.rel_fro(a, a) == 0.0
    assert abs(linear.rel_fro(1.01 * a, a) - 0.01) < 1e-12
    assert linear.rel_fro(np.zeros(2), np.zeros(2)) == 0.0


# --- planted mistakes: each copy of the oracle must fail at least one pin ---

def _mut_fwd_drop_s(X, W, A, B, s):
    return np.asarray(X) @ np.asarray(W).T + (np.asarray(X) @ np.asarray(A).T) @ np.asarray(B).T


def _mut_fwd_sign(X, W, A, B, s):
    return np.asarray(X) @ np.asarray(W).T - s * (np.asarray(X) @ np.asarray(A).T) @ np.asarray(B).T


def _mut_fwd_transposed_w(X, W, A, B, s):
    return linear.forward(X, np.asarray(W).T, A, B, s)


def _mut_bwd_no_dh_term(dY, X, W, A, B, s):
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    return dX - (s * (np.asarray(dY) @ np.asarray(B))) @ np.asarray(A), dA, dB


def _mut_bwd_db_no_s(dY, X, W, A, B, s):
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    return dX, dA, (dB / s if s != 0 else dB)


def _mut_bwd_da_uses_dy(dY, X, W, A, B, s):
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    dH = np.asarray(dY) @ np.asarray(B)      # forgot s
    return dX, dH.T @ np.asarray(X), dB


def _mut_bwd_dx_transposed(dY, X, W, A, B, s):
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    return dX[:, ::-1].copy(), dA, dB


@pytest.mark.parametrize("mut", [_mut_fwd_drop_s, _mut_fwd_sign, _mut_fwd_transposed_w])
def test_planted_forward_mistakes_are_caught(mut):
    assert fwd_pins(mut) != []


@pytest.mark.parametrize("mut", [_mut_bwd_no_dh_term, _mut_bwd_db_no_s, _mut_bwd_da_uses_dy,
                                 _mut_bwd_dx_transposed])
def test_planted_backward_mistakes_are_caught(mut):
    assert bwd_pins(linear.forward, mut) != []
