"""Pins of the oracle's AdamW step.

The checks rest on the textbook AdamW update evaluated in fp64 (the fp32
step must stay within a few fp32 ulps of it), on closed forms (the first step
from zero state moves each parameter by lr g / (|g| + eps), about lr sign(g); with
beta1 = beta2 = 0 the update is g / (|g| + eps)), and on invariants (zero
gradient without decay leaves parameters and a zero state unchanged; decay
alone shrinks parameters by the factor the decoupled form gives).
"""
import numpy as np
import pytest

from oracle import adamw

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def textbook_f64(p, g, m, v, lr, beta1, beta2, eps, wd, t):
    """AdamW in fp64 on the fp32 values of every input and hyperparameter."""
    p, g, m, v = (np.asarray(a, np.float64) for a in (p, g, m, v))
    lr, beta1, beta2, eps, wd = (float(np.float32(x)) for x in (lr, beta1, beta2, eps, wd))
    m2 = beta1 * m + (1 - beta1) * g
    v2 = beta2 * v + (1 - beta2) * g * g
    mh = m2 / (1 - beta1 ** t)
    vh = v2 / (1 - beta2 ** t)
    return p - lr * (mh / (np.sqrt(vh) + eps) + wd * p), m2, v2


def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    return p, g, m, v


@pytest.mark.parametrize("t", [1, 2, 10, 1000])
def test_close_to_textbook_fp64(t):
    p, g, m, v = _state(20000, t)
    if t == 1:
        m[:] = 0
        v[:] = 0
    bc1, bc2 = adamw.bias_corrections(HP["beta1"], HP["beta2"], t)
    p2, m2, v2 = adamw.adamw_step(p, g, m, v, bc1=bc1, bc2=bc2, **HP)
    rp, rm, rv = textbook_f64(p, g, m, v, t=t, **HP)
    # m' may cancel (m and g of opposite signs): bound by the terms' size,
    # three roundings of at most half an fp32 ulp each
    scale_m = np.abs(np.float64(np.float32(HP["beta1"])) * m) + np.abs((1 - np.float64(np.float32(HP["beta1"]))) * g)
    assert np.all(np.abs(m2 - rm) <= 1.5 * 2.0 ** -23 * scale_m + 1e-45)
    assert np.max(np.abs(v2 - rv) / np.maximum(np.abs(rv), 1e-30)) < 6e-7
    # the parameter change (lr-sized) is where the fp32 rounding shows
    dp, rdp = p2.astype(np.float64) - p, rp - p
    assert np.max(np.abs(dp - rdp)) <= 4 * np.spacing(np.abs(p)).max() + 1e-6 * np.abs(rdp).max()


def test_first_step_from_zero_state_is_about_lr_sign_g():
    p, g, m, v = _state(5000, 3)
    m[:] = 0
    v[:] = 0
    bc1, bc2 = adamw.bias_corrections(0.9, 0.999, 1)
    p2, _, _ = adamw.adamw_step(p, g, m, v, 1e-3, 0.9, 0.999, 1e-8, 0.0, bc1, bc2)
    # mh = g and vh = g^2 up to rounding, so the step is lr g / (|g| + eps),
    # about lr sign(g); the fp32 spacing of p (~4e-9) bounds the difference
    want = 1e-3 * g.astype(np.float64) / (np.abs(g).astype(np.float64) + 1e-8)
    assert np.allclose((p - p2).astype(np.float64), want, rtol=2e-5, atol=0)


def test_no_momentum_closed_form():
    p, g, m, v = _state(5000, 4)
    p2, m2, v2 = adamw.adamw_step(p, g, m, v, 1e-2, 0.0, 0.0, 1e-8, 0.0, 1.0, 1.0)
    assert np.array_equal(m2, g) and np.array_equal(v2, (g * g).astype(np.float32))
    want = p.astype(np.float64) - 1e-2 * g / (np.abs(g).astype(np.float64) + 1e-8)
    # p and the step (about lr) may cancel: bound by two fp32 spacings of the
    # largest of p, the step and the result (the step's own rounding and the
    # final subtraction)
    big = np.maximum(np.maximum(np.abs(p), np.float32(1e-2)), np.abs(want).astype(np.float32))
    assert np.all(np.abs(p2 - want) <= 2 * np.spacing(big))


def test_zero_gradient_invariants():
    p, g, m, v = _state(4096, 5)
    g[:] = 0
    z = np.zeros_like(p)
    p2, m2, v2 = adamw.adamw_step(p, g, z, z, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0.1, 0.001)
    assert np.array_equal(p2, p) and not m2.any() and not v2.any()
    # decay alone: p' = p - lr wd p
    p3, _, _ = adamw.adamw_step(p, g, z, z, 1e-2, 0.9, 0.999, 1e-8, 0.1, 0.1, 0.001)
    assert np.allclose(p3, p * (1 - 1e-3), rtol=1e-6, atol=0)


def test_planted_mistakes_are_caught(monkeypatch):
    """A swapped bias correction or a coupled (L2) decay fails the pins."""
    real = adamw.adamw_step

    def swapped(p, g, m, v, lr, beta1, beta2, eps, wd, bc1, bc2):
        return real(p, g, m, v, lr, beta1, beta2, eps, wd, bc2, bc1)
    monkeypatch.setattr(adamw, "adamw_step", swapped)
    with pytest.raises(AssertionError):
        test_close_to_textbook_fp64(10)
    monkeypatch.setattr(adamw, "adamw_step", real)

    def coupled(p, g, m, v, lr, beta1, beta2, eps, wd, bc1, bc2):
        g2 = (np.asarray(g, np.float32) + np.float32(wd) * np.asarray(p, np.float32)).astype(np.float32)
        return real(p, g2, m, v, lr, beta1, beta2, eps, 0.0, bc1, bc2)
    monkeypatch.setattr(adamw, "adamw_step", coupled)
    with pytest.raises(AssertionError):
        test_zero_gradient_invariants()
