"""Pins for the oracle's AdamW step (no GPU): a library implementation of the
same published method, and closed forms that follow from the update rule
(first step from zero state, constant gradient, zero gradient). Planted
variants with a plausible mistake (no bias correction, weight decay coupled
into the gradient) fail the closed forms."""

import numpy as np
import torch

import oracle


def _rand(n, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(n) * scale


def test_matches_torch_adamw_fp64_over_several_steps():
    """torch.optim.AdamW (its single-tensor loop, fp64 on the CPU) is an
    independent implementation of the same method."""
    n = 4096
    p0 = _rand(n, 1, 0.02)
    lr, b1, b2, eps, wd = 2e-4, 0.9, 0.999, 1e-8, 0.01
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 7):
        g = _rand(n, 100 + t, 10.0 ** (t % 3 - 2))
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, t, lr, b1, b2, eps, wd)
        st = opt.state[tp]
        # torch forms m by interpolation (m + (1 - b1)(g - m)): a different
        # rounding, so the agreement is normwise, to a few fp64 ulps
        for got, want in ((st["exp_avg"].numpy(), m), (st["exp_avg_sq"].numpy(), v)):
            assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))
        # the parameters agree to a few ulps of the step (p itself is ~0.02)
        assert np.max(np.abs(tp.detach().numpy() - p)) <= 1e-16 + 1e-12 * lr


def test_first_step_from_zero_state_is_sign_like():
    # m^ = g and v^ = g^2 at t = 1 from zero state: the step is lr g/(|g| + eps)
    g = _rand(1000, 2, 1e-3)
    p0 = _rand(1000, 3, 0.05)
    lr, eps, wd = 1e-3, 1e-8, 0.1
    p, m, v = oracle.adamw_step(p0, g, np.zeros(1000), np.zeros(1000), 1, lr, 0.9, 0.999, eps, wd)
    want = p0 - lr * (g / (np.abs(g) + eps) + wd * p0)
    assert np.allclose(p, want, rtol=1e-14, atol=1e-18)
    assert np.allclose(m, 0.1 * g, rtol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-12)


def _constant_gradient_closed_form(step_fn):
    # with a constant gradient from zero state, m^ = g and v^ = g^2 at every
    # step (the bias corrections undo the zero start exactly), so without
    # weight decay each step moves p by lr g / (|g| + eps)
    g = _rand(500, 4, 1e-2)
    p0 = _rand(500, 5, 0.05)
    lr, eps, steps = 5e-4, 1e-8, 25
    p, m, v = p0, np.zeros(500), np.zeros(500)
    for t in range(1, steps + 1):
        p, m, v = step_fn(p, g, m, v, t, lr, 0.9, 0.999, eps, 0.0)
    want = p0 - steps * lr * g / (np.abs(g) + eps)
    return np.max(np.abs(p - want)) / (steps * lr)


def _zero_gradient_closed_form(step_fn):
    # a zero gradient leaves m and v at zero, so only the decoupled decay acts:
    # p_T = p0 (1 - lr wd)^T
    p0 = _rand(500, 6, 0.05)
    lr, wd, steps = 1e-3, 0.05, 30
    p, m, v = p0, np.zeros(500), np.zeros(500)
    for t in range(1, steps + 1):
        p, m, v = step_fn(p, np.zeros(500), m, v, t, lr, 0.9, 0.999, 1e-8, wd)
    return np.max(np.abs(p - p0 * (1 - lr * wd) ** steps)) / np.max(np.abs(p0))


def test_constant_gradient_closed_form():
    assert _constant_gradient_closed_form(oracle.adamw_step) < 1e-12


def test_zero_gradient_is_pure_decoupled_decay():
    assert _zero_gradient_closed_form(oracle.adamw_step) < 1e-13


def _no_bias_correction(p, g, m, v, step, lr, b1, b2, eps, wd):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return p - lr * (m / (np.sqrt(v) + eps) + wd * p), m, v


def _coupled_decay(p, g, m, v, step, lr, b1, b2, eps, wd):
    return oracle.adamw_step(p, g + wd * p, m, v, step, lr, b1, b2, eps, 0.0)


def test_closed_forms_reject_planted_mistakes():
    assert _constant_gradient_closed_form(_no_bias_correction) > 1e-2
    assert _zero_gradient_closed_form(_coupled_decay) > 1e-3


def test_state_is_unchanged_in_place():
    p, g, m, v = _rand(10, 7), _rand(10, 8), np.abs(_rand(10, 9)), np.abs(_rand(10, 10))
    keep = [a.copy() for a in (p, g, m, v)]
    oracle.adamw_step(p, g, m, v, 3, 1e-3)
    for a, b in zip((p, g, m, v), keep):
        assert np.array_equal(a, b)
