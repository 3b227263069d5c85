"""Pins of the oracle's AdamW step and gradient clipping."""

import numpy as np
import pytest
import torch

from oracle.optim import (BETA1, BETA2, EPS, adamw_multi, adamw_step, clip_coefficient,
                          global_grad_norm)


def _rand(seed, n, scale=1.0):
    return np.random.default_rng(seed).standard_normal(n) * scale


@pytest.mark.parametrize("wd,max_norm", [(0.0, 0.0), (0.001, 0.0), (0.001, 0.3), (0.05, 5.0)])
def test_matches_torch_adamw_over_steps(wd, max_norm):
    """Several steps of the oracle against torch.optim.AdamW (float64, CPU),
    with clipping by torch.nn.utils.clip_grad_norm_."""
    lr = 2e-4
    shapes = [(64, 48), (33,), (7, 5)]
    ps = [_rand(i, int(np.prod(s)), 0.02).reshape(s) for i, s in enumerate(shapes)]
    tp = [torch.tensor(p, dtype=torch.float64, requires_grad=True) for p in ps]
    opt = torch.optim.AdamW(tp, lr=lr, betas=(BETA1, BETA2), eps=EPS, weight_decay=wd)
    ms = [np.zeros_like(p) for p in ps]
    vs = [np.zeros_like(p) for p in ps]
    for step in range(1, 6):
        gs = [_rand(100 * step + i, p.size, 0.5 + i).reshape(p.shape) for i, p in enumerate(ps)]
        for t, g in zip(tp, gs):
            t.grad = torch.tensor(g, dtype=torch.float64)
        if max_norm > 0:
            tn = torch.nn.utils.clip_grad_norm_(tp, max_norm)
        opt.step()
        ps, ms, vs, norm = adamw_multi(ps, gs, ms, vs, step, lr, weight_decay=wd,
                                       max_grad_norm=max_norm)
        if max_norm > 0:
            assert abs(norm - float(tn)) <= 1e-12 * float(tn)
        for p, t in zip(ps, tp):
            np.testing.assert_allclose(p, t.detach().numpy(), rtol=1e-13, atol=1e-16)


def test_first_step_from_zero_moments():
    """m_hat = g and v_hat = g^2 after one step: each weight moves by lr*g/(|g|+eps)."""
    g = np.array([3.0, -2.0, 1e-3, -7.5, 1e-9])
    p0 = np.array([0.5, -0.25, 0.0, 1.0, 2.0])
    lr = 1e-3
    p, m, v = adamw_step(p0, g, np.zeros(5), np.zeros(5), 1, lr)
    np.testing.assert_allclose(p, p0 - lr * g / (np.abs(g) + EPS), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, (1 - BETA1) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - BETA2) * g * g, rtol=1e-15)


def test_constant_gradient_moves_at_constant_speed():
    """With a constant gradient the bias corrections cancel exactly: every step
    moves p by lr*g/(|g|+eps), so p_t = p_0 - t*lr*g/(|g|+eps)."""
    g = np.array([0.7, -1.3, 4.0])
    p0 = np.array([0.1, 0.2, -0.3])
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    lr = 2e-4
    for t in range(1, 51):
        p, m, v = adamw_step(p, g, m, v, t, lr)
        np.testing.assert_allclose(p, p0 - t * lr * g / (np.abs(g) + EPS), rtol=1e-12)


def test_zero_gradient_only_decays():
    p0 = np.array([1.0, -0.5, 0.25])
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    lr, wd = 2e-4, 0.001
    for t in range(1, 11):
        p, m, v = adamw_step(p, np.zeros(3), m, v, t, lr, weight_decay=wd)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) ** 10, rtol=1e-14)
    assert not m.any() and not v.any()


def test_update_is_scale_invariant_without_eps():
    g = _rand(3, 20)
    p0 = _rand(4, 20, 0.1)
    a = adamw_step(p0, g, np.zeros(20), np.zeros(20), 1, 1e-3, eps=0.0)[0]
    b = adamw_step(p0, 1000.0 * g, np.zeros(20), np.zeros(20), 1, 1e-3, eps=0.0)[0]
    np.testing.assert_allclose(a, b, rtol=1e-14)


def test_clip_coefficient():
    gs = [np.array([3.0, 4.0]), np.array([12.0])]
    assert global_grad_norm(gs) == 13.0
    assert clip_coefficient(13.0, 0.3) == pytest.approx(0.3 / (13.0 + 1e-6), rel=1e-15)
    assert clip_coefficient(0.1, 0.3) == 1.0
    assert clip_coefficient(13.0, 0.0) == 1.0
    # against the library routine
    t = [torch.tensor(g, dtype=torch.float64) for g in gs]
    for x in t:
        x.grad = x.clone()
    n = torch.nn.utils.clip_grad_norm_(t, 0.3)
    assert float(n) == 13.0
    np.testing.assert_allclose(t[0].grad.numpy(), gs[0] * clip_coefficient(13.0, 0.3), rtol=1e-15)
