"""Pins of the optimizer-step oracle (oracle/adamw.py).

The update rule is a reading (the pages name none), so the pins are facts of
that rule fixed outside the oracle: closed forms of the first step, of a
constant gradient and of pure weight decay, and agreement with PyTorch's CPU
AdamW (an independent implementation of the same rule) over many steps.
"""

import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_first_step_is_lr_times_sign():
    rng = np.random.default_rng(0)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    hp = dict(HP, weight_decay=0.0)
    p1, m1, v1 = oracle.adamw_step(p, g, np.zeros(1000), np.zeros(1000), 1, **hp)
    # m_hat = g and v_hat = g^2 after one step, so the update is lr g / (|g| + eps)
    np.testing.assert_allclose(p - p1, hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-12, atol=0)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12)


def test_constant_gradient_moves_linearly():
    g = np.array([0.5, -2.0, 3e-3])
    p = np.array([1.0, 1.0, 1.0])
    m = np.zeros(3)
    v = np.zeros(3)
    hp = dict(HP, weight_decay=0.0)
    for t in range(1, 51):
        p, m, v = oracle.adamw_step(p, g, m, v, t, **hp)
        # closed forms: m_t = g (1 - b1^t), v_t = g^2 (1 - b2^t)
        np.testing.assert_allclose(m, g * (1 - 0.9 ** t), rtol=1e-12)
        np.testing.assert_allclose(v, g * g * (1 - 0.999 ** t), rtol=1e-10)
    step = hp["lr"] * g / (np.abs(g) + hp["eps"])
    np.testing.assert_allclose(p, 1.0 - 50 * step, rtol=1e-10)


def test_zero_gradient_is_pure_decay():
    p = np.array([2.0, -0.5, 7.0])
    z = np.zeros(3)
    q = p.copy()
    for t in range(1, 11):
        q, m, v = oracle.adamw_step(q, z, z, z, t, **HP)
    np.testing.assert_allclose(q, p * (1 - HP["lr"] * HP["weight_decay"]) ** 10, rtol=1e-13)


def test_agrees_with_torch_adamw_over_many_steps():
    rng = np.random.default_rng(1)
    n = 4096
    p0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0) for _ in range(20)]
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"])
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for step, g in enumerate(grads, start=1):
        t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, step, **HP)
    st = opt.state[t]
    np.testing.assert_allclose(p, t.detach().numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def test_step_counts_from_one():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), 0, **HP)
