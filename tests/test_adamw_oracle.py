"""Pins of the fp64 AdamW oracle (CPU only): closed forms and an independent
library implementation of the same update."""

import numpy as np
import pytest
import torch

import oracle

H = oracle.ADAMW_DEFAULTS


def test_first_step_closed_form():
    # t = 1 from zero state: m_hat = g, v_hat = g^2, so the step is -lr g / (|g| + eps)
    rng = np.random.default_rng(0)
    p, g = rng.standard_normal(1000), rng.standard_normal(1000) * 1e-3
    p1, m1, v1 = oracle.adamw_step(p, g, np.zeros(1000), np.zeros(1000), 1, **H)
    lr, wd, eps = H["lr"], H["weight_decay"], H["eps"]
    expect = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.allclose(p1, expect, rtol=0, atol=1e-15)
    assert np.allclose(m1, (1 - H["beta1"]) * g, rtol=1e-15, atol=0)
    assert np.allclose(v1, (1 - H["beta2"]) * g * g, rtol=1e-15, atol=0)


@pytest.mark.parametrize("t", [1, 2, 7, 100])
def test_constant_gradient_closed_form(t):
    # a constant g from zero state gives m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2,
    # so every step moves p by exactly -lr g / (|g| + eps) after the decay
    g = np.array([3e-4, -2.0, 0.5, -1e-6])
    p = np.array([0.1, -0.2, 0.3, 0.0])
    m = v = np.zeros(4)
    ref = p.copy()
    lr, wd, eps = H["lr"], H["weight_decay"], H["eps"]
    for s in range(1, t + 1):
        p, m, v = oracle.adamw_step(p, g, m, v, s, **H)
        ref = ref * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.allclose(m, (1 - H["beta1"] ** t) * g, rtol=1e-13, atol=0)
    assert np.allclose(v, (1 - H["beta2"] ** t) * g * g, rtol=1e-12, atol=0)
    assert np.allclose(p, ref, rtol=1e-12, atol=1e-18)


def test_zero_gradient_is_decay_only():
    p = np.linspace(-1, 1, 11)
    p1, m1, v1 = oracle.adamw_step(p, np.zeros(11), np.zeros(11), np.zeros(11), 3, **H)
    assert np.array_equal(m1, np.zeros(11)) and np.array_equal(v1, np.zeros(11))
    assert np.allclose(p1, p * (1 - H["lr"] * H["weight_decay"]), rtol=1e-15, atol=0)


def test_matches_torch_adamw_float64():
    # torch.optim.AdamW on the CPU in float64: the same update from another implementation
    rng = np.random.default_rng(1)
    shape = (37, 19)
    p0 = rng.standard_normal(shape)
    grads = [rng.standard_normal(shape) * 10.0 ** rng.integers(-4, 1) for _ in range(6)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=H["lr"], betas=(H["beta1"], H["beta2"]), eps=H["eps"],
                            weight_decay=H["weight_decay"])
    p, m, v = p0.copy(), np.zeros(shape), np.zeros(shape)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, t, **H)
    st = opt.state[tp]
    assert np.allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-16)
    assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=0)
    assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=0)


def test_step_must_count_from_one():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), 0)
