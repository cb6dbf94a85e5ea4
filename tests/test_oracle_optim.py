"""Pins of the oracle's AdamW (oracle/optim.py) against things other than
itself: PyTorch's AdamW, closed forms and invariants."""
import numpy as np
import torch

import oracle


def _rand(seed, n=257):
    g = np.random.default_rng(seed)
    return g.standard_normal(n), [g.standard_normal(n) * 10.0 ** g.integers(-4, 1) for _ in range(6)]


def test_matches_torch_adamw_over_several_steps():
    theta0, grads = _rand(0)
    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    p = torch.tensor(theta0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], **hp)
    th, m, v = theta0.copy(), np.zeros_like(theta0), np.zeros_like(theta0)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, m, v = oracle.adamw(th, g, m, v, t, hp["lr"], 0.9, 0.999, 1e-8, hp["weight_decay"])
        np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-12, atol=1e-15)
        st = opt.state[p]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-18)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def test_first_step_closed_form():
    theta0, grads = _rand(1)
    g, lr, eps = grads[0], 2e-5, 1e-8
    th, _, _ = oracle.adamw(theta0, g, np.zeros_like(g), np.zeros_like(g), 1, lr, eps=eps)
    np.testing.assert_allclose(th, theta0 - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)


def test_zero_gradient_is_pure_decay():
    theta0, _ = _rand(2)
    th, m, v = theta0.copy(), np.zeros_like(theta0), np.zeros_like(theta0)
    lr, wd = 1e-2, 0.1
    for t in range(1, 6):
        th, m, v = oracle.adamw(th, np.zeros_like(th), m, v, t, lr, weight_decay=wd)
    np.testing.assert_allclose(th, theta0 * (1 - lr * wd) ** 5, rtol=1e-14)


def test_update_is_invariant_to_gradient_scale_without_eps():
    theta0, grads = _rand(3)
    outs = []
    for c in (1.0, 1e3):
        th, m, v = theta0.copy(), np.zeros_like(theta0), np.zeros_like(theta0)
        for t, g in enumerate(grads, start=1):
            th, m, v = oracle.adamw(th, c * g, m, v, t, 1e-3, eps=0.0)
        outs.append(th)
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-12, atol=1e-15)
