"""The optimizer update of a training step, the oracle's version: AdamW on
the LoRA factors.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the example configuration sets the learning rate, 2e-5, and nothing
else about the optimizer (guillermodelpino.com article, "Qué es Soup", the
`training` block). Reading: AdamW, i.e. Adam's bias-corrected moment
estimates (Kingma & Ba, "Adam", Algorithm 1) with decoupled weight decay
(Loshchilov & Hutter, "Decoupled Weight Decay Regularization", Algorithm 2),
the decay multiplied by the learning rate as in PyTorch's AdamW; defaults
beta1 0.9, beta2 0.999, eps 1e-8, weight decay 0 (no schedule: the pages give
none).

Written in the algorithm's own notation, float64:
    theta_t = theta_{t-1} (1 - lr * lambda)
    m_t = beta1 m_{t-1} + (1 - beta1) g_t
    v_t = beta2 v_{t-1} + (1 - beta2) g_t^2
    m_hat = m_t / (1 - beta1^t),  v_hat = v_t / (1 - beta2^t)
    theta_t = theta_t - lr * m_hat / (sqrt(v_hat) + eps)

Parity pins (tests/test_oracle_optim.py): PyTorch's torch.optim.AdamW on the
same float64 tensors (a library routine), the closed-form first step
theta_1 = theta_0 - lr g / (|g| + eps), pure decay theta_t = theta_0 (1 - lr
lambda)^t when every gradient is zero, and invariance of the update to a
positive rescaling of the gradients when eps = 0.
"""
from __future__ import annotations

import numpy as np


def adamw(theta, g, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """One AdamW update of one tensor; t is the 1-based update count.
    Returns (theta, m, v) as new float64 arrays."""
    theta = np.asarray(theta, np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v


def adamw_lora(lora, grads, m, v, t, lr, **hp):
    """AdamW on a model's LoRA factors. lora, grads, m, v: lists (one per
    layer) of {projection: (A, B)}; returns the new (lora, m, v) lists."""
    out_l, out_m, out_v = [], [], []
    for L, G, M, V in zip(lora, grads, m, v):
        nl, nm, nv = {}, {}, {}
        for p in L:
            a = adamw(L[p][0], G[p][0], M[p][0], V[p][0], t, lr, **hp)
            b = adamw(L[p][1], G[p][1], M[p][1], V[p][1], t, lr, **hp)
            nl[p], nm[p], nv[p] = (a[0], b[0]), (a[1], b[1]), (a[2], b[2])
        out_l.append(nl)
        out_m.append(nm)
        out_v.append(nv)
    return out_l, out_m, out_v
