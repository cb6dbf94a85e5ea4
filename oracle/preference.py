"""Preference objectives on the layer stream besides DPO: ORPO, SimPO, KTO.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the tool's v0.72.4 runs DPO, ORPO, SimPO and KTO through the same
layer stream (rug.gal article, intro and "En detalle"; imasters article, "Do
SFT para os métodos de preferência"); KTO, though often called
reference-free, uses the same reference scheme as DPO, the adapters switched
off (rug.gal article, "En detalle"). The objectives themselves are the
published ones; every loss here is a function of per-sequence summed
response log-probs s (and their length n), so the training step is the DPO
step with another dL/ds.

Readings (the pages give no hyperparameters for these):
  * ORPO (Hong, Lee & Thorne 2024, eqs. 2-7): L = mean over pairs of
    [ -s_c/n_c  +  lambda * -log sigmoid(log odds_c - log odds_r) ], with
    the length-normalized likelihood l = s/n, P = exp(l) and
    log odds = l - log(1 - exp(l)); lambda = 0.1. No reference model.
  * SimPO (Meng, Xia & Chen 2024, eq. 6): L = mean over pairs of
    -log sigmoid(beta * (s_c/n_c - s_r/n_r) - gamma); beta 2.0, gamma 0.5.
    No reference model.
  * KTO (Ethayarajh et al. 2024, eq. 8): chosen sequences are desirable,
    rejected undesirable; r = s_pol - s_ref; z0 = max(0, mean over the
    batch's mismatched pairs of s_pol - s_ref), with no gradient through
    z0; the mismatched pair of example j is its prompt followed by the
    completion of example (j + 1) mod B (completions shifted by one within
    the batch); v = lambda_D sigmoid(beta (r - z0)) for desirable and
    lambda_U sigmoid(beta (z0 - r)) for undesirable; L = mean over examples
    of lambda_y - v; beta 0.1, lambda_D = lambda_U = 1.

Each loss returns (loss, dL/ds) with dL/ds laid out like s:
[chosen_1..chosen_P, rejected_1..rejected_P].

Parity pins (tests/test_oracle_preference.py): closed forms at chosen ==
rejected (ORPO odds term ln 2; SimPO log(1 + e^gamma)) and at policy ==
reference (KTO: (lambda_D + lambda_U)/4); central finite differences of
every dL/ds; ORPO's NLL term against the log-softmax of the logits; the
whole step's LoRA gradients against fp64 finite differences.
"""
from __future__ import annotations

import numpy as np


def _log_sigmoid(x):
    return -np.logaddexp(0.0, -x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _log1mexp(l):
    """log(1 - exp(l)) for l < 0, accurate at both ends."""
    l = np.asarray(l, np.float64)
    return np.where(l > -np.log(2.0), np.log(-np.expm1(l)), np.log1p(-np.exp(l)))


def orpo_loss(lp, n, lam=0.1):
    lp = np.asarray(lp, np.float64)
    P = lp.size // 2
    l = lp / n
    lc, lr = l[:P], l[P:]
    z = (lc - _log1mexp(lc)) - (lr - _log1mexp(lr))
    loss = float(np.mean(-lc + lam * -_log_sigmoid(z)))
    s = _sigmoid(-z)                       # -d(-log sigmoid z)/dz
    d_lc = -1.0 - lam * s / (1.0 - np.exp(lc))
    d_lr = lam * s / (1.0 - np.exp(lr))
    return loss, np.concatenate([d_lc, d_lr]) / (P * n)


def simpo_loss(lp, n, beta=2.0, gamma=0.5):
    lp = np.asarray(lp, np.float64)
    P = lp.size // 2
    u = beta * (lp[:P] / n - lp[P:] / n) - gamma
    loss = float(np.mean(-_log_sigmoid(u)))
    g = -_sigmoid(-u) * beta / (P * n)
    return loss, np.concatenate([g, -g])


def kto_loss(lp_pol, lp_ref, z0, beta=0.1, lam_d=1.0, lam_u=1.0):
    """z0 is a given number (no gradient flows through it)."""
    lp_pol = np.asarray(lp_pol, np.float64)
    lp_ref = np.asarray(lp_ref, np.float64)
    B = lp_pol.size
    P = B // 2
    r = lp_pol - lp_ref
    xd = beta * (r[:P] - z0)
    xu = beta * (z0 - r[P:])
    loss = float((np.sum(lam_d - lam_d * _sigmoid(xd)) + np.sum(lam_u - lam_u * _sigmoid(xu))) / B)
    gd = -lam_d * beta * _sigmoid(xd) * _sigmoid(-xd) / B
    gu = lam_u * beta * _sigmoid(xu) * _sigmoid(-xu) / B
    return loss, np.concatenate([gd, gu])


def kto_z0(lp_pol_kl, lp_ref_kl):
    return float(max(0.0, np.mean(np.asarray(lp_pol_kl, np.float64) - np.asarray(lp_ref_kl, np.float64))))


def kl_tokens(toks, prompt_len):
    """Mismatched pairs: prompt of example j + completion of example (j+1) mod B."""
    toks = np.asarray(toks)
    out = toks.copy()
    out[:, prompt_len:] = np.roll(toks[:, prompt_len:], -1, axis=0)
    return out
