"""Pins of the oracle's ORPO, SimPO and KTO (oracle/preference.py and
pref_step): closed forms, finite differences of dL/ds, ORPO's NLL term
against a direct log-softmax, and the whole step's LoRA gradients against
fp64 finite differences."""
import numpy as np
import pytest

import oracle
import synth
from helpers import directional_fd, lora_list, oracle_model
from synth import PROJ_NAMES


def _fd_grad(fun, x, eps=1e-6):
    x = np.array(x, np.float64)
    g = np.zeros_like(x)
    for i in range(x.size):
        e = np.zeros_like(x)
        e[i] = eps
        g[i] = (fun(x + e) - fun(x - e)) / (2 * eps)
    return g


LP = np.array([-380.0, -410.0, -395.0, -402.5])   # two pairs of 384-token responses
N = 384


def test_orpo_closed_form_and_gradient():
    loss, g = oracle.orpo_loss(np.array([-400.0, -400.0]), N, lam=0.1)
    assert loss == pytest.approx(400.0 / N + 0.1 * np.log(2.0), rel=1e-14)   # odds term ln 2 at chosen == rejected
    # log odds directly: l = s/n, odds = P / (1 - P), P = exp(l)
    l = LP / N
    odds = np.exp(l) / (1 - np.exp(l))
    z = np.log(odds[:2]) - np.log(odds[2:])
    want = np.mean(-l[:2] + 0.1 * np.log1p(np.exp(-z)))
    loss, g = oracle.orpo_loss(LP, N, lam=0.1)
    assert loss == pytest.approx(want, rel=1e-12)
    np.testing.assert_allclose(g, _fd_grad(lambda x: oracle.orpo_loss(x, N, 0.1)[0], LP), rtol=1e-6, atol=1e-12)


def test_orpo_log_odds_near_certainty_is_stable():
    # l close to 0 (P -> 1): log(1 - e^l) must not lose the answer
    loss, g = oracle.orpo_loss(np.array([-1e-3 * N, -2.0 * N]), N)
    assert np.isfinite(loss) and np.all(np.isfinite(g))
    l = -1e-3
    assert oracle.preference._log1mexp(l) == pytest.approx(np.log(1 - np.exp(l)), rel=1e-9)


def test_simpo_closed_form_and_gradient():
    loss, _ = oracle.simpo_loss(np.array([-400.0, -400.0]), N, beta=2.0, gamma=0.5)
    assert loss == pytest.approx(np.log1p(np.exp(0.5)), rel=1e-14)
    loss, g = oracle.simpo_loss(LP, N, beta=2.0, gamma=0.5)
    u = 2.0 * (LP[:2] / N - LP[2:] / N) - 0.5
    assert loss == pytest.approx(np.mean(np.log1p(np.exp(-u))), rel=1e-12)
    np.testing.assert_allclose(g, _fd_grad(lambda x: oracle.simpo_loss(x, N, 2.0, 0.5)[0], LP), rtol=1e-6,
                               atol=1e-12)


def test_kto_closed_forms_and_gradient():
    loss, g = oracle.kto_loss(LP, LP, 0.0, beta=0.1, lam_d=1.0, lam_u=1.0)
    assert loss == 0.5 and np.allclose(g, [-0.1 / 16, -0.1 / 16, 0.1 / 16, 0.1 / 16])
    loss, _ = oracle.kto_loss(LP, LP, 0.0, beta=0.1, lam_d=2.0, lam_u=1.0)
    assert loss == pytest.approx((2 * 1.0 + 2 * 0.5) / 4)          # (sum of lambda_y / 2) / B
    ref = LP + np.array([1.0, -2.0, 0.5, 3.0])
    loss, g = oracle.kto_loss(LP, ref, 0.7, beta=0.1)
    np.testing.assert_allclose(g, _fd_grad(lambda x: oracle.kto_loss(x, ref, 0.7, 0.1)[0], LP), rtol=1e-6,
                               atol=1e-12)
    assert oracle.kto_z0([1.0, 2.0], [3.0, 3.0]) == 0.0 and oracle.kto_z0([4.0, 2.0], [1.0, 1.0]) == 2.0


def test_kl_tokens_shift_completions_by_one():
    t = np.arange(4 * 5).reshape(4, 5)
    k = oracle.kl_tokens(t, 2)
    assert np.array_equal(k[:, :2], t[:, :2]) and np.array_equal(k[:, 2:], np.roll(t[:, 2:], -1, axis=0))


def test_orpo_nll_term_is_the_chosen_response_cross_entropy():
    d = synth.MICRO
    model = oracle_model(d, 20, std=0.3, head_std_scale=20.0)
    lora = lora_list(d, 20, "normal")
    ch, rj = synth.dpo_pairs(20, 2, 9, 4, d.vocab)
    _, logps, _ = oracle.pref_step("orpo", model, lora, ch, rj, 4, d, dtype=np.float64, lam=0.0)
    # with lambda = 0 the loss is the mean per-token NLL of the chosen responses
    hL = oracle.model_forward(model, lora, ch, d, np.float64)
    z = oracle.model.head_logits(hL, model["gf"], oracle.model._f16(model["head"]).astype(np.float64), d.rms_eps)[0]
    z = z.reshape(2, 9, -1)[:, 3:8, :]
    logp = z - np.log(np.sum(np.exp(z - z.max(-1, keepdims=True)), -1, keepdims=True)) - z.max(-1, keepdims=True)
    nll = -np.mean(np.take_along_axis(logp, ch[:, 4:, None].astype(np.int64), -1))
    loss, _, _ = oracle.pref_step("orpo", model, lora, ch, rj, 4, d, dtype=np.float64, lam=0.0)
    assert loss == pytest.approx(nll, rel=1e-12)
    assert np.allclose(logps[4:], 0.0)   # no reference pass: the 2P reference entries are 0


@pytest.mark.parametrize("kind,hp", [("orpo", dict(lam=0.5)), ("simpo", dict(beta=2.0, gamma=0.5)),
                                     ("kto", dict(beta=0.5))])
def test_pref_step_finite_differences(kind, hp):
    d = synth.MICRO
    model = oracle_model(d, 14, std=0.3, head_std_scale=20.0)
    lora = [{p: (a.astype(np.float64) * 30, b.astype(np.float64) * 30) for p, (a, b) in l.items()}
            for l in lora_list(d, 14, "normal")]
    ch, rj = synth.dpo_pairs(14, 2, 7, 3, d.vocab)
    loss, _, grads = oracle.pref_step(kind, model, lora, ch, rj, 3, d, dtype=np.float64, **hp)
    z0 = None
    if kind == "kto":   # z0 carries no gradient: hold it at its value for the differences
        kt = oracle.kl_tokens(np.concatenate([ch, rj]), 3)
        kp = oracle.seq_logprobs(oracle.model_forward(model, lora, kt, d, np.float64), model["gf"], model["head"],
                                 kt, 3, d.rms_eps)
        kr = oracle.seq_logprobs(oracle.model_forward(model, None, kt, d, np.float64), model["gf"], model["head"],
                                 kt, 3, d.rms_eps)
        z0 = oracle.kto_z0(kp, kr)
    f = lambda: oracle.pref_step(kind, model, lora, ch, rj, 3, d, dtype=np.float64, z0_override=z0, **hp)[0]
    rng = np.random.default_rng(15)
    for i in range(d.n_layers):
        for p in ("q", "o", "up"):
            for j in range(2):
                arr = lora[i][p][j]
                v = rng.standard_normal(arr.shape)
                fd = directional_fd(f, arr, v, 1e-6)
                assert np.isclose(fd, np.sum(grads[i][p][j] * v), rtol=1e-6, atol=1e-11), (kind, i, p, j)


def test_kto_is_half_when_policy_equals_reference():
    d = synth.MICRO
    model = oracle_model(d, 16, std=0.3)
    ch, rj = synth.dpo_pairs(16, 2, 9, 4, d.vocab)
    loss, logps, _ = oracle.pref_step("kto", model, lora_list(d, 16, "zeroB"), ch, rj, 4, d, dtype=np.float64)
    assert loss == 0.5 and np.array_equal(logps[:4], logps[4:])
