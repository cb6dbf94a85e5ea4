"""GPU parity of the AdamW update (qlx_adamw_lora) against the oracle, and a
short training loop (streamed SFT step + AdamW) against the oracle's loop."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, f32_dev, gpu_model, oracle_lora, run_sft, to_np
from helpers import lora_list, oracle_model, rel_l2
from synth import PROJ_NAMES

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")
B_ = q.binding


def _rand_like_lora(d, seed, scale, positive=False):
    g = np.random.default_rng(seed)
    out = []
    for l in range(d.n_layers):
        lp = synth.lora_params(d, 0, l, "normal")
        layer = {}
        for p in PROJ_NAMES:
            pair = []
            for t in lp[p]:
                x = g.standard_normal(t.shape) * scale
                # fp32 values: the oracle gets exactly what the GPU gets
                pair.append((np.abs(x) if positive else x).astype(np.float32).astype(np.float64))
            layer[p] = tuple(pair)
        out.append(layer)
    return out


def _to_layers(lst):
    return [q.LoraLayer([f32_dev(L[p][0]) for p in PROJ_NAMES], [f32_dev(L[p][1]) for p in PROJ_NAMES]) for L in lst]


@pytest.mark.parametrize("t,wd", [(1, 0.0), (3, 0.01), (1000, 0.1)])
def test_adamw_update_vs_oracle(t, wd):
    d = synth.TINY
    th, g, m = (_rand_like_lora(d, s, sc) for s, sc in ((1, 0.02), (2, 1e-3), (3, 1e-4)))
    v = _rand_like_lora(d, 4, 1e-7, positive=True)
    P, M, V = _to_layers(th), _to_layers(m), _to_layers(v)
    G = []
    for L in g:
        gg = q.LoraGrads(_to_layers([L])[0])
        for i, p in enumerate(PROJ_NAMES):
            gg.dA[i].copy_(f32_dev(L[p][0]))
            gg.dB[i].copy_(f32_dev(L[p][1]))
        G.append(gg)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    B_.adamw_lora(d, P, G, M, V, t, **hp)
    torch.cuda.synchronize()
    rl, rm, rv = oracle.adamw_lora(th, g, m, v, t, **hp)
    for l in range(d.n_layers):
        for i, p in enumerate(PROJ_NAMES):
            for j, (gpu, ref) in enumerate(((P[l].A[i], rl[l][p][0]), (P[l].B[i], rl[l][p][1]))):
                x = to_np(gpu).astype(np.float64)
                assert np.all(np.abs(x - ref) <= 1e-6 * (1 + np.abs(ref))), (l, p, j)
            for j in (0, 1):
                # m = b1 m0 + (1 - b1) g can cancel: bound its fp32 error by the terms forming it
                scale_m = 0.9 * np.abs(m[l][p][j]) + 0.1 * np.abs(g[l][p][j])
                x = to_np((M[l].A, M[l].B)[j][i]).astype(np.float64)
                assert np.all(np.abs(x - rm[l][p][j]) <= 1e-6 * scale_m + 1e-30), (l, p, j, "m")
                x = to_np((V[l].A, V[l].B)[j][i]).astype(np.float64)  # v: positive terms only
                rel = np.abs(x - rv[l][p][j]) / (np.abs(rv[l][p][j]) + 1e-30)
                k = np.unravel_index(np.argmax(rel), rel.shape)
                assert rel[k] <= 1e-6, (f"v {l} {p} {j} at {k}: rel {rel[k]:.3e} gpu {x[k]:.9e} "
                                        f"oracle {rv[l][p][j][k]:.9e} v0 {v[l][p][j][k]:.9e} g {g[l][p][j][k]:.9e}")


def test_adamw_rejects_bad_arguments():
    d = synth.TINY
    P = _to_layers(_rand_like_lora(d, 1, 0.02))
    G = [q.LoraGrads(x) for x in P]
    M, V = _to_layers(_rand_like_lora(d, 3, 0.0)), _to_layers(_rand_like_lora(d, 4, 0.0))
    with pytest.raises(q.QlxError) as e:
        B_.adamw_lora(d, P, G, M, V, 0, lr=1e-3)             # t must be >= 1
    assert e.value.code == B_.QLX_EINVAL
    with pytest.raises(q.QlxError) as e:
        B_.adamw_lora(d, P, G, M, V, 1, lr=1e-3, beta1=1.0)  # beta in [0, 1)
    assert e.value.code == B_.QLX_EINVAL


def _gpu_loop(d, seed, toks, mode, steps, lr):
    m, host = gpu_model(q, d, seed, "normal")
    model = m.with_blobs(host) if mode == B_.QLX_STREAMED else m
    opt = q.AdamW(d, m.lora, lr=lr)
    ctx = q.Context(0)
    losses = []
    for _ in range(steps):
        loss, grads, _ = run_sft(q, model, toks, mode, ctx)
        opt.step(grads)
        losses.append(loss)
    torch.cuda.synchronize()
    return [x.item() for x in losses], losses, m.lora


def test_training_loop_vs_oracle_and_streamed_equals_resident():
    """3 steps at the pages' lr 2e-5. Adam's first updates are ~lr * sign(g),
    so elements whose gradient is within the 1e-2 gradient tolerance of zero
    may move the other way: params are compared at rel-L2 2e-3 (the whole
    update is ~6e-3 of |theta| here), losses at 1e-2 like a single step."""
    d, seed, steps, lr = synth.TINY, 0, 3, 2e-5
    toks = synth.tokens(seed, 1, 64, d.vocab)
    l_s, t_s, lora_s = _gpu_loop(d, seed, toks, B_.QLX_STREAMED, steps, lr)
    l_r, t_r, lora_r = _gpu_loop(d, seed, toks, B_.QLX_RESIDENT, steps, lr)
    assert all(torch.equal(a, b) for a, b in zip(t_s, t_r))
    assert all(torch.equal(x, y) for a, b in zip(lora_s, lora_r) for x, y in zip(a.A + a.B, b.A + b.B))
    model = oracle_model(d, seed)
    lora = lora_list(d, seed, "normal")
    mo = [{p: (np.zeros_like(L[p][0]), np.zeros_like(L[p][1])) for p in L} for L in lora]
    vo = [{p: (np.zeros_like(L[p][0]), np.zeros_like(L[p][1])) for p in L} for L in lora]
    for t in range(1, steps + 1):
        loss, grads = oracle.sft_step(model, lora, toks, d)
        assert abs(l_s[t - 1] - loss) < 1e-2, (t, l_s[t - 1], loss)
        lora, mo, vo = oracle.adamw_lora(lora, grads, mo, vo, t, lr)
    for l in range(d.n_layers):
        got = oracle_lora(lora_s[l])
        for p in PROJ_NAMES:
            for j in (0, 1):
                assert rel_l2(got[p][j], lora[l][p][j]) < 2e-3, (l, p, j)


def test_training_lowers_the_loss_on_a_fixed_batch():
    d = synth.TINY
    toks = synth.tokens(7, 2, 64, d.vocab)
    losses, _, _ = _gpu_loop(d, 7, toks, B_.QLX_STREAMED, 8, 1e-2)
    assert losses[-1] < losses[0] - 0.05, losses
    assert all(np.isfinite(losses))
