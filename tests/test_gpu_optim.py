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


def test_fused_adamw_equals_the_separate_update():
    """AdamW registered on the context (each layer updated right after its
    backward) gives the same bits as qlx_adamw_lora after each step: losses,
    parameters and both moments over 3 steps, SFT and DPO, streamed (with
    keep-layers) and resident; the update count follows the steps."""
    import dataclasses
    d = dataclasses.replace(synth.TINY, n_layers=3)
    toks = torch.from_numpy(synth.tokens(5, 2, 32, d.vocab)).to(DEV)
    ch, rj = (torch.from_numpy(x).to(DEV) for x in synth.dpo_pairs(5, 2, 32, 8, d.vocab))

    def run(fused, mode, kind):
        m, host = gpu_model(q, d, 5, "normal")
        model = m.with_blobs(host) if mode == B_.QLX_STREAMED else m
        opt = q.AdamW(d, m.lora, lr=1e-3, weight_decay=0.01)
        ctx = q.Context(0)
        ctx.set_keep_layers(True)
        if fused:
            ctx.set_adamw(opt)
        ws = B_.workspace(B_.step_workspace_bytes(d, 0 if kind == "sft" else 1, 2, 32))
        out = []
        for _ in range(3):
            grads = [q.LoraGrads(l) for l in m.lora]
            loss = torch.empty(1, dtype=torch.float32, device=DEV)
            if kind == "sft":
                q.stream_step_sft(ctx, model, toks, mode, loss, grads, ws)
            else:
                lp = torch.empty(8, dtype=torch.float32, device=DEV)
                q.stream_step_dpo(ctx, model, ch, rj, 8, 0.1, mode, B_.QLX_DPO_REF_FUSED, loss, lp, grads, ws)
            if not fused:
                opt.step(grads)
            out.append(loss.clone())
        torch.cuda.synchronize()
        assert opt.t == 3
        ctx.close()
        state = [x for L in (opt.params + opt.m + opt.v) for x in L.A + L.B]
        return out, state

    for kind in ("sft", "dpo"):
        for mode in (B_.QLX_STREAMED, B_.QLX_RESIDENT):
            l0, s0 = run(False, mode, kind)
            l1, s1 = run(True, mode, kind)
            assert all(torch.equal(a, b) for a, b in zip(l0, l1)), (kind, mode)
            assert all(torch.equal(a, b) for a, b in zip(s0, s1)), (kind, mode)


def test_fused_adamw_needs_the_models_adapters():
    d = synth.TINY
    m, host = gpu_model(q, d, 6, "normal")
    other = [q.LoraLayer([a.clone() for a in L.A], [b.clone() for b in L.B]) for L in m.lora]
    ctx = q.Context(0)
    ctx.set_adamw(q.AdamW(d, other))
    with pytest.raises(q.QlxError) as e:
        run_sft(q, m, synth.tokens(6, 1, 32, d.vocab), B_.QLX_RESIDENT, ctx)
    assert e.value.code == B_.QLX_EINVAL and "adapters" in str(e.value)
    ctx.set_adamw(None)
    run_sft(q, m, synth.tokens(6, 1, 32, d.vocab), B_.QLX_RESIDENT, ctx)
    ctx.close()
