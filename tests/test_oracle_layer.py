"""Pins of the oracle's decoder-layer pieces against library routines,
closed forms and fp64 finite differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from helpers import directional_fd, oracle_model, lora_list

torch.set_default_dtype(torch.float64)


def test_rmsnorm_matches_torch_and_unit_rms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3
    g = 1 + 0.1 * rng.standard_normal(33)
    y, _ = oracle.rmsnorm_fwd(x, g, 1e-5)
    ref = F.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    y1, _ = oracle.rmsnorm_fwd(x, np.ones(33), 0.0)
    assert np.allclose(np.sqrt(np.mean(y1 ** 2, -1)), 1.0, rtol=1e-12)


def test_rope_properties():
    rng = np.random.default_rng(1)
    S, hd = 9, 16
    cos, sin = oracle.rope_cos_sin(S, hd, 5e5, np.float64)
    x = rng.standard_normal((2, S, 3, hd))
    y = oracle.rope_fwd(x, cos, sin)
    assert np.array_equal(y[:, 0], x[:, 0])                      # position 0 = identity
    h = hd // 2
    pair = lambda t: t[..., :h] ** 2 + t[..., h:] ** 2
    assert np.allclose(pair(y), pair(x), rtol=1e-12)            # rotations keep pair norms
    # <R_m q, R_n k> depends on m - n only
    q = np.broadcast_to(rng.standard_normal(hd), (1, S, 1, hd)).copy()
    k = np.broadcast_to(rng.standard_normal(hd), (1, S, 1, hd)).copy()
    rq, rk = oracle.rope_fwd(q, cos, sin)[0, :, 0], oracle.rope_fwd(k, cos, sin)[0, :, 0]
    assert np.isclose(rq[5] @ rk[2], rq[3] @ rk[0], rtol=1e-10)
    assert np.isclose(rq[8] @ rk[8], rq[0] @ rk[0], rtol=1e-10)
    # the backward is the transpose of the forward map
    dy = rng.standard_normal(x.shape)
    assert np.isclose(np.sum(oracle.rope_bwd(dy, cos, sin) * x), np.sum(dy * y), rtol=1e-12)


def test_rope_matches_transformers():
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    from transformers import LlamaConfig
    S, hd, nh = 12, 16, 2
    cfg = LlamaConfig(hidden_size=hd * nh, num_attention_heads=nh, head_dim=hd, rope_theta=5e5,
                      max_position_embeddings=64)
    rot = LlamaRotaryEmbedding(cfg)
    x = torch.randn(1, nh, S, hd, generator=torch.Generator().manual_seed(0))
    pos = torch.arange(S)[None]
    c, s = rot(x, pos)
    ref, _ = apply_rotary_pos_emb(x, x, c.double(), s.double())
    cos, sin = oracle.rope_cos_sin(S, hd, 5e5, np.float64)
    ours = oracle.rope_fwd(x.numpy().transpose(0, 2, 1, 3), cos, sin).transpose(0, 2, 1, 3)
    # transformers builds its tables in fp32
    assert np.allclose(ours, ref.numpy(), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("S,nH,nKV", [(1, 4, 2), (7, 4, 2), (13, 6, 3), (16, 2, 2)])
def test_attention_matches_torch_sdpa(S, nH, nKV):
    rng = np.random.default_rng(S)
    hd = 8
    q = rng.standard_normal((2, S, nH, hd))
    k = rng.standard_normal((2, S, nKV, hd))
    v = rng.standard_normal((2, S, nKV, hd))
    o, P = oracle.attention_fwd(q, k, v)
    t = lambda a: torch.from_numpy(a.transpose(0, 2, 1, 3).copy())
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, enable_gqa=True)
    assert np.allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)
    # first query attends to key 0 only
    group = nH // nKV
    for h in range(nH):
        assert np.allclose(o[:, 0, h], v[:, 0, h // group])
    assert np.allclose(P.sum(-1), 1.0)


def test_attention_uniform_scores_give_prefix_means():
    rng = np.random.default_rng(3)
    S, hd = 6, 4
    q = np.zeros((1, S, 2, hd))
    k = rng.standard_normal((1, S, 1, hd))
    v = rng.standard_normal((1, S, 1, hd))
    o, _ = oracle.attention_fwd(q, k, v)
    means = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
    assert np.allclose(o[0, :, 0], means) and np.allclose(o[0, :, 1], means)


def test_swiglu_matches_torch():
    rng = np.random.default_rng(4)
    g, u = rng.standard_normal((5, 9)) * 4, rng.standard_normal((5, 9))
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.allclose(oracle.swiglu_fwd(g, u), ref, rtol=1e-13)


def test_lora_zero_B_or_A_is_base_and_merged_weight_identity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 12)).astype(np.float32)
    W = rng.standard_normal((10, 12)).astype(np.float32)
    A = rng.standard_normal((3, 12)).astype(np.float32)
    B = rng.standard_normal((10, 3)).astype(np.float32)
    base, _ = oracle.qlora_linear_fwd(x, W, None, None, 2.0)
    y0, _ = oracle.qlora_linear_fwd(x, W, A, np.zeros_like(B), 2.0)
    y1, _ = oracle.qlora_linear_fwd(x, W, np.zeros_like(A), B, 2.0)
    assert np.array_equal(y0, base) and np.array_equal(y1, base)
    y, _ = oracle.qlora_linear_fwd(x.astype(np.float64), W.astype(np.float64), A.astype(np.float64),
                                   B.astype(np.float64), 2.0)
    merged = x.astype(np.float64) @ (W + 2.0 * B.astype(np.float64) @ A).T
    assert np.allclose(y, merged, rtol=1e-12)


def test_qlora_linear_backward_finite_differences():
    rng = np.random.default_rng(6)
    x, W = rng.standard_normal((5, 7)), rng.standard_normal((6, 7))
    A, B = rng.standard_normal((3, 7)), rng.standard_normal((6, 3))
    R = rng.standard_normal((5, 6))
    s = 0.75
    f = lambda: float(np.sum(oracle.qlora_linear_fwd(x, W, A, B, s)[0] * R))
    _, u = oracle.qlora_linear_fwd(x, W, A, B, s)
    dx, dA, dB = oracle.qlora_linear_bwd(R, x, u, W, A, B, s)
    for arr, g in ((x, dx), (A, dA), (B, dB)):
        v = rng.standard_normal(arr.shape)
        assert np.isclose(directional_fd(f, arr, v, 1e-6), np.sum(g * v), rtol=1e-7)


@pytest.mark.parametrize("random_gamma", [False, True])
def test_layer_backward_finite_differences(random_gamma):
    d = synth.MICRO
    B, S = 2, 5
    m = oracle_model(d, 11, std=0.3, random_gamma=random_gamma)
    lay = m["layers"][0]
    W = {p: w.astype(np.float64) for p, w in oracle.dequant_layer(lay["nf4"], d).items()}
    lora = {p: (a.astype(np.float64), b.astype(np.float64))
            for p, (a, b) in synth.lora_params(d, 11, 0, "normal").items()}
    for p in lora:  # make the adapters matter at this scale
        lora[p] = (lora[p][0] * 30, lora[p][1] * 30)
    rng = np.random.default_rng(7)
    h = rng.standard_normal((B * S, d.hidden))
    R = rng.standard_normal((B * S, d.hidden))
    g1, g2 = lay["g1"].astype(np.float64), lay["g2"].astype(np.float64)
    f = lambda: float(np.sum(oracle.layer_fwd(h, W, g1, g2, lora, d, B, S) * R))
    _, cache = oracle.layer_fwd(h, W, g1, g2, lora, d, B, S, keep=True)
    dh, grads = oracle.layer_bwd(R, W, g1, g2, lora, d, B, S, cache)
    v = rng.standard_normal(h.shape)
    assert np.isclose(directional_fd(f, h, v, 1e-6), np.sum(dh * v), rtol=1e-6)
    for p in lora:
        for j in range(2):
            arr, g = lora[p][j], grads[p][j]
            v = rng.standard_normal(arr.shape)
            assert np.isclose(directional_fd(f, arr, v, 1e-6), np.sum(g * v), rtol=1e-6, atol=1e-10), (p, j)
