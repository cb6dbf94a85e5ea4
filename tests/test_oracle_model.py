"""Pins of the oracle's whole training step (SFT and DPO): transformers'
Llama in fp64 as an independent implementation, closed forms (ln V, ln 2),
and fp64 finite differences."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import directional_fd, lora_list, oracle_model
from synth import PROJ_NAMES

_HF = {"q": ("self_attn", "q_proj"), "k": ("self_attn", "k_proj"), "v": ("self_attn", "v_proj"),
       "o": ("self_attn", "o_proj"), "gate": ("mlp", "gate_proj"), "up": ("mlp", "up_proj"),
       "down": ("mlp", "down_proj")}


def _hf_model(d, model, lora):
    """transformers LlamaForCausalLM (fp64, eager attention) holding the
    dequantized base with each LoRA merged into its weight."""
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(hidden_size=d.hidden, intermediate_size=d.inter, num_attention_heads=d.n_heads,
                      num_key_value_heads=d.n_kv_heads, head_dim=d.head_dim, vocab_size=d.vocab,
                      num_hidden_layers=d.n_layers, rms_norm_eps=d.rms_eps, rope_theta=d.rope_theta,
                      tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                      max_position_embeddings=4096, attn_implementation="eager")
    hf = LlamaForCausalLM(cfg).double()
    s = d.lora_scale
    with torch.no_grad():
        hf.model.embed_tokens.weight.copy_(torch.from_numpy(synth.f16_bits_to_f32(model["embed"]).astype(np.float64)))
        hf.lm_head.weight.copy_(torch.from_numpy(synth.f16_bits_to_f32(model["head"]).astype(np.float64)))
        hf.model.norm.weight.copy_(torch.from_numpy(model["gf"].astype(np.float64)))
        for i, lay in enumerate(model["layers"]):
            W = oracle.dequant_layer(lay["nf4"], d)
            L = hf.model.layers[i]
            L.input_layernorm.weight.copy_(torch.from_numpy(lay["g1"].astype(np.float64)))
            L.post_attention_layernorm.weight.copy_(torch.from_numpy(lay["g2"].astype(np.float64)))
            for p in PROJ_NAMES:
                w = W[p].astype(np.float64)
                if lora is not None:
                    A, B = lora[i][p]
                    w = w + s * B.astype(np.float64) @ A.astype(np.float64)
                getattr(getattr(L, _HF[p][0]), _HF[p][1]).weight.copy_(torch.from_numpy(w))
    return hf


def _hf_lora_grads(d, hf, lora):
    """dL/dA = s B^T dW, dL/dB = s dW A^T from the merged weight's gradient."""
    s = d.lora_scale
    out = []
    for i in range(d.n_layers):
        L = hf.model.layers[i]
        g = {}
        for p in PROJ_NAMES:
            dW = getattr(getattr(L, _HF[p][0]), _HF[p][1]).weight.grad.numpy()
            A, B = (x.astype(np.float64) for x in lora[i][p])
            g[p] = (s * B.T @ dW, s * dW @ A.T)
        out.append(g)
    return out


@pytest.mark.parametrize("d,seed,B,S,std", [(synth.MICRO, 3, 2, 5, 0.3), (synth.TINY, 0, 1, 64, 0.02)])
def test_sft_step_matches_transformers_llama(d, seed, B, S, std):
    model = oracle_model(d, seed, std=std, random_gamma=True)
    lora = lora_list(d, seed, "normal")
    toks = synth.tokens(seed, B, S, d.vocab)
    loss, grads = oracle.sft_step(model, lora, toks, d, dtype=np.float64)
    hf = _hf_model(d, model, lora)
    ids = torch.from_numpy(toks.astype(np.int64))
    logits = hf(ids).logits  # fp64; the loss is taken here in fp64 too
    ref_loss = torch.nn.functional.cross_entropy(logits[:, :-1].reshape(-1, d.vocab), ids[:, 1:].reshape(-1))
    ref_loss.backward()
    # transformers builds its RoPE tables in fp32, which bounds the agreement
    assert abs(loss - ref_loss.item()) < 1e-7 * abs(loss)
    ref = _hf_lora_grads(d, hf, lora)
    for i in range(d.n_layers):
        for p in PROJ_NAMES:
            for j in range(2):
                a, b = grads[i][p][j], ref[i][p][j]
                assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b), (i, p, j)


def test_seq_logprobs_match_transformers_log_softmax():
    d = synth.MICRO
    model = oracle_model(d, 4, std=0.3)
    lora = lora_list(d, 4, "normal")
    toks = synth.tokens(4, 3, 9, d.vocab)
    hL = oracle.model_forward(model, lora, toks, d, np.float64)
    lp = oracle.seq_logprobs(hL, model["gf"], model["head"], toks, 4, d.rms_eps)
    hf = _hf_model(d, model, lora)
    with torch.no_grad():
        logits = hf(torch.from_numpy(toks.astype(np.int64))).logits
    ls = torch.log_softmax(logits, -1)[:, 3:8, :]
    ref = torch.gather(ls, 2, torch.from_numpy(toks[:, 4:].astype(np.int64))[..., None])[..., 0].sum(1)
    assert np.allclose(lp, ref.numpy(), rtol=1e-7)


def test_cross_entropy_uniform_logits_is_ln_vocab():
    d = synth.MICRO
    model = oracle_model(d, 5)
    model["head"] = np.zeros_like(model["head"])  # all logits 0
    toks = synth.tokens(5, 2, 6, d.vocab)
    loss, grads = oracle.sft_step(model, lora_list(d, 5, "normal"), toks, d, dtype=np.float64)
    assert abs(loss - np.log(d.vocab)) < 1e-12
    # with no logit depending on the adapters, their gradients vanish
    assert all(np.all(g[p][j] == 0) for g in grads for p in PROJ_NAMES for j in range(2))


def test_sft_loss_at_init_near_closed_form():
    # z = n . w with n of unit RMS and w ~ N(0, 0.02^2): z ~ N(0, 0.02^2 H),
    # E[loss] ~ ln V + sigma^2 / 2 for small sigma.
    d = synth.TINY
    model = oracle_model(d, 0)
    toks = synth.tokens(0, 1, 64, d.vocab)
    loss, _ = oracle.sft_step(model, lora_list(d, 0, "normal"), toks, d)
    sigma2 = 0.02 ** 2 * d.hidden
    assert abs(loss - (np.log(d.vocab) + sigma2 / 2)) < 0.05


def test_sft_step_finite_differences():
    d = synth.MICRO
    model = oracle_model(d, 8, std=0.3, head_std_scale=20.0)
    lora = [{p: (a.astype(np.float64) * 30, b.astype(np.float64) * 30) for p, (a, b) in l.items()}
            for l in lora_list(d, 8, "normal")]
    toks = synth.tokens(8, 2, 5, d.vocab)
    loss, grads = oracle.sft_step(model, lora, toks, d, dtype=np.float64)
    f = lambda: oracle.sft_step(model, lora, toks, d, dtype=np.float64)[0]
    rng = np.random.default_rng(9)
    for i in range(d.n_layers):
        for p in PROJ_NAMES:
            for j in range(2):
                arr = lora[i][p][j]
                v = rng.standard_normal(arr.shape)
                fd = directional_fd(f, arr, v, 1e-6)
                assert np.isclose(fd, np.sum(grads[i][p][j] * v), rtol=1e-6, atol=1e-11), (i, p, j)


def test_dpo_loss_closed_forms():
    lp = np.array([-3.0, -5.0, -4.0, -2.5])
    loss, g = oracle.dpo_loss(lp, lp, 0.1)
    assert loss == pytest.approx(np.log(2.0), abs=1e-15)
    assert np.allclose(g, [-0.1 / 4, -0.1 / 4, 0.1 / 4, 0.1 / 4])
    # one pair, Delta = 10, beta = 0.1: loss = log(1 + e^-1)
    loss, g = oracle.dpo_loss(np.array([0.0, -10.0]), np.array([0.0, 0.0]), 0.1)
    assert loss == pytest.approx(np.log1p(np.exp(-1.0)), rel=1e-14)
    assert g[0] == pytest.approx(-0.1 / (1 + np.e), rel=1e-14)


def test_dpo_step_ln2_when_policy_equals_reference():
    d = synth.MICRO
    model = oracle_model(d, 10, std=0.3)
    lora0 = lora_list(d, 10, "zeroB")
    ch, rj = synth.dpo_pairs(10, 2, 9, 4, d.vocab)
    loss, logps, grads = oracle.dpo_step(model, lora0, ch, rj, 4, 0.1, d, dtype=np.float64)
    assert loss == np.log(2.0)
    assert np.array_equal(logps[:4], logps[4:])
    # chosen == rejected also gives ln 2 with a nonzero adapter
    loss2, _, _ = oracle.dpo_step(model, lora_list(d, 10, "normal"), ch, ch, 4, 0.1, d, dtype=np.float64)
    assert loss2 == pytest.approx(np.log(2.0), abs=1e-15)


def test_dpo_step_finite_differences():
    d = synth.MICRO
    model = oracle_model(d, 12, std=0.3, head_std_scale=20.0)
    lora = [{p: (a.astype(np.float64) * 30, b.astype(np.float64) * 30) for p, (a, b) in l.items()}
            for l in lora_list(d, 12, "normal")]
    ch, rj = synth.dpo_pairs(12, 2, 7, 3, d.vocab)
    loss, logps, grads = oracle.dpo_step(model, lora, ch, rj, 3, 0.5, d, dtype=np.float64)
    f = lambda: oracle.dpo_step(model, lora, ch, rj, 3, 0.5, d, dtype=np.float64)[0]
    rng = np.random.default_rng(13)
    for i in range(d.n_layers):
        for p in ("q", "v", "down"):
            for j in range(2):
                arr = lora[i][p][j]
                v = rng.standard_normal(arr.shape)
                fd = directional_fd(f, arr, v, 1e-6)
                assert np.isclose(fd, np.sum(grads[i][p][j] * v), rtol=1e-6, atol=1e-11), (i, p, j)
