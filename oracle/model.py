"""The whole training step, the oracle's version: embedding, L decoder layers,
final RMSNorm, untied LM head, next-token cross-entropy (SFT) or the DPO
objective, and the LoRA gradients of every layer.

Pages: one training step over a frozen NF4 base whose only trainable
parameters are the LoRA adapters (rug.gal article, "En detalle";
guillermodelpino.com article, "El streaming de capas"). Streaming only
reorders when each layer's bytes reach the GPU, so the result must equal a
non-streamed run of the same loss exactly (rug.gal intro and "En detalle";
imasters article, "Do SFT para os métodos de preferência"): the oracle is
the non-streamed computation. DPO's reference model is the same base with the
adapters switched off (same sections).

Readings:
  * SFT loss = mean over b and t < S-1 of logsumexp(z[b,t]) - z[b,t,tok[b,t+1]]
    (N = B*(S-1) positions, no ignore index).
  * Embedding and LM head are untied fp16 matrices, frozen.
  * DPO (Rafailov et al. 2023, eq. 7): lp = sum over response positions
    t = prompt_len..S-1 of log softmax(z[t-1])[tok[t]]; per pair
    Delta = (lp_pol(c) - lp_ref(c)) - (lp_pol(r) - lp_ref(r)) and the loss is
    the mean over pairs of -log sigmoid(beta * Delta). Batch order is
    [chosen_1..chosen_P, rejected_1..rejected_P].
  * A "step" returns the loss and the LoRA gradients; the optimizer update is
    not part of it.

Parity pins: loss = ln V for uniform logits, each dz row sums to zero; the
full SFT loss and LoRA gradients vs transformers' LlamaForCausalLM in fp64
(gradients through the merged weight); DPO = ln 2 when policy equals
reference; central finite differences in fp64 for every gradient.
"""
from __future__ import annotations

import numpy as np

from .layer import PROJ, dequant_layer, layer_bwd, layer_fwd, rmsnorm_bwd, rmsnorm_fwd


def _f16(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def embed(tokens, E_f16_bits, dtype=np.float32):
    """h0[b*S + t] = E[tokens[b, t]] (fp16 values, exact in fp32)."""
    E = _f16(E_f16_bits)
    return E[np.asarray(tokens).reshape(-1)].astype(dtype)


def _logsumexp(z):
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def _softmax(z):
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def head_logits(hL, gf, Wh, eps):
    """Final RMSNorm and LM head: returns (z [T, V], normed, rstd)."""
    n, r = rmsnorm_fwd(hL, gf.astype(hL.dtype), eps)
    return n @ Wh.T, n, r


def head_ce(hL, gf, Wh_f16_bits, tokens, eps):
    """SFT next-token cross-entropy. Returns (loss, dhL)."""
    dt = hL.dtype
    Wh = _f16(Wh_f16_bits).astype(dt)
    B, S = tokens.shape
    z, n, r = head_logits(hL, gf, Wh, eps)
    z = z.reshape(B, S, -1)
    tgt = tokens[:, 1:]
    zz = z[:, :-1, :]
    lse = _logsumexp(zz)
    picked = np.take_along_axis(zz, tgt[..., None].astype(np.int64), axis=-1)[..., 0]
    N = B * (S - 1)
    loss = float(np.sum(lse - picked) / N)
    dz = np.zeros_like(z)
    p = _softmax(zz)
    np.put_along_axis(p, tgt[..., None].astype(np.int64),
                      np.take_along_axis(p, tgt[..., None].astype(np.int64), axis=-1) - 1.0, axis=-1)
    dz[:, :-1, :] = p / dt.type(N)
    dn = dz.reshape(B * S, -1) @ Wh
    dh = rmsnorm_bwd(dn, hL, gf.astype(dt), r)
    return loss, dh.astype(dt)


def seq_logprobs(hL, gf, Wh_f16_bits, tokens, prompt_len, eps, g=None):
    """Per-sequence summed log-probs of the response tokens t >= prompt_len.
    With g (dL/dlp per sequence) also returns dhL."""
    dt = hL.dtype
    Wh = _f16(Wh_f16_bits).astype(dt)
    B, S = tokens.shape
    z, n, r = head_logits(hL, gf, Wh, eps)
    z = z.reshape(B, S, -1)
    rows = z[:, prompt_len - 1: S - 1, :]
    tgt = tokens[:, prompt_len:].astype(np.int64)
    lse = _logsumexp(rows)
    picked = np.take_along_axis(rows, tgt[..., None], axis=-1)[..., 0]
    lp = np.sum(picked - lse, axis=1)
    if g is None:
        return lp
    p = _softmax(rows)
    onehot = np.zeros_like(p)
    np.put_along_axis(onehot, tgt[..., None], 1.0, axis=-1)
    dz = np.zeros_like(z)
    dz[:, prompt_len - 1: S - 1, :] = np.asarray(g, dt)[:, None, None] * (onehot - p)
    dn = dz.reshape(B * S, -1) @ Wh
    dh = rmsnorm_bwd(dn, hL, gf.astype(dt), r)
    return lp, dh.astype(dt)


def dpo_loss(lp_pol, lp_ref, beta):
    """Mean over pairs of -log sigmoid(beta * Delta). lp_* hold
    [chosen_1..chosen_P, rejected_1..rejected_P]. Returns (loss, dL/dlp_pol)."""
    lp_pol = np.asarray(lp_pol, np.float64)
    lp_ref = np.asarray(lp_ref, np.float64)
    P = lp_pol.size // 2
    delta = (lp_pol[:P] - lp_ref[:P]) - (lp_pol[P:] - lp_ref[P:])
    x = beta * delta
    loss = float(np.mean(np.logaddexp(0.0, -x)))
    sig_neg = 1.0 / (1.0 + np.exp(x))          # sigmoid(-x)
    g_c = -beta * sig_neg / P
    return loss, np.concatenate([g_c, -g_c])



def _lora_of(lora, i, dtype):
    if lora is None:
        return None
    return {p: (lora[i][p][0].astype(dtype), lora[i][p][1].astype(dtype)) for p in PROJ}


def model_forward(model, lora, tokens, d, dtype=np.float32, keep_ckpt=False):
    """Embedding + L layers. model = {"layers": [{"nf4": {proj: (packed, absmax)},
    "g1", "g2"}], "embed", "head" (fp16 bits), "gf"}. Returns hL (and the
    layer-boundary states h_0..h_{L-1} when keep_ckpt)."""
    B, S = tokens.shape
    h = embed(tokens, model["embed"], dtype)
    ckpt = []
    for i, lay in enumerate(model["layers"]):
        W = {p: w.astype(dtype) for p, w in dequant_layer(lay["nf4"], d).items()}
        if keep_ckpt:
            ckpt.append(h)
        h = layer_fwd(h, W, lay["g1"], lay["g2"], _lora_of(lora, i, dtype), d, B, S)
    return (h, ckpt) if keep_ckpt else h


def _backward_layers(model, lora, ckpt, dh, d, B, S, dtype):
    grads = [None] * len(model["layers"])
    for i in reversed(range(len(model["layers"]))):
        lay = model["layers"][i]
        W = {p: w.astype(dtype) for p, w in dequant_layer(lay["nf4"], d).items()}
        lo = _lora_of(lora, i, dtype)
        _, cache = layer_fwd(ckpt[i], W, lay["g1"], lay["g2"], lo, d, B, S, keep=True)
        dh, grads[i] = layer_bwd(dh, W, lay["g1"], lay["g2"], lo, d, B, S, cache, need_dx=(i > 0))
    return grads


def sft_step(model, lora, tokens, d, dtype=np.float32):
    """One SFT step: returns (loss, grads) with grads[i][proj] = (dA, dB).
    Layer-boundary states are kept and each layer is recomputed in backward
    (the same arithmetic as keeping everything)."""
    tokens = np.asarray(tokens)
    B, S = tokens.shape
    hL, ckpt = model_forward(model, lora, tokens, d, dtype, keep_ckpt=True)
    loss, dh = head_ce(hL, model["gf"], model["head"], tokens, d.rms_eps)
    grads = _backward_layers(model, lora, ckpt, dh, d, B, S, dtype)
    return loss, grads


def dpo_step(model, lora, chosen, rejected, prompt_len, beta, d, dtype=np.float32):
    """One DPO step: the reference log-probs come from the same layers with
    LoRA off. Returns (loss, logps [4P] = pol_c, pol_r, ref_c, ref_r, grads)."""
    toks = np.concatenate([np.asarray(chosen), np.asarray(rejected)], axis=0)
    B, S = toks.shape
    P = B // 2
    href = model_forward(model, None, toks, d, dtype)
    lp_ref = seq_logprobs(href, model["gf"], model["head"], toks, prompt_len, d.rms_eps)
    hL, ckpt = model_forward(model, lora, toks, d, dtype, keep_ckpt=True)
    lp_pol = seq_logprobs(hL, model["gf"], model["head"], toks, prompt_len, d.rms_eps)
    loss, g = dpo_loss(lp_pol, lp_ref, beta)
    _, dh = seq_logprobs(hL, model["gf"], model["head"], toks, prompt_len, d.rms_eps, g=g.astype(dtype))
    grads = _backward_layers(model, lora, ckpt, dh, d, B, S, dtype)
    logps = np.concatenate([lp_pol[:P], lp_pol[P:], lp_ref[:P], lp_ref[P:]])
    return loss, logps, grads


def pref_step(kind, model, lora, chosen, rejected, prompt_len, d, dtype=np.float32, z0_override=None, **hp):
    """One preference step on the stream: kind "dpo" | "orpo" | "simpo" | "kto".
    Returns (loss, logps [4P] = pol_c, pol_r, ref_c, ref_r (reference entries 0
    for the reference-free kinds), grads). hp: the kind's hyperparameters.
    z0_override (KTO only, for finite differences): use this z0."""
    from .preference import kl_tokens, kto_loss, kto_z0, orpo_loss, simpo_loss
    toks = np.concatenate([np.asarray(chosen), np.asarray(rejected)], axis=0)
    B, S = toks.shape
    P = B // 2
    n = S - prompt_len
    lp_ref = np.zeros(B)
    if kind in ("dpo", "kto"):
        href = model_forward(model, None, toks, d, dtype)
        lp_ref = seq_logprobs(href, model["gf"], model["head"], toks, prompt_len, d.rms_eps)
    hL, ckpt = model_forward(model, lora, toks, d, dtype, keep_ckpt=True)
    lp_pol = seq_logprobs(hL, model["gf"], model["head"], toks, prompt_len, d.rms_eps)
    if kind == "dpo":
        loss, g = dpo_loss(lp_pol, lp_ref, hp.get("beta", 0.1))
    elif kind == "orpo":
        loss, g = orpo_loss(lp_pol, n, hp.get("lam", 0.1))
    elif kind == "simpo":
        loss, g = simpo_loss(lp_pol, n, hp.get("beta", 2.0), hp.get("gamma", 0.5))
    elif kind == "kto":
        if z0_override is None:
            kt = kl_tokens(toks, prompt_len)
            kp = seq_logprobs(model_forward(model, lora, kt, d, dtype), model["gf"], model["head"], kt, prompt_len,
                              d.rms_eps)
            kr = seq_logprobs(model_forward(model, None, kt, d, dtype), model["gf"], model["head"], kt, prompt_len,
                              d.rms_eps)
            z0 = kto_z0(kp, kr)
        else:
            z0 = z0_override
        loss, g = kto_loss(lp_pol, lp_ref, z0, hp.get("beta", 0.1), hp.get("lam_d", 1.0), hp.get("lam_u", 1.0))
    else:
        raise ValueError(kind)
    _, dh = seq_logprobs(hL, model["gf"], model["head"], toks, prompt_len, d.rms_eps, g=g.astype(dtype))
    grads = _backward_layers(model, lora, ckpt, dh, d, B, S, dtype)
    logps = np.concatenate([lp_pol[:P], lp_pol[P:], lp_ref[:P], lp_ref[P:]])
    return loss, logps, grads

