"""One Llama-style decoder layer with a frozen NF4 base and LoRA adapters,
forward and backward, the oracle's version.

Pages: the base stays frozen and is fed one decoder layer at a time; LoRA
adapters (r 64, alpha 16 in the example config) are the only trainable
parameters (rug.gal article, "En detalle"; guillermodelpino.com article,
"Qué es exactamente" and "El streaming de capas"). The trained model is
Llama-3.1-8B-Instruct (all pages' intros), so the layer is the Llama decoder:

  n1 = RMSNorm(h; g1)
  q, k, v = QLoRA(n1)                       (q: n_heads*hd, k/v: n_kv_heads*hd)
  q, k = RoPE(q), RoPE(k)                   rotate-half, theta, positions 0..S-1
  o = softmax(q k^T / sqrt(hd) + causal) v  per head, head h reads KV head
                                            h // (n_heads / n_kv_heads)
  h1 = h + QLoRA_o(o)
  n2 = RMSNorm(h1; g2)
  out = h1 + QLoRA_down(silu(QLoRA_gate(n2)) * QLoRA_up(n2))

QLoRA(x) = x W'^T + s (x A^T) B^T with W' the dequantized NF4 weight,
A [r, in], B [out, r], s = alpha / r (LoRA, Hu et al. 2021, section 4.1).

Readings where the pages are silent: no dropout; no Llama-3.1 RoPE frequency
rescaling; RMSNorm eps 1e-5; inverse frequencies theta^(-2j/hd) computed in
fp64; the frozen weight enters each matmul as its NF4 value rounded to bf16,
the computation data type QLoRA dequantizes to (QLoRA paper, section 3);
everything else (activations, LoRA adapters, reductions) stays in the
working precision (fp32, or fp64 for the finite-difference checks).

Parity pins: RMSNorm vs torch.nn.functional.rms_norm and RMS(out)=1; RoPE
norm preservation, identity at position 0, relative-position property; causal
attention vs torch scaled_dot_product_attention, S=1 gives v, the first query
gives v_0, uniform scores give prefix means; LoRA with B=0 or A=0 equals the
base; LoRA equals the merged weight; the whole layer vs transformers'
LlamaDecoderLayer; every backward vs central finite differences in fp64.
"""
from __future__ import annotations

import numpy as np

from .nf4 import bf16_round, nf4_dequant

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


# RMSNorm ---------------------------------------------------------------------
def rmsnorm_fwd(x, g, eps):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis. Returns (y, rstd)."""
    dt = x.dtype
    rstd = (1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + dt.type(eps))).astype(dt)
    return (x * rstd * g).astype(dt), rstd


def rmsnorm_bwd(dy, x, g, rstd):
    """dx for y = x*rstd*g with g frozen."""
    xhat = x * rstd
    dyg = dy * g
    return (rstd * (dyg - xhat * np.mean(dyg * xhat, axis=-1, keepdims=True))).astype(x.dtype)


# RoPE ------------------------------------------------------------------------
def rope_cos_sin(seq: int, hd: int, theta: float, dtype=np.float32):
    """cos, sin tables [seq, hd/2] for positions 0..seq-1 and inverse
    frequencies theta^(-2j/hd), j = 0..hd/2-1 (computed in fp64)."""
    j = np.arange(hd // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / hd)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope_fwd(x, cos, sin):
    """Rotate-half RoPE. x [B, S, nh, hd]; pairs (j, j + hd/2) rotate by angle
    pos * inv_freq_j."""
    half = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(x.dtype)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation (a rotation by -angle)."""
    half = dy.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1).astype(dy.dtype)


# Attention -------------------------------------------------------------------
def _expand_kv(t, group):
    # [B, S, nkv, hd] -> [B, nkv*group, S, hd] with head h reading kv head h // group
    return np.repeat(t.transpose(0, 2, 1, 3), group, axis=1)


def attention_fwd(q, k, v):
    """Causal grouped-query attention. q [B,S,nH,hd], k,v [B,S,nKV,hd].
    Returns (o [B,S,nH,hd], P [B,nH,S,S])."""
    B, S, nH, hd = q.shape
    group = nH // k.shape[2]
    dt = q.dtype
    qh = q.transpose(0, 2, 1, 3)
    kh, vh = _expand_kv(k, group), _expand_kv(v, group)
    scale = dt.type(1.0 / np.sqrt(hd))
    s = (qh @ kh.transpose(0, 1, 3, 2)) * scale
    mask = np.triu(np.ones((S, S), bool), k=1)
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    P = (e / e.sum(axis=-1, keepdims=True)).astype(dt)
    o = (P @ vh).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(o, dtype=dt), P


def attention_bwd(do, q, k, v, P):
    """Gradients (dq, dk, dv) of causal GQA attention given dO [B,S,nH,hd]."""
    B, S, nH, hd = q.shape
    nKV = k.shape[2]
    group = nH // nKV
    dt = q.dtype
    scale = dt.type(1.0 / np.sqrt(hd))
    qh = q.transpose(0, 2, 1, 3)
    kh, vh = _expand_kv(k, group), _expand_kv(v, group)
    doh = do.transpose(0, 2, 1, 3)
    dvh = P.transpose(0, 1, 3, 2) @ doh
    dP = doh @ vh.transpose(0, 1, 3, 2)
    dS = P * (dP - np.sum(dP * P, axis=-1, keepdims=True))
    dqh = (dS @ kh) * scale
    dkh = (dS.transpose(0, 1, 3, 2) @ qh) * scale
    dk = dkh.reshape(B, nKV, group, S, hd).sum(axis=2).transpose(0, 2, 1, 3)
    dv = dvh.reshape(B, nKV, group, S, hd).sum(axis=2).transpose(0, 2, 1, 3)
    dq = dqh.transpose(0, 2, 1, 3)
    return (np.ascontiguousarray(dq, dtype=dt), np.ascontiguousarray(dk, dtype=dt),
            np.ascontiguousarray(dv, dtype=dt))


# SwiGLU ----------------------------------------------------------------------
def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu_fwd(g, u):
    """silu(g) * u."""
    return (g * _sigmoid(g) * u).astype(g.dtype)


def swiglu_bwd(da, g, u):
    """(dg, du) for a = silu(g) * u."""
    sg = _sigmoid(g)
    silu = g * sg
    dsilu = sg * (1.0 + g * (1.0 - sg))
    return (da * u * dsilu).astype(g.dtype), (da * silu).astype(g.dtype)


# QLoRA linear ----------------------------------------------------------------
def qlora_linear_fwd(x, W, A, B, s):
    """y = x W^T + s (x A^T) B^T. x [T,in], W [out,in] (dequantized),
    A [r,in], B [out,r]. A or B None means LoRA off. Returns (y, u = x A^T)."""
    y = x @ W.T
    if A is None or B is None:
        return y.astype(x.dtype), None
    u = x @ A.T
    return (y + x.dtype.type(s) * (u @ B.T)).astype(x.dtype), u.astype(x.dtype)


def qlora_linear_bwd(dy, x, u, W, A, B, s, need_dx=True):
    """Backward of qlora_linear_fwd with W frozen.

    du = s dy B;  dx = dy W + du A;  dB = s dy^T u;  dA = du^T x."""
    dt = x.dtype
    s = dt.type(s)
    dx = (dy @ W) if need_dx else None
    if A is None or B is None:
        return (dx.astype(dt) if dx is not None else None), None, None
    du = s * (dy @ B)
    if need_dx:
        dx = dx + du @ A
    dB = s * (dy.T @ u)
    dA = du.T @ x
    return (dx.astype(dt) if dx is not None else None), dA.astype(dt), dB.astype(dt)


# Decoder layer ---------------------------------------------------------------
def dequant_layer(layer_nf4: dict, d) -> dict:
    """{proj: (packed, absmax)} -> {proj: W' [out, in]}, the weight operand of
    the layer's matmuls: the NF4 value fl32(c[code] * absmax) rounded to the
    bf16 computation data type (QLoRA dequantizes its 4-bit storage type to
    the 16-bit BrainFloat computation type before each matmul, section 3 and
    equation 5 of the QLoRA paper). Values are returned as float32 arrays."""
    out = {}
    for p in PROJ:
        o, i = d.proj_shape(p)
        packed, absmax = layer_nf4[p]
        out[p] = bf16_round(nf4_dequant(packed, absmax, o * i)).reshape(o, i)
    return out


def _lin(x, W, lora, p, s):
    if lora is None:
        return qlora_linear_fwd(x, W[p], None, None, s)
    A, B = lora[p]
    return qlora_linear_fwd(x, W[p], A.astype(x.dtype), B.astype(x.dtype), s)


def layer_fwd(h, W, g1, g2, lora, d, batch, seq, keep=False):
    """One decoder layer. h [T, H] with T = batch*seq (row b*seq + t).
    W: {proj: W'} in the working dtype; lora: {proj: (A, B)} or None (off).
    Returns out [T, H] (and a cache for layer_bwd when keep=True)."""
    dt = h.dtype
    T, H = h.shape
    nH, nKV, hd = d.n_heads, d.n_kv_heads, d.head_dim
    s = d.lora_scale
    g1, g2 = g1.astype(dt), g2.astype(dt)
    n1, r1 = rmsnorm_fwd(h, g1, d.rms_eps)
    q, uq = _lin(n1, W, lora, "q", s)
    k, uk = _lin(n1, W, lora, "k", s)
    v, uv = _lin(n1, W, lora, "v", s)
    cos, sin = rope_cos_sin(seq, hd, d.rope_theta, dt)
    q4 = rope_fwd(q.reshape(batch, seq, nH, hd), cos, sin)
    k4 = rope_fwd(k.reshape(batch, seq, nKV, hd), cos, sin)
    v4 = v.reshape(batch, seq, nKV, hd)
    o4, P = attention_fwd(q4, k4, v4)
    o = o4.reshape(T, nH * hd)
    yo, uo = _lin(o, W, lora, "o", s)
    h1 = h + yo
    n2, r2 = rmsnorm_fwd(h1, g2, d.rms_eps)
    gt, ug = _lin(n2, W, lora, "gate", s)
    up, uu = _lin(n2, W, lora, "up", s)
    a = swiglu_fwd(gt, up)
    yd, ud = _lin(a, W, lora, "down", s)
    out = (h1 + yd).astype(dt)
    if not keep:
        return out
    cache = dict(h=h, n1=n1, r1=r1, q4=q4, k4=k4, v4=v4, P=P, o=o, h1=h1, n2=n2, r2=r2,
                 gt=gt, up=up, a=a, u={"q": uq, "k": uk, "v": uv, "o": uo, "gate": ug,
                                       "up": uu, "down": ud}, cos=cos, sin=sin)
    return out, cache


def layer_bwd(dout, W, g1, g2, lora, d, batch, seq, cache, need_dx=True):
    """Backward of layer_fwd. Returns (dh [T,H] or None, {proj: (dA, dB)})."""
    dt = dout.dtype
    T, H = dout.shape
    nH, nKV, hd = d.n_heads, d.n_kv_heads, d.head_dim
    s = d.lora_scale
    g1, g2 = g1.astype(dt), g2.astype(dt)
    c = cache
    grads = {}

    def lin_bwd(dy, x, p, nd=True):
        A, B = (None, None) if lora is None else (lora[p][0].astype(dt), lora[p][1].astype(dt))
        dx, dA, dB = qlora_linear_bwd(dy, x, c["u"][p], W[p], A, B, s, need_dx=nd)
        grads[p] = (dA, dB)
        return dx

    # out = h1 + down(a)
    da = lin_bwd(dout, c["a"], "down")
    dg, du = swiglu_bwd(da, c["gt"], c["up"])
    dn2 = lin_bwd(dg, c["n2"], "gate") + lin_bwd(du, c["n2"], "up")
    dh1 = dout + rmsnorm_bwd(dn2, c["h1"], g2, c["r2"])
    # h1 = h + o_proj(o)
    do = lin_bwd(dh1, c["o"], "o")
    dq4, dk4, dv4 = attention_bwd(do.reshape(batch, seq, nH, hd), c["q4"], c["k4"], c["v4"], c["P"])
    dq = rope_bwd(dq4, c["cos"], c["sin"]).reshape(T, nH * hd)
    dk = rope_bwd(dk4, c["cos"], c["sin"]).reshape(T, nKV * hd)
    dv = dv4.reshape(T, nKV * hd)
    dn1 = lin_bwd(dq, c["n1"], "q", need_dx)
    dn1k = lin_bwd(dk, c["n1"], "k", need_dx)
    dn1v = lin_bwd(dv, c["n1"], "v", need_dx)
    if not need_dx:
        return None, grads
    dn1 = dn1 + dn1k + dn1v
    dh = dh1 + rmsnorm_bwd(dn1, c["h"], g1, c["r1"])
    return dh.astype(dt), grads
