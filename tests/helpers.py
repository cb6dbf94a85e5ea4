"""Shared test helpers: build oracle-side models from the seeded generators,
rel-L2, finite differences."""
from __future__ import annotations

import numpy as np

import oracle
import synth
from synth import PROJ_NAMES


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def layer_bf16_weights(d, seed, layer, std=0.02):
    return {p: synth.proj_weight_bf16(d, seed, layer, p, std=std) for p in PROJ_NAMES}


def oracle_model(d, seed, std=0.02, random_gamma=False, head_std_scale=1.0):
    """{"layers": [{"nf4", "g1", "g2"}], "embed", "head", "gf"} with the
    oracle's own NF4 quantization of the seeded bf16 weights."""
    layers = []
    for l in range(d.n_layers):
        wb = layer_bf16_weights(d, seed, l, std)
        nf4 = {p: oracle.nf4_quantize(synth.bf16_bits_to_f32(w)) for p, w in wb.items()}
        g1, g2 = synth.norm_weights(d, seed, l, random_gamma)
        layers.append(dict(nf4=nf4, g1=g1, g2=g2))
    head = synth.lm_head_f16(d, seed)
    if head_std_scale != 1.0:
        head = synth.to_f16_bits(synth.f16_bits_to_f32(head) * head_std_scale)
    return dict(layers=layers, embed=synth.embedding_f16(d, seed), head=head,
                gf=synth.final_norm_weight(d, seed, random_gamma))


def lora_list(d, seed, init):
    return [synth.lora_params(d, seed, l, init) for l in range(d.n_layers)]


def directional_fd(f, x, v, eps):
    """(f(x + eps v) - f(x - eps v)) / (2 eps) with x modified in place and restored."""
    x0 = x.copy()
    x[...] = x0 + eps * v
    fp = f()
    x[...] = x0 - eps * v
    fm = f()
    x[...] = x0
    return (fp - fm) / (2 * eps)
