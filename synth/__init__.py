"""Seeded synthetic inputs for the layer-streamed QLoRA training step.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no quantization, no layer math, no loss). Both the oracle
checks and the GPU path consume exactly these arrays, so every comparison runs
on identical inputs.

Workload recipes follow the configurations the pages' numbers are quoted on
(Llama-3.1-8B-Instruct shape, batch 1 or 4, sequence 512, LoRA r 64 alpha 16,
NF4 4-bit base) plus a tiny 2-layer model and a micro model for
finite-difference checks.

Random streams
--------------
Every array comes from its own PCG64 stream keyed by
``SeedSequence(entropy=seed, spawn_key=(stream, *index))`` so that any layer,
projection or row-chunk can be generated on its own, in any order and in
parallel threads, with the same result.

Weights are drawn in fp32 and rounded to bf16 the way a bf16 checkpoint would
hold them (round-to-nearest-even, done by torch's dtype conversion); the
embedding and LM head are fp16.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Stream ids (first element of the spawn key).
_S_WEIGHT, _S_LORA, _S_EMBED, _S_HEAD, _S_TOKENS, _S_ACT, _S_DPO, _S_NORM = range(8)

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass(frozen=True)
class Dims:
    """Decoder dimensions (Llama-style) plus LoRA rank/alpha."""
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    n_layers: int
    lora_r: int
    lora_alpha: float
    rms_eps: float = 1e-5
    rope_theta: float = 5e5

    def proj_shape(self, name: str) -> tuple[int, int]:
        """(out, in) of projection ``name``."""
        H, hd = self.hidden, self.head_dim
        return {
            "q": (self.n_heads * hd, H),
            "k": (self.n_kv_heads * hd, H),
            "v": (self.n_kv_heads * hd, H),
            "o": (H, self.n_heads * hd),
            "gate": (self.inter, H),
            "up": (self.inter, H),
            "down": (H, self.inter),
        }[name]

    @property
    def lora_scale(self) -> float:
        return float(self.lora_alpha) / float(self.lora_r)


# Workloads -----------------------------------------------------------------
TINY = Dims(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, inter=688,
            vocab=1024, n_layers=2, lora_r=8, lora_alpha=16.0)
LLAMA8B = Dims(hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, inter=14336,
               vocab=128256, n_layers=32, lora_r=64, lora_alpha=16.0)
LLAMA8B_LAYER = dataclasses.replace(LLAMA8B, n_layers=1)
# Micro model for fp64 finite-difference checks of the oracle.
MICRO = Dims(hidden=16, n_heads=2, n_kv_heads=1, head_dim=8, inter=24, vocab=32,
             n_layers=2, lora_r=4, lora_alpha=8.0)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(int(k) for k in key))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_f32(n: int, std: float, seed: int, *key: int) -> np.ndarray:
    """n fp32 draws of N(0, std^2) in independently seeded chunks."""
    out = np.empty(n, dtype=np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        _rng(seed, *key, c).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(std)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def _uniform_f32(n: int, bound: float, seed: int, *key: int) -> np.ndarray:
    g = _rng(seed, *key)
    return (g.random(n, dtype=np.float32) * np.float32(2 * bound) - np.float32(bound)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return b.view(np.float16).astype(np.float32)


# Base model ------------------------------------------------------------------
def proj_weight_bf16(d: Dims, seed: int, layer: int, name: str, std: float = 0.02) -> np.ndarray:
    """Frozen base weight [out, in] as bf16 bits, N(0, std^2) before rounding."""
    out_f, in_f = d.proj_shape(name)
    w = _normal_f32(out_f * in_f, std, seed, _S_WEIGHT, layer, PROJ_NAMES.index(name))
    return to_bf16_bits(w).reshape(out_f, in_f)


def layer_weights_bf16(d: Dims, seed: int, layer: int) -> dict[str, np.ndarray]:
    return {p: proj_weight_bf16(d, seed, layer, p) for p in PROJ_NAMES}


def norm_weights(d: Dims, seed: int, layer: int, random_gamma: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm gains (attention, MLP) in fp32: ones (Llama init) or 1 + N(0, 0.1)."""
    if not random_gamma:
        return np.ones(d.hidden, np.float32), np.ones(d.hidden, np.float32)
    g = _normal_f32(2 * d.hidden, 0.1, seed, _S_NORM, layer) + np.float32(1.0)
    return g[: d.hidden].copy(), g[d.hidden:].copy()


def final_norm_weight(d: Dims, seed: int, random_gamma: bool = False) -> np.ndarray:
    if not random_gamma:
        return np.ones(d.hidden, np.float32)
    return _normal_f32(d.hidden, 0.1, seed, _S_NORM, 1 << 20) + np.float32(1.0)


def embedding_f16(d: Dims, seed: int) -> np.ndarray:
    """Token embedding [vocab, hidden] as fp16 bits, N(0, 0.02^2)."""
    return to_f16_bits(_normal_f32(d.vocab * d.hidden, 0.02, seed, _S_EMBED)).reshape(d.vocab, d.hidden)


def lm_head_f16(d: Dims, seed: int) -> np.ndarray:
    """Untied LM head [vocab, hidden] as fp16 bits, N(0, 0.02^2)."""
    return to_f16_bits(_normal_f32(d.vocab * d.hidden, 0.02, seed, _S_HEAD)).reshape(d.vocab, d.hidden)


# LoRA ------------------------------------------------------------------------
def lora_params(d: Dims, seed: int, layer: int, init: str) -> dict[str, tuple[np.ndarray, np.ndarray]]:
    """LoRA (A [r, in], B [out, r]) fp32 per projection.

    init = "normal":  A, B ~ N(0, 0.01^2)                  (tiny workload)
    init = "kaiming": A ~ U(-1/sqrt(in), 1/sqrt(in)), B ~ N(0, 1e-3^2)   (8B-shaped)
    init = "zeroB":   A ~ U(+-1/sqrt(in)), B = 0            (standard LoRA start)
    """
    out = {}
    r = d.lora_r
    for i, p in enumerate(PROJ_NAMES):
        o, n = d.proj_shape(p)
        if init == "normal":
            A = _normal_f32(r * n, 0.01, seed, _S_LORA, layer, i, 0).reshape(r, n)
            B = _normal_f32(o * r, 0.01, seed, _S_LORA, layer, i, 1).reshape(o, r)
        elif init in ("kaiming", "zeroB"):
            A = _uniform_f32(r * n, 1.0 / np.sqrt(n), seed, _S_LORA, layer, i, 0).reshape(r, n)
            if init == "kaiming":
                B = _normal_f32(o * r, 1e-3, seed, _S_LORA, layer, i, 1).reshape(o, r)
            else:
                B = np.zeros((o, r), np.float32)
        else:
            raise ValueError(init)
        out[p] = (np.ascontiguousarray(A), np.ascontiguousarray(B))
    return out


# Data ------------------------------------------------------------------------
def tokens(seed: int, batch: int, seq: int, vocab: int) -> np.ndarray:
    """Uniform random token ids in [0, vocab), int32 [batch, seq]."""
    return _rng(seed, _S_TOKENS, batch, seq).integers(0, vocab, size=(batch, seq), dtype=np.int32)


def activations_bf16(seed: int, rows: int, cols: int, which: int = 0) -> np.ndarray:
    """N(0, 1) activations as bf16 bits [rows, cols] (which=0: x, which=1: upstream dY)."""
    return to_bf16_bits(_normal_f32(rows * cols, 1.0, seed, _S_ACT, which)).reshape(rows, cols)


def activations_f32(seed: int, rows: int, cols: int, which: int = 0) -> np.ndarray:
    return _normal_f32(rows * cols, 1.0, seed, _S_ACT, which).reshape(rows, cols)


def dpo_pairs(seed: int, pairs: int, seq: int, prompt_len: int, vocab: int) -> tuple[np.ndarray, np.ndarray]:
    """Preference pairs: each pair shares its own random prompt of prompt_len
    tokens; chosen and rejected responses are independent uniform tokens.
    Returns (chosen, rejected), each int32 [pairs, seq]."""
    g = _rng(seed, _S_DPO, pairs, seq, prompt_len)
    prompt = g.integers(0, vocab, size=(pairs, prompt_len), dtype=np.int32)
    resp_c = g.integers(0, vocab, size=(pairs, seq - prompt_len), dtype=np.int32)
    resp_r = g.integers(0, vocab, size=(pairs, seq - prompt_len), dtype=np.int32)
    return (np.concatenate([prompt, resp_c], axis=1), np.concatenate([prompt, resp_r], axis=1))
