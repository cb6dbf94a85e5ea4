"""Writes the oracle's results for the full-depth 8B-shaped steps, for the GPU
parity tests at the sizes the pages quote (rug.gal "Soup: fine-tune 8B on a
4 GB laptop GPU", intro and "En detalle": the 8B model at batch 1, seq 512;
imasters.com.br "Soup promete fine-tuning...", "Do SFT para os metodos de
preferencia": DPO on the same stream).

Calls only oracle/ (and the seeded input generators in synth/); no value comes
from the GPU path. The LoRA gradients of 32 layers are 168 M floats, so the
file keeps, per layer and projection, the fp64 norm of dA and dB and a fixed
sample of their entries (indices from a seeded generator the test repeats);
the loss (and for DPO the four sequence log-probs per pair) in full.

    python tests/golden/make_fullsize_golden.py [sft] [dpo]

writes tests/golden/sft8b_32l_b1x512_seed1.npz and
tests/golden/dpo8b_32l_2x512_p128_seed1.npz (about 20 to 60 minutes of CPU
each on 8 cores).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

SEED = 1
SAMPLES = 512  # entries kept per gradient tensor


def sample_index(layer: int, proj: int, which: int, size: int) -> np.ndarray:
    """The flat indices kept for one gradient tensor (which: 0 = dA, 1 = dB)."""
    g = np.random.default_rng([20261203, layer, proj, which])
    return np.sort(g.choice(size, size=min(SAMPLES, size), replace=False))


def model(d):
    layers = []
    for l in range(d.n_layers):
        t = time.time()
        nf4 = {p: oracle.nf4_quantize(synth.bf16_bits_to_f32(synth.proj_weight_bf16(d, SEED, l, p)))
               for p in synth.PROJ_NAMES}
        g1, g2 = synth.norm_weights(d, SEED, l)
        layers.append(dict(nf4=nf4, g1=g1, g2=g2))
        print(f"  layer {l} quantized ({time.time() - t:.0f} s)", flush=True)
    return dict(layers=layers, embed=synth.embedding_f16(d, SEED), head=synth.lm_head_f16(d, SEED),
                gf=synth.final_norm_weight(d, SEED))


def pack(grads, d) -> dict:
    out = {}
    for l, gl in enumerate(grads):
        for j, p in enumerate(synth.PROJ_NAMES):
            for w, arr in enumerate(gl[p]):
                a = np.asarray(arr, np.float64).ravel()
                idx = sample_index(l, j, w, a.size)
                key = f"L{l}_{p}_{'dA' if w == 0 else 'dB'}"
                out[key + "_norm"] = np.float64(np.linalg.norm(a))
                out[key + "_sample"] = a[idx].astype(np.float32)
    return out


def main(which) -> None:
    d = synth.LLAMA8B
    lora = [synth.lora_params(d, SEED, l, "kaiming") for l in range(d.n_layers)]
    t0 = time.time()
    m = model(d)
    print(f"model quantized in {time.time() - t0:.0f} s", flush=True)
    if "sft" in which:
        toks = synth.tokens(SEED, 1, 512, d.vocab)
        t = time.time()
        loss, grads = oracle.sft_step(m, lora, toks, d)
        print(f"sft step {time.time() - t:.0f} s, loss {loss}", flush=True)
        np.savez_compressed(os.path.join(HERE, "sft8b_32l_b1x512_seed1.npz"), loss=np.float64(loss),
                            samples=np.int64(SAMPLES), **pack(grads, d))
    if "dpo" in which:
        ch, rj = synth.dpo_pairs(SEED, 2, 512, 128, d.vocab)
        t = time.time()
        loss, logps, grads = oracle.dpo_step(m, lora, ch, rj, 128, 0.1, d)
        print(f"dpo step {time.time() - t:.0f} s, loss {loss}, logps {logps}", flush=True)
        np.savez_compressed(os.path.join(HERE, "dpo8b_32l_2x512_p128_seed1.npz"), loss=np.float64(loss),
                            logps=np.asarray(logps, np.float64), samples=np.int64(SAMPLES), **pack(grads, d))


if __name__ == "__main__":
    main(sys.argv[1:] or ["sft", "dpo"])
