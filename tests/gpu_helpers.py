"""Builds GPU-side inputs (through the C ABI) from the same seeded arrays the
oracle consumes."""
from __future__ import annotations

import numpy as np
import torch

import synth
from synth import PROJ_NAMES

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.detach().cpu().numpy()


def device_blob(q, d, seed, layer, std=0.02, random_gamma=False) -> torch.Tensor:
    """Quantize one layer's seeded bf16 weights on the GPU into a device blob."""
    offs, total = q.binding.blob_layout(d)
    blob = torch.zeros(total, dtype=torch.uint8, device=DEV)
    w = {p: bf16_dev(synth.proj_weight_bf16(d, seed, layer, p, std=std)) for p in PROJ_NAMES}
    g1, g2 = synth.norm_weights(d, seed, layer, random_gamma)
    q.binding.fill_blob(d, blob, w, f32_dev(g1), f32_dev(g2))
    return blob


def lora_layer(q, d, seed, layer, init, mult=1.0):
    lp = synth.lora_params(d, seed, layer, init)
    A = [f32_dev(lp[p][0] * mult) for p in PROJ_NAMES]
    B = [f32_dev(lp[p][1] * mult) for p in PROJ_NAMES]
    return q.LoraLayer(A, B)


def gpu_model(q, d, seed, lora_init, std=0.02, random_gamma=False, lora_mult=1.0):
    """Returns (StreamModel with device blobs, list of pinned host blobs)."""
    blobs = [device_blob(q, d, seed, l, std, random_gamma) for l in range(d.n_layers)]
    loras = [lora_layer(q, d, seed, l, lora_init, lora_mult) for l in range(d.n_layers)]
    m = q.StreamModel(d, blobs, f16_dev(synth.embedding_f16(d, seed)), f16_dev(synth.lm_head_f16(d, seed)),
                      f32_dev(synth.final_norm_weight(d, seed, random_gamma)), loras)
    torch.cuda.synchronize()
    host = []
    for b in blobs:
        h = torch.empty(b.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(b)
        host.append(h)
    return m, host


def oracle_lora(q_lora) -> dict:
    return {p: (to_np(q_lora.A[i]), to_np(q_lora.B[i])) for i, p in enumerate(PROJ_NAMES)}


def run_sft(q, m, toks, mode, ctx=None, ws_fill=None):
    """One stream_step_sft; returns (loss tensor, grads, stats). ws_fill: a
    byte the workspace and the gradient outputs are filled with first."""
    B_ = q.binding
    d = m.dims
    ctx = ctx or q.Context(0)
    grads = [q.LoraGrads(l) for l in m.lora]
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = B_.workspace(B_.step_workspace_bytes(d, 0, toks.shape[0], toks.shape[1]))
    if ws_fill is not None:
        _fill(ws, grads, ws_fill)
    q.stream_step_sft(ctx, m, torch.from_numpy(toks).to(DEV), mode, loss, grads, ws)
    stats = ctx.sync()
    return loss, grads, stats


def _fill(ws, grads, byte):
    ws.fill_(byte)
    for g in grads:
        for t in g.dA + g.dB:
            t.view(torch.uint8).fill_(byte)


def run_dpo(q, m, ch, rj, prompt_len, beta, mode, sched, ctx=None, ws_fill=None):
    """One stream_step_dpo; returns (loss, logps, grads, stats)."""
    B_ = q.binding
    d = m.dims
    ctx = ctx or q.Context(0)
    grads = [q.LoraGrads(l) for l in m.lora]
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    logps = torch.empty(4 * ch.shape[0], dtype=torch.float32, device=DEV)
    ws = B_.workspace(B_.step_workspace_bytes(d, 1, ch.shape[0], ch.shape[1]))
    if ws_fill is not None:
        _fill(ws, grads, ws_fill)
    q.stream_step_dpo(ctx, m, torch.from_numpy(ch).to(DEV), torch.from_numpy(rj).to(DEV), prompt_len, beta, mode,
                      sched, loss, logps, grads, ws)
    stats = ctx.sync()
    return loss, logps, grads, stats


def same_grads(ga, gb) -> bool:
    return all(torch.equal(x, y) for a, b in zip(ga, gb) for x, y in zip(a.dA + a.dB, b.dA + b.dB))


def grad_errors(grads, ref) -> dict:
    from helpers import rel_l2
    out = {}
    for i, g in enumerate(grads):
        for j, p in enumerate(PROJ_NAMES):
            out[f"L{i}.dA_{p}"] = rel_l2(to_np(g.dA[j]), ref[i][p][0])
            out[f"L{i}.dB_{p}"] = rel_l2(to_np(g.dB[j]), ref[i][p][1])
    return out
