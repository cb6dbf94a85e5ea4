#!/usr/bin/env python3
"""Throughput of the layer-streamed QLoRA training step on one MI355X.

Default workload: one streamed SFT step of a 32-layer Llama-3.1-8B-shaped
model (hidden 4096, 32/8 heads, head_dim 128, SwiGLU 14336, vocab 128256),
NF4 base layers in pinned host RAM fed to the GPU one decoder layer at a time,
LoRA r 64 / alpha 16 on all 7 projections resident, batch 1, sequence 512,
seeded synthetic weights and uniform random tokens (seed 1); each step ends
with the AdamW update of every LoRA factor (lr 2e-5). Other workloads:
--workload sft8b_b4 (batch 4), dpo8b (2 preference pairs, 128-token
prompts, beta 0.1), and orpo8b / simpo8b / kto8b on the same pairs.
--source disk streams the stack from a file read with O_DIRECT (disk ->
pinned staging -> device); --source auto takes RAM when the stack fits in
available host memory and the file otherwise.

Prints ONE JSON line. `value` is tokens/s over the timed steps (inputs
resident: weights in pinned host RAM as the method keeps them, tokens on the
device), which run with no profiling events. The same number of steps then
runs again, untimed, with the library bracketing only the fused NF4-dequant
MFMA GEMMs with HIP events (every other kernel runs with none); `roofline`
reports the dominant one of them from those events. One further, untimed
step with events around every kernel gives the per-kernel table (`kernels`,
`gpu_time`). `cpu_baseline` times the oracle on a bounded sample
on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import tempfile
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/s, streamed NF4+LoRA Llama-8B-shape step; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
SEED = 1
LR = 2e-5  # the pages' learning rate (AdamW, betas 0.9 / 0.999, eps 1e-8, no weight decay)

WORKLOADS = {
    "sft8b_b1": dict(kind="sft", batch=1, seq=512,
                     name="streamed SFT step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, batch 1, seq 512"),
    "sft8b_b4": dict(kind="sft", batch=4, seq=512,
                     name="streamed SFT step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, batch 4, seq 512"),
    # out-of-config batch sweep (where copies start to hide behind compute)
    "sft8b_b8": dict(kind="sft", batch=8, seq=512,
                     name="streamed SFT step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, batch 8, seq 512"),
    "sft8b_b16": dict(kind="sft", batch=16, seq=512,
                      name="streamed SFT step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, batch 16, seq 512"),
    "dpo8b": dict(kind="dpo", batch=2, seq=512, prompt=128, beta=0.1,
                  name="streamed DPO step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, 2 pairs x seq 512"),
    "orpo8b": dict(kind="orpo", batch=2, seq=512, prompt=128,
                   name="streamed ORPO step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, 2 pairs x seq 512"),
    "simpo8b": dict(kind="simpo", batch=2, seq=512, prompt=128,
                    name="streamed SimPO step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, 2 pairs x seq 512"),
    "kto8b": dict(kind="kto", batch=2, seq=512, prompt=128,
                  name="streamed KTO step, 32-layer Llama-3.1-8B-shaped NF4 base + LoRA r64, 2 pairs x seq 512"),
    # one decoder layer alone (layer_fwd, then layer_bwd with its recomputed
    # forward: the per-layer work of a streamed step), resident on the device
    "layer8b": dict(kind="layer", batch=1, seq=512,
                    name="one Llama-3.1-8B-shaped NF4 + LoRA r64 decoder layer, forward then backward, batch 1, seq 512"),
}


# HBM bytes per launch of the NF4 GEMM rows that can come out dominant on the
# default workload (gemm_nf4_nt, the forward and recompute products, or
# gemm_nf4_nn, the dX products; the two run within a few percent of each
# other), from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) over the
# default workload, each scaled by the same counter on a plain 1 GiB device
# copy (factors 2.000 and 1.000), weighted over the row's dispatches; valid only
# for the kernel source they were taken on (SHA-256 prefix of csrc/k_gemm.hip).
MEASURED_TRAFFIC = {("sft8b_b1", "streamed", "gemm_nf4_nt"): {"bytes": int((100.4 + 30.2) * 1e6),
                                                              "k_gemm_sha256": "3901c14538590722"},
                    ("sft8b_b1", "streamed", "gemm_nf4_nn"): {"bytes": int((115.2 + 28.8) * 1e6),
                                                              "k_gemm_sha256": "3901c14538590722"}}


def measured_traffic(workload: str, mode: str, kernel: str):
    import hashlib
    rec = MEASURED_TRAFFIC.get((workload, mode, kernel))
    if rec is None:
        return None
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "qlora_fine_tuning_dequant_amd", "csrc",
                       "k_gemm.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return rec["bytes"] if sha == rec["k_gemm_sha256"] else None


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def build_model(q, d, seed: int, want_device_blobs: bool = False, wire: bool = False, act: int | None = None):
    """Quantize every layer's seeded bf16 weights on the GPU (nf4_quantize)
    into a device blob and keep a pinned host copy (in the wire form, block
    maxima as bf16, when wire=True). Host-side generation of layer i+1
    overlaps the GPU work of layer i."""
    import numpy as np
    import torch

    import synth
    dev = "cuda:0"
    _, total = q.binding.blob_layout(d)
    host, dev_blobs = [], []
    staging = torch.empty(total, dtype=torch.uint8, device=dev)
    host_staging = torch.empty(total, dtype=torch.uint8, pin_memory=True) if wire else None

    def gen(layer):
        return {p: synth.proj_weight_bf16(d, seed, layer, p) for p in synth.PROJ_NAMES}

    nxt = {}
    th = None

    def start(layer):
        nonlocal th
        def run():
            nxt[layer] = gen(layer)
        th = threading.Thread(target=run)
        th.start()

    start(0)
    for layer in range(d.n_layers):
        th.join()
        w_np = nxt.pop(layer)
        if layer + 1 < d.n_layers:
            start(layer + 1)
        w = {p: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev) for p, a in w_np.items()}
        g1, g2 = synth.norm_weights(d, seed, layer)
        blob = torch.empty(total, dtype=torch.uint8, device=dev) if want_device_blobs else staging
        q.binding.fill_blob(d, blob, w, torch.from_numpy(g1).to(dev), torch.from_numpy(g2).to(dev))
        h = host_staging if wire else torch.empty(total, dtype=torch.uint8, pin_memory=True)
        h.copy_(blob)
        host.append(q.binding.blob_to_wire(d, h) if wire else h)
        if want_device_blobs:
            dev_blobs.append(blob)
        del w
        if layer % 8 == 7:
            log(f"  layers quantized: {layer + 1}/{d.n_layers}")
    loras = []
    for layer in range(d.n_layers):
        lp = synth.lora_params(d, seed, layer, "kaiming")
        loras.append(q.LoraLayer([torch.from_numpy(lp[p][0]).to(dev) for p in synth.PROJ_NAMES],
                                 [torch.from_numpy(lp[p][1]).to(dev) for p in synth.PROJ_NAMES]))
    emb = torch.from_numpy(synth.embedding_f16(d, seed).view(np.int16)).view(torch.float16).to(dev)
    head = torch.from_numpy(synth.lm_head_f16(d, seed).view(np.int16)).view(torch.float16).to(dev)
    gf = torch.from_numpy(synth.final_norm_weight(d, seed)).to(dev)
    m = q.StreamModel(d, host, emb, head, gf, loras,
                      q.binding.QLX_BLOB_WIRE if wire else q.binding.QLX_BLOB_FULL, act_dtype=act)
    return m, dev_blobs


def cpu_baseline(d, batch: int, seq: int) -> dict:
    """The oracle on a bounded sample of the step: one of the 32 decoder
    layers (dequantize, forward, recompute, backward; timed up to three
    times until about 8 s of CPU work, the mean taken) and the final norm +
    LM head + cross-entropy, both at the full batch x seq shape; the step time
    is extrapolated as n_layers x layer + head."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    T = batch * seq
    nf4 = {p: oracle.nf4_quantize(synth.bf16_bits_to_f32(synth.proj_weight_bf16(d, SEED, 0, p)))
           for p in synth.PROJ_NAMES}
    lp = synth.lora_params(d, SEED, 0, "kaiming")
    g1, g2 = synth.norm_weights(d, SEED, 0)
    toks = synth.tokens(SEED, batch, seq, d.vocab)
    h = oracle.embed(toks, synth.embedding_f16(d, SEED))
    dh = synth.activations_f32(SEED, T, d.hidden, 1) * np.float32(1e-4)
    reps, t_sum = 0, 0.0
    while True:  # the layer once, or up to 3 times until ~8 s of CPU work (the mean is used)
        t0 = time.perf_counter()
        W = oracle.dequant_layer(nf4, d)                                       # forward pass dequant
        out = oracle.layer_fwd(h, W, g1, g2, lp, d, batch, seq)
        W = oracle.dequant_layer(nf4, d)                                       # backward pass dequant
        _, cache = oracle.layer_fwd(h, W, g1, g2, lp, d, batch, seq, keep=True)  # recompute
        oracle.layer_bwd(dh, W, g1, g2, lp, d, batch, seq, cache)
        t_sum += time.perf_counter() - t0
        reps += 1
        del W, cache
        if t_sum >= 8.0 or reps == 3:
            break
    t_layer = t_sum / reps
    head = synth.lm_head_f16(d, SEED)
    t0 = time.perf_counter()
    oracle.head_ce(out, synth.final_norm_weight(d, SEED), head, toks, d.rms_eps)
    t_head = time.perf_counter() - t0
    step_s = d.n_layers * t_layer + t_head
    return {"value": round(T / step_s, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {d.n_layers} decoder layers (dequant + fwd + recompute + bwd, {t_layer:.2f} s, mean of "
                      f"{reps} run{'s' if reps > 1 else ''}) and "
                      f"the LM head + cross-entropy ({t_head:.2f} s) at batch {batch} x seq {seq}; "
                      f"step = {d.n_layers} x layer + head = {step_s:.1f} s"}


def cpu_baseline_detail() -> dict:
    """The CPU-baseline leg in full (the oracle as it stands, on this host):
    the tiny model's whole SFT step (L 2, H 256, batch 1 x 64) and one
    8B-shaped layer's forward + recompute + backward at batch 1 x 512, each
    with every BLAS thread and with one; the 32-layer step estimate is 32 x
    that layer + the LM head."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synth
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])

    def model(d, seed):
        layers = []
        for l in range(d.n_layers):
            nf4 = {p: oracle.nf4_quantize(synth.bf16_bits_to_f32(synth.proj_weight_bf16(d, seed, l, p)))
                   for p in synth.PROJ_NAMES}
            g1, g2 = synth.norm_weights(d, seed, l)
            layers.append(dict(nf4=nf4, g1=g1, g2=g2))
        return dict(layers=layers, embed=synth.embedding_f16(d, seed), head=synth.lm_head_f16(d, seed),
                    gf=synth.final_norm_weight(d, seed))

    def c1():
        d = synth.TINY
        m = model(d, 0)
        lora = [synth.lora_params(d, 0, l, "normal") for l in range(d.n_layers)]
        toks = synth.tokens(0, 1, 64, d.vocab)
        t0 = time.perf_counter()
        oracle.sft_step(m, lora, toks, d)
        return time.perf_counter() - t0

    def c2():
        d, batch, seq = synth.LLAMA8B, 1, 512
        T = batch * seq
        nf4 = {p: oracle.nf4_quantize(synth.bf16_bits_to_f32(synth.proj_weight_bf16(d, SEED, 0, p)))
               for p in synth.PROJ_NAMES}
        lp = synth.lora_params(d, SEED, 0, "kaiming")
        g1, g2 = synth.norm_weights(d, SEED, 0)
        h = synth.activations_f32(SEED, T, d.hidden, 0)
        dh = synth.activations_f32(SEED, T, d.hidden, 1) * np.float32(1e-4)
        t0 = time.perf_counter()
        W = oracle.dequant_layer(nf4, d)
        oracle.layer_fwd(h, W, g1, g2, lp, d, batch, seq)
        W = oracle.dequant_layer(nf4, d)
        _, cache = oracle.layer_fwd(h, W, g1, g2, lp, d, batch, seq, keep=True)
        oracle.layer_bwd(dh, W, g1, g2, lp, d, batch, seq, cache)
        return time.perf_counter() - t0

    out = {"host_cpus": os.cpu_count(), "blas_threads": int(threads)}
    out["C1_sft_step_s"] = round(c1(), 3)
    out["C2_layer_fwd_recompute_bwd_s"] = round(c2(), 3)
    with threadpool_limits(limits=1):
        out["C1_sft_step_s_1thread"] = round(c1(), 3)
        out["C2_layer_fwd_recompute_bwd_s_1thread"] = round(c2(), 3)
    return out


def gemm_shapes(q) -> dict:
    """TFLOP/s of the 8B-shaped NF4 GEMMs (LoRA off) through qlora_linear_fwd
    (y = x W'^T) and qlora_linear_bwd (dx = dy W'), from the library's events."""
    import torch
    B_ = q.binding
    dev = "cuda:0"
    shapes = {"qkv": (4096, 6144), "o": (4096, 4096), "gate_up": (4096, 28672), "down": (14336, 4096)}
    g = torch.Generator(device=dev).manual_seed(0)
    out = {}
    for T in (512, 2048):
        for name, (K, N) in shapes.items():
            W = q.NF4Matrix.quantize((torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16))
            x = torch.randn(T, K, device=dev, generator=g).to(torch.bfloat16)
            dy = torch.randn(T, N, device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty(T, N, device=dev, dtype=torch.bfloat16)
            dx = torch.empty(T, K, device=dev, dtype=torch.bfloat16)
            ws = B_.workspace(B_.linear_workspace_bytes(T, K, N, 0))
            for _ in range(3):
                q.qlora_linear_fwd(x, W, None, None, 1.0, y, ws)
                q.qlora_linear_bwd(dy, x, W, None, None, 1.0, dx, None, None, ws=ws)
            torch.cuda.synchronize()
            B_.profile_begin()
            for _ in range(10):
                q.qlora_linear_fwd(x, W, None, None, 1.0, y, ws)
            for _ in range(10):
                q.qlora_linear_bwd(dy, x, W, None, None, 1.0, dx, None, None, ws=ws)
            torch.cuda.synchronize()
            pr = B_.profile_end()
            row = {}
            for k, lab in (("gemm_nf4_nt", "fwd"), ("gemm_nf4_nn", "dx")):
                rows = [v for name_, v in pr.items() if name_.startswith(k)]  # 256- or 512-row tile
                ms, n, fl = (sum(v[f] for v in rows) for f in ("ms", "launches", "flops"))
                row[lab + "_us"] = round(1000 * ms / n, 1)
                row[lab + "_TFLOPs"] = round(fl / ms / 1e9, 1)
                row[lab + "_tile"] = "512x128" if any(nm.endswith("_wide") for nm in pr if nm.startswith(k)) else "256x128"
            if "splitk_reduce" in pr:
                row["splitk_reduce_us_per_launch"] = round(1000 * pr["splitk_reduce"]["ms"] / pr["splitk_reduce"]["launches"], 1)
            out[f"T{T}_{name}"] = row
            log(f"gemm T={T} {name}: {row}")
    return out


def merge_shapes(q) -> dict:
    """Adapter merge (W' + s B A, r 64, alpha 16) of one 8B-shaped decoder
    layer's seven projections, to bf16 and re-quantized to NF4, from the
    library's events. The merge does 2 r fp32 flops per element against
    2.5625 B of HBM traffic (codes, absmax, bf16 out), so it is bound by the
    fp32 vector ALU (157.3 TFLOP/s) rather than HBM at r 64."""
    import torch
    B_ = q.binding
    dev = "cuda:0"
    r, scale = 64, 16.0 / 64
    shapes = {"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
              "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336)}
    g = torch.Generator(device=dev).manual_seed(0)
    out, tot = {}, {"lora_merge": [0.0, 0.0, 0.0], "nf4_quantize": [0.0, 0.0, 0.0]}
    for name, (rows, cols) in shapes.items():
        W = q.NF4Matrix.quantize((torch.randn(rows, cols, device=dev, generator=g) * 0.02).to(torch.bfloat16))
        A = torch.randn(r, cols, device=dev, generator=g) * 0.01
        Bm = torch.randn(rows, r, device=dev, generator=g) * 0.01
        for _ in range(2):
            q.lora_merge(W, A, Bm, scale)
            q.lora_merge(W, A, Bm, scale, to_nf4=True)
        torch.cuda.synchronize()
        B_.profile_begin()
        for _ in range(10):
            q.lora_merge(W, A, Bm, scale)
            q.lora_merge(W, A, Bm, scale, to_nf4=True)
        torch.cuda.synchronize()
        pr = B_.profile_end()
        row = {}
        for k in tot:
            v = pr[k]
            row[k + "_us"] = round(1000 * v["ms"] / v["launches"], 1)
            for i, f in enumerate(("ms", "flops", "bytes")):
                tot[k][i] += v[f] / v["launches"] if f != "ms" else v["ms"] / v["launches"]
        row["merge_TFLOPs"] = round(pr["lora_merge"]["flops"] / pr["lora_merge"]["ms"] / 1e9, 1)
        out[name] = row
        log(f"merge {name} [{rows}x{cols}]: {row}")
    ms, fl, by = tot["lora_merge"]
    out["layer"] = {"lora_merge_us": round(1000 * ms, 1), "nf4_quantize_us": round(1000 * tot["nf4_quantize"][0], 1),
                    "merge_TFLOPs": round(fl / ms / 1e9, 1), "merge_frac_fp32_alu": round(fl / ms / 1e9 / 157.3, 3),
                    "merge_GBs": round(by / ms / 1e6, 1),
                    "nf4_quantize_GBs": round(tot["nf4_quantize"][2] / tot["nf4_quantize"][0] / 1e6, 1)}
    log(f"merge layer: {out['layer']}")
    return out


def measure_peaks(q) -> dict:
    """The device's own peaks next to the vendor's: a bf16 MFMA loop and a
    16-byte HBM copy kernel from the library, and one layer-blob-sized
    (122.7 MB) pinned host-to-device hipMemcpyAsync."""
    import torch
    import synth
    B_ = q.binding
    L = B_.lib()
    dev = "cuda:0"
    s = torch.cuda.current_stream()
    out = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    wgs, iters = 256 * 8, 20000
    buf = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    for shape, key in ((0, "mfma_bf16_16x16x32_TFLOPs"), (1, "mfma_bf16_32x32x16_TFLOPs")):
        ms = timed(lambda: B_._check(L.qlx_peak_mfma(iters, wgs, shape, buf.data_ptr(), s.cuda_stream)), 3)
        out[key] = round(131072.0 * iters * wgs * 4 / ms / 1e9, 1)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = timed(lambda: B_._check(L.qlx_peak_copy(src.data_ptr(), dst.data_ptr(), n, s.cuda_stream)), 10)
    out["hbm_copy_GBps"] = round(2.0 * n / ms / 1e6, 1)
    del src, dst
    _, blob = B_.blob_layout(synth.LLAMA8B)
    h = torch.empty(blob, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(blob, dtype=torch.uint8, device=dev)
    ms = timed(lambda: d.copy_(h, non_blocking=True), 10)
    out["h2d_pinned_GBps"] = round(blob / ms / 1e6, 1)
    out["h2d_bytes"] = blob
    out["vendor"] = {"mfma_bf16_TFLOPs": PEAK_BF16_TFLOPS, "hbm_GBps": 8000.0, "pcie_gen5_x16_GBps": 64.0}
    return out


def _union(iv):
    """Total length of the union of [start, end) intervals (ns)."""
    tot, cur_s, cur_e = 0, None, None
    for a, b in sorted(iv):
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                tot += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    return tot + (cur_e - cur_s if cur_e is not None else 0)


def _overlap(a_iv, b_iv):
    """Length of (union of a) intersected with (union of b), in ns."""
    def merged(iv):
        out = []
        for x, y in sorted(iv):
            if out and x <= out[-1][1]:
                out[-1][1] = max(out[-1][1], y)
            else:
                out.append([x, y])
        return out
    A, B = merged(a_iv), merged(b_iv)
    i = j = tot = 0
    while i < len(A) and j < len(B):
        lo, hi = max(A[i][0], B[j][0]), min(A[i][1], B[j][1])
        if hi > lo:
            tot += hi - lo
        if A[i][1] < B[j][1]:
            i += 1
        else:
            j += 1
    return tot


def layer_bench(q, args, wl) -> dict:
    """One 8B-shaped decoder layer: layer_fwd then layer_bwd (which recomputes
    the forward from h_in), resident, on seeded weights, LoRA and N(0, 1)
    activations; tokens/s of the pair and the per-kernel table of one more
    pass with events around every kernel."""
    import dataclasses
    import torch
    import synth
    B_ = q.binding
    dev = "cuda:0"
    act = B_.QLX_ACT_F16 if args.act == "f16" else B_.QLX_ACT_BF16
    d = dataclasses.replace(synth.LLAMA8B, n_layers=1)
    m, dev_blobs = build_model(q, d, SEED, want_device_blobs=True, act=act)
    dims = B_.Dims.of(d, act)
    batch, seq = wl["batch"], wl["seq"]
    T = batch * seq
    g = torch.Generator(device=dev).manual_seed(SEED)
    h_in = torch.randn(T, d.hidden, device=dev, generator=g)
    dh_out = torch.randn(T, d.hidden, device=dev, generator=g) / T
    h_out, dh_in = torch.empty_like(h_in), torch.empty_like(h_in)
    lora, grads = m.lora[0], q.LoraGrads(m.lora[0])
    ws = B_.workspace(B_.layer_workspace_bytes(dims, batch, seq))

    def step():
        q.layer_fwd(dims, dev_blobs[0], lora, h_in, batch, seq, h_out, ws)
        q.layer_bwd(dims, dev_blobs[0], lora, h_in, dh_out, batch, seq, dh_in, grads, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    B_.profile_begin()
    step()
    torch.cuda.synchronize()
    prof = B_.profile_end()
    gemm = {k: v for k, v in prof.items() if k.startswith("gemm")}
    flops = sum(v["flops"] for v in gemm.values())
    gms = sum(v["ms"] for v in gemm.values())
    log(f"layer fwd+bwd: {1000 * elapsed / args.steps:.3f} ms, GEMMs {gms:.3f} ms at {flops / gms / 1e9:.0f} TFLOP/s")
    return {"metric": "train tokens/s through one decoder layer (forward + backward)", "value":
            round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(1000 * elapsed / args.steps, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": args.act, "data": "synthetic",
            "config": {"workload": wl["name"], "global_batch": batch, "seq_len": seq, "mode": "resident",
                       "activations": args.act, "weight_operand": "bf16 of the NF4 value", "lora_r": d.lora_r},
            "gpu_time": {"kernels_ms": round(sum(v["ms"] for v in prof.values()), 4), "gemm_ms": round(gms, 4),
                         "gemm_TFLOP": round(flops / 1e12, 4), "gemm_TFLOPs_avg": round(flops / gms / 1e9, 1)},
            "kernels": {k: {"launches": v["launches"], "ms": round(v["ms"], 4),
                            "TFLOP/s": round(v["flops"] / max(v["ms"], 1e-9) / 1e9, 1),
                            "GB/s": round(v["bytes"] / max(v["ms"], 1e-9) / 1e6, 1)}
                        for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"])}}


def rocpd_summary(path: str, top: int = 25) -> str:
    """Text summary of a rocprofv3 trace database (--kernel-trace and
    --memory-copy-trace): per-kernel dispatch statistics, and the layer
    stream's host-to-device copies (those above 4 MB: the streamer's halves
    of each layer blob) with their rate and their overlap with kernels, over
    the window from the first to the last such copy."""
    import sqlite3
    db = sqlite3.connect(path)
    cur = db.cursor()
    lines = []
    ks = cur.execute("select name, start, end from kernels").fetchall()
    agg = {}
    for name, a, b in ks:
        e = agg.setdefault(name, [0, 0])
        e[0] += 1
        e[1] += b - a
    total = sum(v[1] for v in agg.values())
    lines.append(f"kernel dispatches: {len(ks)}, total kernel time {total / 1e6:.2f} ms")
    lines.append("")
    lines.append("| kernel | calls | total ms | avg us | % |")
    lines.append("|---|---|---|---|---|")
    for name, (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
        lines.append(f"| `{name[:90]}` | {n} | {t / 1e6:.3f} | {t / n / 1e3:.2f} | {100.0 * t / max(total, 1):.1f} |")
    try:
        cps = cur.execute("select start, end, size, stream_id, name from memory_copies").fetchall()
    except sqlite3.OperationalError:
        cps = []
    h2d = [c for c in cps if c[4] == "MEMORY_COPY_HOST_TO_DEVICE" and c[2] > 4_000_000]
    if h2d:
        w0, w1 = min(c[0] for c in h2d), max(c[1] for c in h2d)
        kin = [(max(a, w0), min(b, w1)) for _, a, b in ks if b > w0 and a < w1]
        civ = [(c[0], c[1]) for c in h2d]
        nbytes = sum(c[2] for c in h2d)
        busy = _union(civ)
        kbusy = _union(kin)
        ov = _overlap(civ, kin)
        streams = {}
        for c in h2d:
            e = streams.setdefault(c[3], [0, 0, 0])
            e[0] += 1
            e[1] += c[2]
            e[2] += c[1] - c[0]
        lines.append("")
        lines.append(f"layer-stream host-to-device copies (> 4 MB): {len(h2d)} copies, {nbytes / 1e9:.3f} GB, "
                     f"window {(w1 - w0) / 1e6:.1f} ms")
        lines.append(f"- link busy (union of copy intervals): {busy / 1e6:.1f} ms -> {nbytes / max(busy, 1):.1f} GB/s "
                     f"while copying; {nbytes / max(w1 - w0, 1):.1f} GB/s over the window")
        for sid, (n, b, t) in sorted(streams.items()):
            lines.append(f"- stream {sid}: {n} copies, {b / 1e9:.3f} GB, {t / 1e6:.1f} ms of copy time, "
                         f"{b / max(t, 1):.1f} GB/s per copy")
        lines.append(f"- kernels busy inside the window: {kbusy / 1e6:.1f} ms ({100.0 * kbusy / max(w1 - w0, 1):.1f}%)")
        lines.append(f"- copy time overlapped by kernels: {ov / 1e6:.1f} ms = {100.0 * ov / max(busy, 1):.1f}% of link-busy "
                     f"time; kernel time overlapped by copies: {100.0 * ov / max(kbusy, 1):.1f}%")
        lines.append(f"- neither copying nor computing: {(w1 - w0 - busy - kbusy + ov) / 1e6:.1f} ms")
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="sft8b_b1", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="streamed", choices=["streamed", "resident"])
    ap.add_argument("--blob-form", default="wire", choices=["wire", "full"],
                    help="streamed layer blobs: wire = block maxima as bf16 (lossless for bf16 weights, "
                         "widened on the GPU), full = fp32 maxima as the kernels read them")
    ap.add_argument("--keep-layers", default="on", choices=["on", "off"],
                    help="streamed: the two layers a step leaves in the slots serve the next step's forward "
                         "(qlx_ctx_set_keep_layers); off copies every layer every step")
    ap.add_argument("--source", default="ram", choices=["ram", "disk", "auto"],
                    help="where the streamed stack lives: pinned host RAM, a stack file read with O_DIRECT, or "
                         "RAM when it fits in available memory and the file otherwise")
    ap.add_argument("--stack-file", default=None,
                    help="stack file for --source disk/auto (default: a file in the temp directory, removed at exit)")
    ap.add_argument("--dpo-ref", default="fused", choices=["fused", "separate"],
                    help="DPO reference schedule: fused with the policy forward, or a separate pass")
    ap.add_argument("--act", default="f16", choices=["f16", "bf16"],
                    help="16-bit type of activations and gradients between kernels and in the MFMA products (the "
                         "weight operand is bf16 of its NF4 value either way): f16 (10 significand bits, meets the "
                         "2e-2 gradient tolerance at 32 layers) or bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--optimizer", default="fused", choices=["fused", "separate"],
                    help="AdamW on the adapters: fused = each layer updated inside the step right after its "
                         "backward (qlx_ctx_set_adamw), separate = one qlx_adamw_lora call after the step")
    ap.add_argument("--no-optimizer", action="store_true",
                    help="leave the AdamW update out of the step (loss + LoRA gradients only)")
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="only time the 8B-shaped NF4 GEMMs (fwd and dX) at 512 and 2048 tokens")
    ap.add_argument("--merge-shapes", action="store_true",
                    help="only time the adapter merge of one 8B-shaped layer's seven projections (bf16 and NF4 out)")
    ap.add_argument("--cpu-baseline-detail", action="store_true",
                    help="only time the oracle on this host: tiny SFT step and one 8B layer, all threads and one")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the device's peaks: bf16 MFMA loop, HBM copy, 122.7 MB pinned H2D copy")
    ap.add_argument("--rocpd-summary", default=None, metavar="DB",
                    help="only print a summary of a rocprofv3 trace database (kernels; layer-stream copies and "
                         "their overlap with kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        return 2

    if args.rocpd_summary:
        print(rocpd_summary(args.rocpd_summary))
        return 0

    import numpy as np

    if args.cpu_baseline_detail:
        print(json.dumps({"cpu_baseline_detail": cpu_baseline_detail()}))
        return 0
    import torch

    if args.copy_calibration:
        n = 1 << 29  # 2^29 bf16 = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 2 * n, "bytes_written_per_copy": 2 * n,
                                               "copies": 5}}))
        return 0

    import qlora_fine_tuning_dequant_amd as q
    import synth
    B_ = q.binding
    if args.gemm_shapes:
        print(json.dumps({"gemm_shapes": gemm_shapes(q)}))
        return 0
    if args.merge_shapes:
        print(json.dumps({"merge_shapes": merge_shapes(q)}))
        return 0
    if args.peaks:
        print(json.dumps({"peaks": measure_peaks(q)}))
        return 0
    wl = WORKLOADS[args.workload]
    if wl["kind"] == "layer":
        print(json.dumps(layer_bench(q, args, wl)))
        return 0
    d = synth.LLAMA8B
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"workload {args.workload}: {wl['name']} ({args.mode})")
    t0 = time.perf_counter()
    wire = args.mode == "streamed" and args.blob_form == "wire"
    act = B_.QLX_ACT_F16 if args.act == "f16" else B_.QLX_ACT_BF16
    m, dev_blobs = build_model(q, d, SEED, want_device_blobs=(args.mode == "resident"), wire=wire, act=act)
    if args.mode == "resident":
        m = m.with_blobs(dev_blobs)
    log(f"model ready in {time.perf_counter() - t0:.1f} s")
    mode = B_.QLX_STREAMED if args.mode == "streamed" else B_.QLX_RESIDENT
    ctx = q.Context(0)
    keep = args.mode == "streamed" and args.keep_layers == "on"
    ctx.set_keep_layers(keep)
    source, layer_file, stack_path = "ram" if args.mode == "streamed" else "device", None, None
    if args.mode == "streamed" and args.source != "ram":
        _, blob_bytes = B_.wire_layout(d) if wire else B_.blob_layout(d)
        if args.source == "auto":
            mode = B_.stream_source_auto(d.n_layers * blob_bytes, reserve_bytes=8 << 30)
        else:
            mode = B_.QLX_STREAMED_DISK
        if mode == B_.QLX_STREAMED_DISK:
            stack_path = args.stack_file or os.path.join(tempfile.gettempdir(), f"qlx_stack_{os.getpid()}.bin")
            t0 = time.perf_counter()
            q.LayerFile.write(stack_path, d, m.blobs, wire=wire)
            log(f"stack file {stack_path}: {d.n_layers} x {blob_bytes / 1e6:.1f} MB written in "
                f"{time.perf_counter() - t0:.1f} s")
            layer_file = q.LayerFile(stack_path, d, wire=wire)
            ctx.set_layer_source(layer_file)
            source = "disk (O_DIRECT)" if layer_file.info()["direct"] else "disk (page cache)"
        log(f"stream source: {source}")
    grads = [q.LoraGrads(l) for l in m.lora]
    # the step's optimizer update: AdamW on every LoRA factor at the pages' lr
    opt = None if args.no_optimizer else q.AdamW(d, m.lora, lr=LR)
    fused_opt = opt is not None and args.optimizer == "fused"
    if fused_opt:  # each layer's adapters updated inside the step, right after its backward
        ctx.set_adamw(opt)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    batch, seq = wl["batch"], wl["seq"]
    if wl["kind"] == "sft":
        toks = torch.from_numpy(synth.tokens(SEED, batch, seq, d.vocab)).to(dev)
        ws = B_.workspace(B_.step_workspace_bytes(d, 0, batch, seq))
        tokens_per_step = batch * seq

        def step():
            q.stream_step_sft(ctx, m, toks, mode, loss, grads, ws)
            if opt and not fused_opt:
                opt.step(grads)
    else:
        pairs = batch
        ch, rj = synth.dpo_pairs(SEED, pairs, seq, wl["prompt"], d.vocab)
        ch, rj = torch.from_numpy(ch).to(dev), torch.from_numpy(rj).to(dev)
        logps = torch.empty(4 * pairs, dtype=torch.float32, device=dev)
        sched = B_.QLX_DPO_REF_FUSED if args.dpo_ref == "fused" else B_.QLX_DPO_REF_SEPARATE
        ws = B_.workspace(B_.step_workspace_bytes(d, 2 if wl["kind"] == "kto" else 1, pairs, seq))
        tokens_per_step = 2 * pairs * seq

        def step():
            if wl["kind"] == "dpo":
                q.stream_step_dpo(ctx, m, ch, rj, wl["prompt"], wl["beta"], mode, sched, loss, logps, grads, ws)
            else:  # ORPO, SimPO, KTO with the readings' hyperparameters
                q.stream_step_pref(ctx, m, wl["kind"], ch, rj, wl["prompt"], mode, loss, logps, grads, ws,
                                   ref_schedule=sched)
            if opt and not fused_opt:
                opt.step(grads)

    for i in range(args.warmup):
        step()
        st = ctx.sync()
        log(f"warmup {i + 1}/{args.warmup}: {st['step_ms']:.1f} ms, loss {loss.item():.4f}")
    torch.cuda.synchronize()
    # the steps are enqueued back to back (the host never waits between them)
    # with no profiling events; the context's statistics are those of the last step
    t_start = time.perf_counter()
    for i in range(args.steps):
        step()
    stats = [ctx.sync()]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = 1000.0 * elapsed / args.steps
    value = tokens_per_step * args.steps / elapsed
    log(f"timed {args.steps} steps: {ms_step:.1f} ms/step, {value:.1f} tokens/s, loss {loss.item():.4f}")
    live, prof = {}, {}
    if not args.no_profile:
        # after the timed steps, the same number of steps again (untimed) with
        # events around the NF4 GEMMs only, for the roofline of the dominant one
        B_.profile_begin("gemm_nf4")
        for i in range(args.steps):
            step()
        ctx.sync()
        torch.cuda.synchronize()
        live = B_.profile_end()
        # and one more step with events around every kernel
        B_.profile_begin()
        step()
        ctx.sync()
        torch.cuda.synchronize()
        prof = B_.profile_end()

    if layer_file is not None:
        ctx.set_layer_source(None)
        layer_file.close()
        if args.stack_file is None:
            os.remove(stack_path)
    reads = stats[-1]["layer_reads"]
    h2d_ms = float(np.mean([s["h2d_ms"] for s in stats]))
    h2d_bytes = stats[-1]["h2d_bytes"]
    gemm_ms = sum(v["ms"] for k, v in prof.items() if k.startswith("gemm"))
    gemm_tf = sum(v["flops"] for k, v in prof.items() if k.startswith("gemm"))
    all_kernel_ms = sum(v["ms"] for v in prof.values())
    roofline = None
    if live:
        dom = max(live, key=lambda k: live[k]["ms"])
        p = live[dom]
        ach = p["flops"] / (p["ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(args.workload, args.mode if args.source == "ram" else "disk", dom),
                    "launches": p["launches"], "avg_launch_us": round(1000.0 * p["ms"] / p["launches"], 2),
                    "flops_per_launch": p["flops"] / p["launches"]}
    # per kernel: rate and fraction of the vendor peak that bounds it (MFMA for
    # the products, HBM for the rest; attention at 512 tokens sits near the
    # ridge, so it gets both)
    def fracs(k, v):
        mf = {"mfma_frac": round(v["flops"] / max(v["ms"], 1e-9) / 1e9 / PEAK_BF16_TFLOPS, 4)}
        hb = {"hbm_frac": round(v["bytes"] / max(v["ms"], 1e-9) / 1e6 / 8000.0, 4)}
        if k.startswith(("attn_fwd", "attn_bwd_kv", "attn_bwd_q")):
            return {**mf, **hb}
        return mf if k.startswith("gemm") else hb

    kernels = {k: {"launches_per_step": v["launches"], "ms_per_step": round(v["ms"], 3),
                   "TFLOP/s": round(v["flops"] / max(v["ms"], 1e-9) / 1e9, 2),
                   "GB/s": round(v["bytes"] / max(v["ms"], 1e-9) / 1e6, 1), **fracs(k, v)}
               for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"])}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.act, "data": "synthetic",
        "config": {"workload": wl["name"], "global_batch": batch if wl["kind"] == "sft" else 2 * batch,
                   "seq_len": seq, "mode": args.mode, "source": source,
                   "activations": args.act, "weight_operand": "bf16 of the NF4 value",
                   "blob_form": "wire" if wire else "full", "keep_layers": keep, "layers": d.n_layers,
                   "lora_r": d.lora_r,
                   "optimizer": None if args.no_optimizer else
                   f"adamw lr {LR}" + (", per layer inside the backward" if fused_opt else ", after the step"),
                   **({"dpo_reference": args.dpo_ref} if wl["kind"] in ("dpo", "kto") else {})},
        "roofline": roofline,
        "stream": {"layer_reads_per_step": reads, "h2d_GB_per_step": round(h2d_bytes / 1e9, 3),
                   "h2d_ms_per_step": round(h2d_ms, 2),
                   "h2d_GBps": round(h2d_bytes / max(h2d_ms, 1e-9) / 1e6, 1) if h2d_ms else None,
                   **({"disk_GB_per_step": round(stats[-1]["disk_bytes"] / 1e9, 3),
                       "disk_read_ms_per_step": round(float(np.mean([s["disk_ms"] for s in stats])), 1),
                       "disk_GBps": round(stats[-1]["disk_bytes"] / max(float(np.mean([s["disk_ms"] for s in stats])),
                                                                        1e-9) / 1e6, 1)}
                      if layer_file is not None else {})},
        "gpu_time": {"kernels_ms_per_step": round(all_kernel_ms, 2), "gemm_ms_per_step": round(gemm_ms, 2),
                     "gemm_TFLOP_per_step": round(gemm_tf / 1e12, 3),
                     "gemm_TFLOPs_avg": round(gemm_tf / max(gemm_ms, 1e-9) / 1e9, 1)},
        "peak_vram_GB": round(torch.cuda.max_memory_allocated() / 1e9, 3),
        "kernels": kernels,
        "loss": float(loss.item()),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        del ws
        out["cpu_baseline"] = cpu_baseline(d, wl["batch"] if wl["kind"] == "sft" else 2 * wl["batch"], seq)
        log(f"cpu baseline: {out['cpu_baseline']['value']} tokens/s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
