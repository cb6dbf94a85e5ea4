"""GPU parity of one decoder layer (forward and backward through the C ABI)
against the oracle: the tiny workload, a ragged batch, and one
Llama-3.1-8B-shaped layer at batch 1, sequence 512."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, device_blob, f32_dev, lora_layer, oracle_lora, to_np
from helpers import oracle_model, rel_l2
from synth import PROJ_NAMES

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")
TOL = 2e-2


def _run(d, seed, batch, seq, lora_init, random_gamma=False, x_scale=1.0):
    blob = device_blob(q, d, seed, 0, random_gamma=random_gamma)
    lo = lora_layer(q, d, seed, 0, lora_init)
    T = batch * seq
    h = synth.activations_f32(seed, T, d.hidden, 0) * np.float32(x_scale)
    dh = synth.activations_f32(seed, T, d.hidden, 1)
    h_in, dh_out = f32_dev(h), f32_dev(dh)
    h_out = torch.empty_like(h_in)
    ws = q.binding.workspace(q.binding.layer_workspace_bytes(d, batch, seq))
    q.layer_fwd(d, blob, lo, h_in, batch, seq, h_out, ws)
    grads = q.LoraGrads(lo)
    dh_in = torch.empty_like(h_in)
    q.layer_bwd(d, blob, lo, h_in, dh_out, batch, seq, dh_in, grads, ws)
    torch.cuda.synchronize()
    # oracle
    m = oracle_model(dataclass_one_layer(d), seed, random_gamma=random_gamma)
    W = oracle.dequant_layer(m["layers"][0]["nf4"], d)
    L = oracle_lora(lo)
    out_ref, cache = oracle.layer_fwd(h, W, m["layers"][0]["g1"], m["layers"][0]["g2"], L, d, batch, seq, keep=True)
    dh_ref, g_ref = oracle.layer_bwd(dh, W, m["layers"][0]["g1"], m["layers"][0]["g2"], L, d, batch, seq, cache)
    res = {"out": rel_l2(to_np(h_out), out_ref), "dh": rel_l2(to_np(dh_in), dh_ref)}
    # the residual carries h through; compare the layer's own contribution too
    res["delta"] = rel_l2(to_np(h_out) - h, out_ref - h)
    res["ddelta"] = rel_l2(to_np(dh_in) - dh, dh_ref - dh)
    for i, p in enumerate(PROJ_NAMES):
        res["dA_" + p] = rel_l2(to_np(grads.dA[i]), g_ref[p][0])
        res["dB_" + p] = rel_l2(to_np(grads.dB[i]), g_ref[p][1])
    return res


def dataclass_one_layer(d):
    import dataclasses
    return dataclasses.replace(d, n_layers=1)


@pytest.mark.parametrize("batch,seq,random_gamma", [(1, 64, False), (2, 48, True), (3, 17, False)])
def test_tiny_layer_vs_oracle(batch, seq, random_gamma):
    res = _run(synth.TINY, 0, batch, seq, "normal", random_gamma)
    bad = {k: v for k, v in res.items() if not v < TOL}
    assert not bad, (bad, res)


@pytest.mark.parametrize("hidden,inter,r", [(1024, 2816, 8), (2048, 5464, 16), (3072, 8196, 12)])
def test_mid_width_layer_vs_oracle(hidden, inter, r):
    """Hidden sizes 1024, 2048 and 3072 (each register-resident RMSNorm width);
    intermediate sizes that are (2816, 5464) and are not (8196) a multiple of
    8, and LoRA ranks that are (8, 16) and are not (12): both paths of the
    SwiGLU and adapter-packing kernels."""
    import dataclasses
    d = dataclasses.replace(synth.TINY, hidden=hidden, n_heads=hidden // 128, n_kv_heads=2, head_dim=128,
                            inter=inter, n_layers=1, lora_r=r)
    res = _run(d, 4, 1, 40, "normal")
    bad = {k: v for k, v in res.items() if not v < TOL}
    assert not bad, (bad, res)


def test_llama8b_layer_vs_oracle():
    """One Llama-3.1-8B-shaped layer, batch 1, seq 512 (full size)."""
    res = _run(synth.LLAMA8B_LAYER, 2, 1, 512, "kaiming")
    print({k: f"{v:.2e}" for k, v in res.items()})
    bad = {k: v for k, v in res.items() if not v < TOL}
    assert not bad, (bad, res)


def test_layer_fwd_lora_off_equals_zero_B_bit_exact():
    d = synth.TINY
    blob = device_blob(q, d, 3, 0)
    lo = lora_layer(q, d, 3, 0, "zeroB")
    h = f32_dev(synth.activations_f32(3, 64, d.hidden, 0))
    a, b = torch.empty_like(h), torch.empty_like(h)
    q.layer_fwd(d, blob, lo, h, 1, 64, a)
    q.layer_fwd(d, blob, None, h, 1, 64, b)
    assert torch.equal(a, b)
