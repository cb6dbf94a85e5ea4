"""Full-size GPU checks on Llama-3.1-8B-shaped layers (hidden 4096, 32/8
heads, head_dim 128, SwiGLU 14336, vocab 128256, LoRA r 64 alpha 16):

* streamed and resident runs of the 32-layer model at batch 4 x seq 512 give
  the same loss and LoRA gradients bit for bit (the pages' "difference 0.0"),
  with 2L-2 layer reads and a loss near its closed form at initialization;
* at full width with 2 layers (so the oracle finishes in seconds), streamed
  SFT and DPO steps match the oracle, DPO with B = 0 gives exactly ln 2, and
  the fused and separate reference schedules give identical bits."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import gpu_model, grad_errors, run_dpo, run_sft, same_grads, to_np
from helpers import lora_list, oracle_model

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")
B_ = q.binding
# bf16 activations at hidden 4096 cost about 0.6-0.9% rel-L2 per layer (the
# single-layer 8B test); errors add along the residual stream, so a 2-layer
# full-width step is held to 3e-2 on every LoRA gradient.
TOL2 = 3e-2
# DPO: each summed log-prob (|lp| ~ 600 here) carries the bf16 activation
# error, measured below 4e-4 relative; Delta combines four of them and the loss
# moves by beta/2 per unit Delta near Delta = 0, so
# |dloss| <= beta/2 * 4 * 4e-4 * max|lp|.
LP_REL = 4e-4


def test_llama8b_32_layers_batch4_streamed_equals_resident():
    d = synth.LLAMA8B
    m, host = gpu_model(q, d, 1, "kaiming")
    toks = synth.tokens(1, 4, 512, d.vocab)
    loss_s, g_s, st_s = run_sft(q, m.with_blobs(host), toks, B_.QLX_STREAMED)
    loss_r, g_r, st_r = run_sft(q, m, toks, B_.QLX_RESIDENT)
    assert torch.equal(loss_s, loss_r) and same_grads(g_s, g_r)
    assert st_s["layer_reads"] == 2 * d.n_layers - 2 and st_r["layer_reads"] == 0
    # logits z = n . w, n of unit RMS, w ~ N(0, 0.02^2): E[loss] ~ ln V + 0.02^2 H / 2
    closed = np.log(d.vocab) + 0.02 ** 2 * d.hidden / 2
    assert abs(loss_s.item() - closed) < 0.05, (loss_s.item(), closed)
    assert all(torch.isfinite(t).all() for g in g_s for t in g.dA + g.dB)


@pytest.fixture(scope="module")
def wide2():
    d = dataclasses.replace(synth.LLAMA8B, n_layers=2)
    m, host = gpu_model(q, d, 3, "kaiming")
    return d, m, host, oracle_model(d, 3), lora_list(d, 3, "kaiming")


def test_llama8b_width_sft_step_vs_oracle(wide2):
    d, m, host, om, ol = wide2
    toks = synth.tokens(3, 1, 64, d.vocab)
    loss, g, st = run_sft(q, m.with_blobs(host), toks, B_.QLX_STREAMED)
    ref_loss, ref_g = oracle.sft_step(om, ol, toks, d)
    assert abs(loss.item() - ref_loss) < 1e-2, (loss.item(), ref_loss)
    errs = grad_errors(g, ref_g)
    print({k: f"{v:.1e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v < TOL2}
    assert not bad, bad


def test_llama8b_width_dpo_vs_oracle_and_schedules(wide2):
    d, m, host, om, ol = wide2
    ch, rj = synth.dpo_pairs(3, 2, 64, 16, d.vocab)
    sm = m.with_blobs(host)
    l_f, lp_f, g_f, st_f = run_dpo(q, sm, ch, rj, 16, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_FUSED)
    l_s, lp_s, g_s, st_s = run_dpo(q, sm, ch, rj, 16, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE)
    assert torch.equal(l_f, l_s) and torch.equal(lp_f, lp_s) and same_grads(g_f, g_s)
    assert st_f["layer_reads"] == 2 * 2 - 2 and st_s["layer_reads"] == 3 * 2 - 2
    ref_loss, ref_lp, ref_g = oracle.dpo_step(om, ol, ch, rj, 16, 0.1, d)
    lp = to_np(lp_f)
    assert np.all(np.abs(lp - ref_lp) <= LP_REL * np.abs(ref_lp)), (lp, ref_lp)
    bound = 0.1 / 2 * 4 * LP_REL * np.max(np.abs(ref_lp))
    assert abs(l_f.item() - ref_loss) <= bound, (l_f.item(), ref_loss, bound)
    bad = {k: v for k, v in grad_errors(g_f, ref_g).items() if not v < TOL2}
    assert not bad, bad


def test_llama8b_width_dpo_zero_adapter_is_exactly_ln2():
    d = dataclasses.replace(synth.LLAMA8B, n_layers=2)
    m, host = gpu_model(q, d, 4, "zeroB")
    ch, rj = synth.dpo_pairs(4, 2, 64, 16, d.vocab)
    loss, logps, _, _ = run_dpo(q, m.with_blobs(host), ch, rj, 16, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_FUSED)
    lp = to_np(logps)
    assert np.array_equal(lp[:4], lp[4:])
    assert loss.item() == float(np.float32(np.log(2.0)))
