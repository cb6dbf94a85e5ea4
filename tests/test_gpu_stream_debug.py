"""Fault injection on the layer stream: the one race the streamer can have is
a copy overwriting a slot that a kernel still reads. Serializing everything,
poisoning every freed slot with NaN bytes before it is refilled, and delaying
the copies or the compute must all leave the loss and every gradient
identical to the normal run; poisoning the live slot instead (the control)
must show up as NaN."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import gpu_model, run_dpo, run_sft, same_grads

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")
B_ = q.binding


@pytest.fixture(scope="module")
def four():
    d = dataclasses.replace(synth.TINY, n_layers=4)
    m, host = gpu_model(q, d, 3, "normal")
    return d, m.with_blobs(host)


MODES = [
    ("serialize", B_.QLX_DEBUG_SERIALIZE, 0),
    ("poison", B_.QLX_DEBUG_POISON, 0),
    ("poison+delay_copy", B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COPY, 300),
    ("poison+delay_compute", B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COMPUTE, 300),
    ("poison+serialize", B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_SERIALIZE, 0),
]


@pytest.mark.parametrize("name,flags,delay", MODES, ids=[m[0] for m in MODES])
def test_sft_under_fault_injection_is_bit_identical(four, name, flags, delay):
    d, sm = four
    toks = synth.tokens(3, 2, 32, d.vocab)
    l0, g0, _ = run_sft(q, sm, toks, B_.QLX_STREAMED)
    ctx = q.Context(0)
    ctx.set_debug(flags, delay)
    print("debug mode", name, flush=True)
    l1, g1, st = run_sft(q, sm, toks, B_.QLX_STREAMED, ctx)
    assert np.isfinite(l1.item())
    assert torch.equal(l0, l1) and same_grads(g0, g1)
    assert st["layer_reads"] == 2 * 4 - 2
    ctx.close()


def test_dpo_separate_reference_under_poison_and_delays(four):
    d, sm = four
    ch, rj = synth.dpo_pairs(3, 2, 32, 8, d.vocab)
    l0, lp0, g0, _ = run_dpo(q, sm, ch, rj, 8, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE)
    for flags in (B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COPY, B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COMPUTE):
        ctx = q.Context(0)
        ctx.set_debug(flags, 300)
        l1, lp1, g1, _ = run_dpo(q, sm, ch, rj, 8, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE, ctx)
        assert torch.equal(l0, l1) and torch.equal(lp0, lp1) and same_grads(g0, g1)
        ctx.close()


def test_one_copy_stream_equals_two(four, monkeypatch):
    """Each layer copy runs in two halves on two streams by default;
    QLX_COPY_SPLIT=1 at context creation keeps one stream: same bits."""
    d, sm = four
    toks = synth.tokens(3, 1, 32, d.vocab)
    l2, g2, _ = run_sft(q, sm, toks, B_.QLX_STREAMED)
    monkeypatch.setenv("QLX_COPY_SPLIT", "1")
    ctx = q.Context(0)
    monkeypatch.delenv("QLX_COPY_SPLIT")
    ctx.set_debug(B_.QLX_DEBUG_POISON)
    l1, g1, _ = run_sft(q, sm, toks, B_.QLX_STREAMED, ctx)
    assert torch.equal(l1, l2) and same_grads(g1, g2)
    ctx.close()


def test_poisoning_the_live_slot_shows_up(four):
    """Control: the poison reaches what the kernels read."""
    d, sm = four
    toks = synth.tokens(3, 1, 32, d.vocab)
    ctx = q.Context(0)
    ctx.set_debug(B_.QLX_DEBUG_POISON_LIVE)
    l1, _, _ = run_sft(q, sm, toks, B_.QLX_STREAMED, ctx)
    assert np.isnan(l1.item())
    ctx.close()


def test_bad_debug_arguments():
    ctx = q.Context(0)
    L = B_.lib()
    assert L.qlx_ctx_set_debug(ctx.h, 64, 0) == B_.QLX_EINVAL
    assert L.qlx_ctx_set_debug(ctx.h, B_.QLX_DEBUG_DELAY_COPY, -1) == B_.QLX_EINVAL
    assert L.qlx_ctx_set_debug(None, 0, 0) == B_.QLX_EINVAL
    assert L.qlx_ctx_set_debug(ctx.h, 0, 0) == B_.QLX_OK
    ctx.close()


@pytest.mark.parametrize("flags", [B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COPY,
                                   B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_DELAY_COMPUTE,
                                   B_.QLX_DEBUG_POISON | B_.QLX_DEBUG_SERIALIZE],
                         ids=["poison+delay_copy", "poison+delay_compute", "poison+serialize"])
def test_wire_form_under_fault_injection(four, flags, monkeypatch):
    """Wire-form blobs: the widen kernel runs on the copy stream between the
    copy and the slot's ready event; a poisoned slot (whole slot, tail
    staging included) still gives the normal bits, with one or two copy
    streams."""
    d, sm = four
    wire = [B_.blob_to_wire(d, h) for h in sm.blobs]
    sw = sm.with_blobs(wire, B_.QLX_BLOB_WIRE)
    toks = synth.tokens(3, 2, 32, d.vocab)
    l0, g0, _ = run_sft(q, sm, toks, B_.QLX_STREAMED)
    for split in ("2", "1"):
        monkeypatch.setenv("QLX_COPY_SPLIT", split)
        ctx = q.Context(0)
        monkeypatch.delenv("QLX_COPY_SPLIT")
        ctx.set_debug(flags, 300)
        print("wire debug", flags, "split", split, flush=True)
        l1, g1, _ = run_sft(q, sw, toks, B_.QLX_STREAMED, ctx)
        assert torch.equal(l0, l1) and same_grads(g0, g1)
        ctx.close()


def test_wire_form_poisoning_the_live_slot_shows_up(four):
    d, sm = four
    sw = sm.with_blobs([B_.blob_to_wire(d, h) for h in sm.blobs], B_.QLX_BLOB_WIRE)
    ctx = q.Context(0)
    ctx.set_debug(B_.QLX_DEBUG_POISON_LIVE)
    l1, _, _ = run_sft(q, sw, synth.tokens(3, 1, 32, d.vocab), B_.QLX_STREAMED, ctx)
    assert np.isnan(l1.item())
    ctx.close()


def _sft_ws(sm, toks, ctx, ws):
    grads = [q.LoraGrads(l) for l in sm.lora]
    loss = torch.empty(1, dtype=torch.float32, device="cuda:0")
    q.stream_step_sft(ctx, sm, torch.from_numpy(toks).to("cuda:0"), B_.QLX_STREAMED, loss, grads, ws)
    return loss, grads, ctx.sync()


def test_keep_layers_across_steps(four):
    """Keep-layers: the second step on the same context, workspace and blobs
    reuses the two layers the first left in the slots (2L - 4 reads instead of
    2L - 2) and gives the same bits; other blobs, another workspace, or the
    setting switched off copy every layer again."""
    d, sm = four
    toks = synth.tokens(3, 2, 32, d.vocab)
    l0, g0, _ = run_sft(q, sm, toks, B_.QLX_STREAMED)
    ws = B_.workspace(B_.step_workspace_bytes(d, 0, 2, 32))
    ctx = q.Context(0)
    ctx.set_keep_layers(True)
    reads = []
    for _ in range(3):
        l1, g1, st = _sft_ws(sm, toks, ctx, ws)
        assert torch.equal(l0, l1) and same_grads(g0, g1)
        reads.append(st["layer_reads"])
    assert reads == [2 * 4 - 2, 2 * 4 - 4, 2 * 4 - 4]
    # the same bytes at other host addresses: copied again
    other = sm.with_blobs([h.clone().pin_memory() for h in sm.blobs])
    l2, g2, st = _sft_ws(other, toks, ctx, ws)
    assert st["layer_reads"] == 2 * 4 - 2 and torch.equal(l0, l2) and same_grads(g0, g2)
    # another workspace: copied again
    ws2 = B_.workspace(B_.step_workspace_bytes(d, 0, 2, 32))
    _, _, st = _sft_ws(other, toks, ctx, ws2)
    assert st["layer_reads"] == 2 * 4 - 2
    # poisoning freed slots does not touch the kept ones
    ctx.set_debug(B_.QLX_DEBUG_POISON)
    l3, g3, st = _sft_ws(other, toks, ctx, ws2)
    assert st["layer_reads"] == 2 * 4 - 4 and torch.equal(l0, l3) and same_grads(g0, g3)
    ctx.set_keep_layers(False)
    _, _, st = _sft_ws(other, toks, ctx, ws2)
    assert st["layer_reads"] == 2 * 4 - 2
    ctx.close()


def test_keep_layers_dpo_and_wire_form(four):
    d, sm = four
    ch, rj = synth.dpo_pairs(3, 2, 32, 8, d.vocab)
    l0, lp0, g0, _ = run_dpo(q, sm, ch, rj, 8, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE)
    sw = sm.with_blobs([B_.blob_to_wire(d, h) for h in sm.blobs], B_.QLX_BLOB_WIRE)
    for model in (sm, sw):
        ws = B_.workspace(B_.step_workspace_bytes(d, 1, 2, 32))
        ctx = q.Context(0)
        ctx.set_keep_layers(True)
        reads = []
        for _ in range(2):
            grads = [q.LoraGrads(l) for l in model.lora]
            loss = torch.empty(1, dtype=torch.float32, device="cuda:0")
            logps = torch.empty(8, dtype=torch.float32, device="cuda:0")
            q.stream_step_dpo(ctx, model, torch.from_numpy(ch).to("cuda:0"), torch.from_numpy(rj).to("cuda:0"), 8,
                              0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE, loss, logps, grads, ws)
            reads.append(ctx.sync()["layer_reads"])
            assert torch.equal(loss, l0) and torch.equal(logps, lp0) and same_grads(grads, g0)
        assert reads == [3 * 4 - 2, 3 * 4 - 4]
        ctx.close()


@pytest.mark.parametrize("form", ["full", "wire"])
def test_split_copies_with_delayed_compute_alone(four, form):
    """The production branch of the split copy (no poison fill): the second
    copy stream waits only for the slot's previous user. With the compute
    delayed by a spin before every layer, a half copy that started before
    that user finished would overwrite weights still being read and change
    the bits; SFT and separate-reference DPO must equal the resident run."""
    d, sm = four
    rm = sm.with_blobs([b.to("cuda:0") for b in sm.blobs])
    model = sm if form == "full" else sm.with_blobs([B_.blob_to_wire(d, h) for h in sm.blobs], B_.QLX_BLOB_WIRE)
    toks = synth.tokens(3, 2, 32, d.vocab)
    l0, g0, _ = run_sft(q, rm, toks, B_.QLX_RESIDENT)
    ch, rj = synth.dpo_pairs(3, 2, 32, 8, d.vocab)
    dl0, dlp0, dg0, _ = run_dpo(q, rm, ch, rj, 8, 0.1, B_.QLX_RESIDENT, B_.QLX_DPO_REF_SEPARATE)
    ctx = q.Context(0)  # default: two copy streams
    ctx.set_debug(B_.QLX_DEBUG_DELAY_COMPUTE, 300)
    print("split copies, delayed compute, form", form, flush=True)
    l1, g1, st = run_sft(q, model, toks, B_.QLX_STREAMED, ctx)
    assert torch.equal(l0, l1) and same_grads(g0, g1) and st["layer_reads"] == 2 * 4 - 2
    dl1, dlp1, dg1, st = run_dpo(q, model, ch, rj, 8, 0.1, B_.QLX_STREAMED, B_.QLX_DPO_REF_SEPARATE, ctx)
    assert torch.equal(dl0, dl1) and torch.equal(dlp0, dlp1) and same_grads(dg0, dg1)
    assert st["layer_reads"] == 3 * 4 - 2
    ctx.close()
