"""GPU checks of the disk stream source: steps whose layers come from a stack
file (disk -> pinned staging -> device slot) match the oracle's SFT and DPO
steps on the same seeded model, give the same bits as the RAM-streamed and
resident runs, read the stack as often, and reject a missing or mismatched
file before any launch."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import grad_errors, gpu_model, run_dpo, run_sft, same_grads, to_np
from helpers import lora_list, oracle_model

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")
B_ = q.binding
# each sequence's summed response log-prob against the oracle's, relative
LP_REL = 1e-3


@pytest.fixture(scope="module")
def four(tmp_path_factory):
    d = dataclasses.replace(synth.TINY, n_layers=4)
    m, host = gpu_model(q, d, 1, "normal")
    path = str(tmp_path_factory.mktemp("stack") / "stack.bin")
    q.LayerFile.write(path, d, host)
    return d, m, host, path


def _disk_model(m):
    return q.StreamModel(m.dims, None, m.embed, m.head, m.final_norm, m.lora)


@pytest.mark.parametrize("buffered", [False, True])
def test_sft_from_disk_equals_ram_and_resident(four, buffered):
    d, m, host, path = four
    toks = synth.tokens(1, 2, 32, d.vocab)
    f = q.LayerFile(path, d, buffered=buffered)
    print("layer file", f.info(), flush=True)
    ctx = q.Context(0)
    ctx.set_layer_source(f)
    l_d, g_d, st_d = run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)
    l_s, g_s, st_s = run_sft(q, m.with_blobs(host), toks, B_.QLX_STREAMED)
    l_r, g_r, _ = run_sft(q, m, toks, B_.QLX_RESIDENT)
    assert torch.equal(l_d, l_s) and same_grads(g_d, g_s)
    assert torch.equal(l_d, l_r) and same_grads(g_d, g_r)
    # and against the oracle's step on the same seeded model
    ref_loss, ref_g = oracle.sft_step(oracle_model(d, 1), lora_list(d, 1, "normal"), toks, d)
    assert abs(l_d.item() - ref_loss) <= 1e-2, (l_d.item(), ref_loss)
    bad = {k: v for k, v in grad_errors(g_d, ref_g).items() if not v <= 2e-2}
    assert not bad, bad
    assert st_d["layer_reads"] == 2 * 4 - 2 and st_d["h2d_bytes"] == st_s["h2d_bytes"]
    assert st_d["disk_bytes"] == st_d["layer_reads"] * f.info()["stride"] and st_s["disk_bytes"] == 0
    # the same context again: the staging ring is reused across steps
    for _ in range(2):
        l2, g2, _ = run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)
        assert torch.equal(l2, l_d) and same_grads(g2, g_d)
    ctx.set_layer_source(None)
    ctx.close()
    f.close()


def test_dpo_from_disk_both_schedules(four):
    d, m, host, path = four
    ch, rj = synth.dpo_pairs(1, 2, 32, 8, d.vocab)
    f = q.LayerFile(path, d)
    ctx = q.Context(0)
    ctx.set_layer_source(f)
    ref_loss, ref_lp, ref_g = oracle.dpo_step(oracle_model(d, 1), lora_list(d, 1, "normal"), ch, rj, 8, 0.1, d)
    for sched, reads in ((B_.QLX_DPO_REF_FUSED, 2 * 4 - 2), (B_.QLX_DPO_REF_SEPARATE, 3 * 4 - 2)):
        l_d, lp_d, g_d, st_d = run_dpo(q, _disk_model(m), ch, rj, 8, 0.1, B_.QLX_STREAMED_DISK, sched, ctx)
        l_s, lp_s, g_s, _ = run_dpo(q, m.with_blobs(host), ch, rj, 8, 0.1, B_.QLX_STREAMED, sched)
        assert torch.equal(l_d, l_s) and torch.equal(lp_d, lp_s) and same_grads(g_d, g_s)
        assert st_d["layer_reads"] == reads and st_d["disk_bytes"] == reads * f.info()["stride"]
        # against the oracle: loss, each sequence's summed log-prob, every gradient
        assert abs(l_d.item() - ref_loss) <= 1e-2, (l_d.item(), ref_loss)
        lp = to_np(lp_d)
        assert np.all(np.abs(lp - ref_lp) <= LP_REL * np.abs(ref_lp)), (lp, ref_lp)
        bad = {k: v for k, v in grad_errors(g_d, ref_g).items() if not v <= 2e-2}
        assert not bad, bad
    ctx.set_layer_source(None)
    ctx.close()
    f.close()


def test_disk_mode_needs_a_matching_file(four, tmp_path):
    d, m, host, path = four
    toks = synth.tokens(1, 1, 32, d.vocab)
    ctx = q.Context(0)
    with pytest.raises(B_.QlxError) as e:        # no file attached
        run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)
    assert e.value.code == B_.QLX_EINVAL and "layer file" in str(e.value)
    d2 = dataclasses.replace(d, n_layers=2)      # a file for a 2-layer stack
    p2 = str(tmp_path / "two.bin")
    q.LayerFile.write(p2, d2, host[:2])
    f2 = q.LayerFile(p2, d2)
    ctx.set_layer_source(f2)
    with pytest.raises(B_.QlxError) as e:
        run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)
    assert e.value.code == B_.QLX_EINVAL and "other model dims" in str(e.value)
    ctx.set_layer_source(None)
    ctx.close()
    f2.close()


def test_attached_file_cannot_be_closed(four):
    d, m, host, path = four
    f = q.LayerFile(path, d)
    ctx = q.Context(0)
    ctx.set_layer_source(f)
    with pytest.raises(B_.QlxError) as e:  # still held by the context: nothing freed
        f.close()
    assert e.value.code == B_.QLX_EINVAL and "attached" in str(e.value)
    toks = synth.tokens(1, 1, 32, d.vocab)
    l_d, _, _ = run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)  # the file still works
    l_s, _, _ = run_sft(q, m.with_blobs(host), toks, B_.QLX_STREAMED)
    assert torch.equal(l_d, l_s)
    ctx.set_layer_source(f)  # attaching the same file twice counts once
    ctx.close()              # a destroyed context releases its file
    f.close()
    g = q.LayerFile(path, d)
    ctx2 = q.Context(0)
    ctx2.set_layer_source(g)
    ctx2.set_layer_source(None)
    g.close()
    ctx2.close()


def test_wire_form_stack_file(four, tmp_path):
    """A stack file of wire-form blobs: SFT and DPO give the resident run's
    bits while reading (and copying) the smaller blobs."""
    d, m, host, path = four
    wire = [B_.blob_to_wire(d, h, pin_memory=False) for h in host]
    wpath = str(tmp_path / "wire.bin")
    q.LayerFile.write(wpath, d, wire, wire=True)
    f = q.LayerFile(wpath, d, wire=True)
    full = q.LayerFile(path, d)
    assert f.info()["stride"] < full.info()["stride"]
    full.close()
    ctx = q.Context(0)
    ctx.set_layer_source(f)
    toks = synth.tokens(1, 2, 32, d.vocab)
    l_d, g_d, st_d = run_sft(q, _disk_model(m), toks, B_.QLX_STREAMED_DISK, ctx)
    l_r, g_r, _ = run_sft(q, m, toks, B_.QLX_RESIDENT)
    assert torch.equal(l_d, l_r) and same_grads(g_d, g_r)
    _, wt = B_.wire_layout(d)
    assert st_d["h2d_bytes"] == st_d["layer_reads"] * wt
    assert st_d["disk_bytes"] == st_d["layer_reads"] * f.info()["stride"]
    ch, rj = synth.dpo_pairs(1, 2, 32, 8, d.vocab)
    l_d, lp_d, g_d, _ = run_dpo(q, _disk_model(m), ch, rj, 8, 0.1, B_.QLX_STREAMED_DISK, B_.QLX_DPO_REF_SEPARATE, ctx)
    l_r, lp_r, g_r, _ = run_dpo(q, m, ch, rj, 8, 0.1, B_.QLX_RESIDENT, B_.QLX_DPO_REF_FUSED)
    assert torch.equal(l_d, l_r) and torch.equal(lp_d, lp_r) and same_grads(g_d, g_r)
    ctx.set_layer_source(None)
    ctx.close()
    f.close()


def test_keep_layers_with_a_layer_file(four):
    """Keep-layers on the disk source: the second step reuses the two slot
    layers; re-attaching a source forgets them (a new file could sit at the
    old one's address)."""
    d, m, host, path = four
    toks = synth.tokens(1, 2, 32, d.vocab)
    l_r, g_r, _ = run_sft(q, m, toks, B_.QLX_RESIDENT)
    f = q.LayerFile(path, d)
    ctx = q.Context(0)
    ctx.set_layer_source(f)
    ctx.set_keep_layers(True)
    ws = B_.workspace(B_.step_workspace_bytes(d, 0, 2, 32))
    dm = _disk_model(m)

    def step():
        grads = [q.LoraGrads(l) for l in dm.lora]
        loss = torch.empty(1, dtype=torch.float32, device="cuda:0")
        q.stream_step_sft(ctx, dm, torch.from_numpy(toks).to("cuda:0"), B_.QLX_STREAMED_DISK, loss, grads, ws)
        st = ctx.sync()
        assert torch.equal(loss, l_r) and same_grads(grads, g_r)
        return st["layer_reads"], st["disk_bytes"]

    r1, b1 = step()
    r2, b2 = step()
    assert (r1, r2) == (2 * 4 - 2, 2 * 4 - 4) and b2 == r2 * f.info()["stride"]
    ctx.set_layer_source(None)
    ctx.set_layer_source(f)
    assert step()[0] == 2 * 4 - 2
    ctx.set_layer_source(None)
    ctx.close()
    f.close()
