"""GPU parity of NF4 quantize/dequant (bit-exact) and the QLoRA linear
(fused NF4-dequant MFMA GEMM + LoRA slab) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, bf16_dev, f32_dev, to_np
from helpers import rel_l2

pytestmark = pytest.mark.gpu
q = pytest.importorskip("qlora_fine_tuning_dequant_amd")

TOL = 2e-2


def _w_bits(rows, cols, seed, std=0.02):
    return synth.to_bf16_bits(synth._normal_f32(rows * cols, std, seed, 99, rows, cols)).reshape(rows, cols)


@pytest.mark.parametrize("rows,cols", [(1, 64), (3, 40), (5, 13), (256, 688), (688, 256), (1, 1), (7, 64 * 5 + 3),
                                       (1024, 4096), (4096, 14336)])
def test_nf4_quantize_and_dequant_bit_exact(rows, cols):
    wb = _w_bits(rows, cols, rows * 31 + cols)
    w = bf16_dev(wb)
    n = rows * cols
    packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=DEV)
    q.nf4_quantize(w, packed, absmax)
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    assert np.array_equal(to_np(packed), p_ref)
    assert np.array_equal(to_np(absmax).view(np.uint32), a_ref.view(np.uint32))
    out32 = torch.empty(n, dtype=torch.float32, device=DEV)
    out16 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    q.nf4_dequant(packed, absmax, rows, cols, out32)
    q.nf4_dequant(packed, absmax, rows, cols, out16)
    d_ref = oracle.nf4_dequant(p_ref, a_ref, n)
    assert np.array_equal(to_np(out32).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(out16.view(torch.int16).cpu().numpy().view(np.uint16), oracle.bf16_rne_bits(d_ref))


@pytest.mark.parametrize("n", [64 * 40, 64 * 40 + 21])
def test_nf4_quantize_unaligned_buffers_bit_exact(n):
    """Inputs and codes at odd offsets take the element-wise path (no 16-B
    loads or 4-B stores): same codes and scales as the oracle."""
    wb = _w_bits(1, n, 7 + n).reshape(-1)
    w_full = torch.zeros(n + 1, dtype=torch.bfloat16, device=DEV)
    w_full[1:] = bf16_dev(wb)
    w = w_full[1:]                                            # 2-B aligned only
    p_full = torch.zeros((n + 1) // 2 + 1, dtype=torch.uint8, device=DEV)
    packed = p_full[1:]                                       # odd address
    absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=DEV)
    q.nf4_quantize(w, packed, absmax)
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    assert np.array_equal(to_np(packed), p_ref)
    assert np.array_equal(to_np(absmax).view(np.uint32), a_ref.view(np.uint32))
    assert int(p_full[0]) == 0


def test_nf4_special_blocks_bit_exact():
    c = oracle.nf4_codebook()
    rows = []
    for k in (-20, 0, 7):  # every code at a power-of-two scale round-trips exactly
        blk = np.full(64, c[3], np.float32)
        blk[:16] = c
        rows.append(blk * np.float32(2.0 ** k))
    rows.append(np.zeros(64, np.float32))                     # all-zero block
    rows.append(np.concatenate([np.full(32, 0.5, np.float32), np.full(32, -1e-30, np.float32)]))
    mids = oracle.nf4_midpoints()
    blk = np.zeros(64, np.float32)
    blk[0] = 1.0
    blk[1:16] = mids                                          # exact midpoints go to the lower code
    rows.append(blk)
    w = np.concatenate(rows)
    wb = oracle.bf16_rne_bits(w)
    # keep exact bf16 representability for the midpoint case by comparing on the rounded values
    wf = synth.bf16_bits_to_f32(wb)
    packed = torch.empty(w.size // 2, dtype=torch.uint8, device=DEV)
    absmax = torch.empty(w.size // 64, dtype=torch.float32, device=DEV)
    q.nf4_quantize(bf16_dev(wb).view(1, -1), packed, absmax)
    p_ref, a_ref = oracle.nf4_quantize(wf)
    assert np.array_equal(to_np(packed), p_ref) and np.array_equal(to_np(absmax), a_ref)


def _oracle_linear(xb, W_deq, A, B, s):
    return oracle.qlora_linear_fwd(synth.bf16_bits_to_f32(xb), W_deq, A, B, s)


# (T, in, out, r): ragged tails in every dimension, the tiny workload's down
# projection (blocks straddle rows), and 8B-shaped q / down projections.
# (256, 384, 640, 8): full-tile kernel both ways, 6 and 10 K chunks (the
# pipeline runs in steps of three); (256, 1216, 384, 8): split-K into 10 + 9
# chunks; (512, 256, 16640, 8) forward and (512, 16640, 256, 8) dX: 260
# tiles of 256 x 128 (two rounds), so the 512 x 128 tile runs them; the
# 4096 / 14336 shapes split-K an 8B-width projection.
SHAPES = [(64, 256, 512, 8), (37, 688, 256, 8), (200, 256, 1376, 16), (130, 96, 200, 4),
          (256, 384, 640, 8), (256, 1216, 384, 8), (512, 256, 16640, 8), (512, 16640, 256, 8),
          (512, 4096, 4096, 64), (512, 14336, 4096, 64)]


@pytest.mark.parametrize("T,in_f,out_f,r", SHAPES)
def test_qlora_linear_fwd_bwd_vs_oracle(T, in_f, out_f, r):
    seed = T + in_f + out_f
    wb = _w_bits(out_f, in_f, seed)
    W = q.NF4Matrix.quantize(bf16_dev(wb))
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    Wd = oracle.nf4_dequant(p_ref, a_ref, out_f * in_f).reshape(out_f, in_f)
    xb = synth.activations_bf16(seed, T, in_f, 0)
    dyb = synth.activations_bf16(seed, T, out_f, 1)
    g = np.random.default_rng(seed)
    A = (g.uniform(-1, 1, (r, in_f)) / np.sqrt(in_f)).astype(np.float32)
    B = (g.standard_normal((out_f, r)) * 0.05).astype(np.float32)
    s = 16.0 / r
    x, dy = bf16_dev(xb), bf16_dev(dyb)
    y = torch.empty(T, out_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_fwd(x, W, f32_dev(A), f32_dev(B), s, y)
    y_ref, u_ref = _oracle_linear(xb, Wd, A, B, s)
    assert rel_l2(to_np(y), y_ref) < TOL
    dx = torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV)
    dA = torch.empty(r, in_f, dtype=torch.float32, device=DEV)
    dB = torch.empty(out_f, r, dtype=torch.float32, device=DEV)
    q.qlora_linear_bwd(dy, x, W, f32_dev(A), f32_dev(B), s, dx, dA, dB)
    dx_ref, dA_ref, dB_ref = oracle.qlora_linear_bwd(synth.bf16_bits_to_f32(dyb), synth.bf16_bits_to_f32(xb), u_ref,
                                                     Wd, A, B, s)
    assert rel_l2(to_np(dx), dx_ref) < TOL
    assert rel_l2(to_np(dA), dA_ref) < TOL
    assert rel_l2(to_np(dB), dB_ref) < TOL
    # accumulate adds onto what is there
    q.qlora_linear_bwd(dy, x, W, f32_dev(A), f32_dev(B), s, None, dA, dB, accumulate=True)
    assert rel_l2(to_np(dA), 2 * dA_ref) < TOL and rel_l2(to_np(dB), 2 * dB_ref) < TOL


# (256, 512, 256, 8): full-tile kernel with a slab that is not a whole K chunk
@pytest.mark.parametrize("T,in_f,out_f,r", [(64, 256, 512, 8), (256, 512, 256, 8), (256, 384, 640, 8),
                                           (512, 256, 16640, 8), (512, 16640, 256, 8), (512, 4096, 4096, 64)])
def test_lora_zero_B_is_bit_exact_base_and_lora_off(T, in_f, out_f, r):
    wb = _w_bits(out_f, in_f, 5)
    W = q.NF4Matrix.quantize(bf16_dev(wb))
    x = bf16_dev(synth.activations_bf16(5, T, in_f, 0))
    A = f32_dev(np.random.default_rng(0).standard_normal((r, in_f)).astype(np.float32))
    B0 = torch.zeros(out_f, r, dtype=torch.float32, device=DEV)
    y0 = torch.empty(T, out_f, dtype=torch.bfloat16, device=DEV)
    y_off = torch.empty_like(y0)
    q.qlora_linear_fwd(x, W, A, B0, 2.0, y0)
    q.qlora_linear_fwd(x, W, None, None, 2.0, y_off)
    assert torch.equal(y0.view(torch.int16), y_off.view(torch.int16))
    # and in the backward dX GEMM (slab du . A with B = 0 adds exact zeros)
    dy = bf16_dev(synth.activations_bf16(6, T, out_f, 1))
    dx0, dx_off = torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV), torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV)
    dA = torch.empty(r, in_f, dtype=torch.float32, device=DEV)
    dB = torch.empty(out_f, r, dtype=torch.float32, device=DEV)
    q.qlora_linear_bwd(dy, x, W, A, B0, 2.0, dx0, dA, dB)
    q.qlora_linear_bwd(dy, x, W, None, None, 2.0, dx_off, None, None)
    assert torch.equal(dx0.view(torch.int16), dx_off.view(torch.int16))
    # and the base itself matches the oracle
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    Wd = oracle.nf4_dequant(p_ref, a_ref, out_f * in_f).reshape(out_f, in_f)
    y_ref = synth.bf16_bits_to_f32(synth.activations_bf16(5, T, in_f, 0)) @ Wd.T
    assert rel_l2(to_np(y_off), y_ref) < TOL


def test_empty_inputs():
    """Zero elements / zero tokens: quantize and dequant leave their outputs
    alone, the forward writes nothing, and the backward's empty sums over the
    tokens give dA = dB = +0.0 exactly (accumulating leaves them unchanged)."""
    packed = torch.full((4,), 0xAB, dtype=torch.uint8, device=DEV)
    absmax = torch.full((2,), 3.0, dtype=torch.float32, device=DEV)
    q.nf4_quantize(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), packed, absmax)
    out = torch.full((8,), 5.0, dtype=torch.float32, device=DEV)
    q.nf4_dequant(packed, absmax, 0, 64, out)
    torch.cuda.synchronize()
    assert (packed == 0xAB).all() and (absmax == 3.0).all() and (out == 5.0).all()

    out_f, in_f, r = 256, 512, 8
    W = q.NF4Matrix.quantize(bf16_dev(_w_bits(out_f, in_f, 3)))
    g = np.random.default_rng(3)
    A = f32_dev(g.standard_normal((r, in_f)).astype(np.float32))
    B = f32_dev(g.standard_normal((out_f, r)).astype(np.float32))
    x = torch.empty(0, in_f, dtype=torch.bfloat16, device=DEV)
    dy = torch.empty(0, out_f, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(0, out_f, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(0, in_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_fwd(x, W, A, B, 2.0, y)
    dA = torch.full((r, in_f), float("nan"), dtype=torch.float32, device=DEV)
    dB = torch.full((out_f, r), float("nan"), dtype=torch.float32, device=DEV)
    q.qlora_linear_bwd(dy, x, W, A, B, 2.0, dx, dA, dB)
    torch.cuda.synchronize()
    assert (dA.view(torch.int32) == 0).all() and (dB.view(torch.int32) == 0).all()
    dA.fill_(1.5)
    dB.fill_(-2.5)
    q.qlora_linear_bwd(dy, x, W, A, B, 2.0, None, dA, dB, accumulate=True)
    torch.cuda.synchronize()
    assert (dA == 1.5).all() and (dB == -2.5).all()


def test_linear_dequant_operand_is_exactly_bf16_of_dequant():
    """A one-hot input row selects a weight column, so y = bf16(W'[:, j]) exactly."""
    out_f, in_f = 256, 512
    wb = _w_bits(out_f, in_f, 9)
    W = q.NF4Matrix.quantize(bf16_dev(wb))
    xb = np.zeros((16, in_f), np.float32)
    for i in range(16):
        xb[i, i * 31] = 1.0
    x = bf16_dev(oracle.bf16_rne_bits(xb))
    y = torch.empty(16, out_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_fwd(x, W, None, None, 1.0, y)
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    Wd = oracle.nf4_dequant(p_ref, a_ref, out_f * in_f).reshape(out_f, in_f)
    expect = oracle.bf16_rne_bits(np.stack([Wd[:, i * 31] for i in range(16)]))
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), expect)


# Every full-tile NF4 kernel shape (QLX_NF4_TILE pins it; by default a cost
# model picks one) on 8B-width projections at 512 and 1024 tokens, forward and
# dX with the LoRA slab, against the oracle; and the one-hot check that the
# weight operand is exactly bf16 of the dequantized value.
@pytest.mark.parametrize("tile", ["256x128", "512x128", "512x64"])
@pytest.mark.parametrize("T,in_f,out_f,r", [(512, 4096, 6144, 64), (1024, 14336, 4096, 64), (512, 4096, 28672, 64),
                                           (1024, 4096, 4096, 64)])
def test_each_nf4_tile_shape_vs_oracle(monkeypatch, tile, T, in_f, out_f, r):
    monkeypatch.setenv("QLX_NF4_TILE", tile)
    seed = T + in_f + out_f + 7
    wb = _w_bits(out_f, in_f, seed)
    W = q.NF4Matrix.quantize(bf16_dev(wb))
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    Wd = oracle.nf4_dequant(p_ref, a_ref, out_f * in_f).reshape(out_f, in_f)
    xb = synth.activations_bf16(seed, T, in_f, 0)
    dyb = synth.activations_bf16(seed, T, out_f, 1)
    g = np.random.default_rng(seed)
    A = (g.uniform(-1, 1, (r, in_f)) / np.sqrt(in_f)).astype(np.float32)
    B = (g.standard_normal((out_f, r)) * 0.05).astype(np.float32)
    s = 16.0 / r
    x, dy = bf16_dev(xb), bf16_dev(dyb)
    y = torch.empty(T, out_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_fwd(x, W, f32_dev(A), f32_dev(B), s, y)
    y_ref, u_ref = _oracle_linear(xb, Wd, A, B, s)
    dx = torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV)
    dA = torch.empty(r, in_f, dtype=torch.float32, device=DEV)
    dB = torch.empty(out_f, r, dtype=torch.float32, device=DEV)
    q.qlora_linear_bwd(dy, x, W, f32_dev(A), f32_dev(B), s, dx, dA, dB)
    dx_ref, _, _ = oracle.qlora_linear_bwd(synth.bf16_bits_to_f32(dyb), synth.bf16_bits_to_f32(xb), u_ref, Wd, A, B, s)
    print(tile, T, in_f, out_f, "y", rel_l2(to_np(y), y_ref), "dx", rel_l2(to_np(dx), dx_ref), flush=True)
    assert rel_l2(to_np(y), y_ref) < TOL and rel_l2(to_np(dx), dx_ref) < TOL
    # B = 0 equals LoRA off bit for bit on this kernel too
    y0, y_off = torch.empty_like(y), torch.empty_like(y)
    q.qlora_linear_fwd(x, W, f32_dev(A), torch.zeros(out_f, r, dtype=torch.float32, device=DEV), s, y0)
    q.qlora_linear_fwd(x, W, None, None, s, y_off)
    assert torch.equal(y0.view(torch.int16), y_off.view(torch.int16))


@pytest.mark.parametrize("tile", ["256x128", "512x128", "512x64"])
def test_each_nf4_tile_operand_is_bf16_of_dequant(monkeypatch, tile):
    """One-hot rows at 512 tokens (full-tile kernels): forward y row i =
    bf16(W'[:, j_i]) exactly, and dX row i = bf16(W'[j_i, :]) exactly."""
    monkeypatch.setenv("QLX_NF4_TILE", tile)
    out_f, in_f, T = 1024, 2048, 512
    wb = _w_bits(out_f, in_f, 11)
    W = q.NF4Matrix.quantize(bf16_dev(wb))
    p_ref, a_ref = oracle.nf4_quantize(synth.bf16_bits_to_f32(wb))
    Wd = oracle.nf4_dequant(p_ref, a_ref, out_f * in_f).reshape(out_f, in_f)
    jx = (np.arange(T) * 37) % in_f
    xb = np.zeros((T, in_f), np.float32)
    xb[np.arange(T), jx] = 1.0
    y = torch.empty(T, out_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_fwd(bf16_dev(oracle.bf16_rne_bits(xb)), W, None, None, 1.0, y)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), oracle.bf16_rne_bits(Wd[:, jx].T))
    jy = (np.arange(T) * 13) % out_f
    dyb = np.zeros((T, out_f), np.float32)
    dyb[np.arange(T), jy] = 1.0
    dx = torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV)
    q.qlora_linear_bwd(bf16_dev(oracle.bf16_rne_bits(dyb)), bf16_dev(oracle.bf16_rne_bits(xb)), W, None, None, 1.0,
                       dx, None, None)
    assert np.array_equal(dx.view(torch.int16).cpu().numpy().view(np.uint16), oracle.bf16_rne_bits(Wd[jy, :]))


# The 256 x 128 tile has three kernels: the persistent warp-specialized one
# (default), the one-tile-per-workgroup warp-specialized one
# (QLX_NF4_PERSIST=0) and k_nf4_tile (QLX_NF4_WS=0). Same operand values, MFMA
# order and output arithmetic under the same split, so forward, dX and the
# LoRA gradients agree bit for bit, split or not, one tile per workgroup or
# several (2048 x 6144: 384 tiles on 256 workgroups). The persistent kernel's
# edge cases: one K chunk per tile plus its slab chunk (in 64), two K chunks
# per tile over 512 tiles (only the general per-chunk path runs: the tight
# loop needs four chunks of lookahead inside a tile), and a rank whose slab
# is not a whole number of 64-wide chunks (r 16: the one-tile kernel runs).
@pytest.mark.parametrize("T,in_f,out_f,r", [(512, 4096, 4096, 64), (2048, 4096, 6144, 64), (512, 14336, 4096, 64),
                                            (256, 64, 8192, 64), (512, 128, 32768, 64), (512, 4096, 4096, 16)])
def test_warp_specialized_tile_equals_plain_tile(monkeypatch, T, in_f, out_f, r):
    monkeypatch.setenv("QLX_NF4_TILE", "256x128")
    seed = T + in_f + 3 * out_f
    W = q.NF4Matrix.quantize(bf16_dev(_w_bits(out_f, in_f, seed)))
    x = bf16_dev(synth.activations_bf16(seed, T, in_f, 0))
    dy = bf16_dev(synth.activations_bf16(seed, T, out_f, 1))
    g = np.random.default_rng(seed)
    A = f32_dev((g.uniform(-1, 1, (r, in_f)) / np.sqrt(in_f)).astype(np.float32))
    B = f32_dev((g.standard_normal((out_f, r)) * 0.05).astype(np.float32))
    res = {}
    for ws, persist in (("1", "1"), ("1", "0"), ("0", "1")):
        monkeypatch.setenv("QLX_NF4_WS", ws)
        monkeypatch.setenv("QLX_NF4_PERSIST", persist)
        y = torch.empty(T, out_f, dtype=torch.bfloat16, device=DEV)
        dx = torch.empty(T, in_f, dtype=torch.bfloat16, device=DEV)
        dA = torch.empty(r, in_f, dtype=torch.float32, device=DEV)
        dB = torch.empty(out_f, r, dtype=torch.float32, device=DEV)
        q.qlora_linear_fwd(x, W, A, B, 0.25, y)
        q.qlora_linear_bwd(dy, x, W, A, B, 0.25, dx, dA, dB)
        res[ws + persist] = (y, dx, dA, dB)
    for other in ("10", "01"):
        for a, b in zip(res["11"], res[other]):
            assert torch.equal(a, b), other
