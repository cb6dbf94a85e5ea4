"""Pins of the oracle's NF4 quantization against things other than itself:
the published NF4 table, exact round trips, brute-force nearest-value search,
torch's bf16 rounding, and closed-form error bounds."""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_codebook_qlora.txt")


def _golden():
    dec, bits = [], []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        a, b = line.split()
        dec.append(float(a))
        bits.append(int(b, 16))
    return np.array(dec, np.float64), np.array(bits, np.uint32)


def test_codebook_matches_published_table_bit_exact():
    dec, bits = _golden()
    c = oracle.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.array_equal(c.view(np.uint32), bits)
    # the printed decimals are those same float32 values
    assert np.array_equal(dec.astype(np.float32).view(np.uint32), bits)


def test_codebook_structure():
    c = oracle.nf4_codebook()
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert np.all(np.diff(c) > 0)
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8


def test_midpoint_rule_matches_bruteforce_nearest():
    c = oracle.nf4_codebook().astype(np.float64)
    m = oracle.nf4_midpoints().astype(np.float64)
    rng = np.random.default_rng(0)
    x = rng.uniform(-1, 1, 200_000).astype(np.float32)
    x = np.concatenate([x, oracle.nf4_codebook()])
    rule = np.searchsorted(m.astype(np.float32), x, side="left")
    brute = np.argmin(np.abs(x.astype(np.float64)[:, None] - c[None, :]), axis=1)
    near_tie = np.min(np.abs(x.astype(np.float64)[:, None] - m[None, :]), axis=1) < 1e-6
    assert np.array_equal(rule[~near_tie], brute[~near_tie])
    # an exact midpoint goes to the lower code
    for i, mi in enumerate(oracle.nf4_midpoints()):
        w = np.zeros(64, np.float32)
        w[0] = 1.0
        w[1] = mi
        packed, absmax = oracle.nf4_quantize(w)
        codes = nf4.nf4_unpack(packed, 64)
        assert codes[1] == i


@pytest.mark.parametrize("k", [-20, -7, 0, 3, 10])
def test_round_trip_every_code_at_power_of_two_scale(k):
    c = oracle.nf4_codebook()
    scale = np.float32(2.0 ** k)
    w = np.zeros(64, np.float32)
    w[:16] = c * scale
    w[16] = scale  # absmax = 2^k exactly
    w[17:] = c[3] * scale  # any codebook value round-trips exactly
    packed, absmax = oracle.nf4_quantize(w)
    assert absmax[0] == scale
    codes = nf4.nf4_unpack(packed, 64)
    assert np.array_equal(codes[:16], np.arange(16))
    deq = oracle.nf4_dequant(packed, absmax, 64)
    assert np.array_equal(deq, w)


def test_pack_order_high_nibble_is_even_element():
    c = oracle.nf4_codebook()
    w = np.zeros(64, np.float32)
    w[0], w[1], w[2], w[3] = c[15], c[0], c[3], c[12]
    packed, _ = oracle.nf4_quantize(w)
    assert packed[0] == 0xF0 and packed[1] == 0x3C
    assert np.all(packed[2:] == 0x77)


def test_zero_block_and_odd_length():
    w = np.zeros(70, np.float32)
    w[65] = -3.0
    w[69] = 1.5
    packed, absmax = oracle.nf4_quantize(w[:69])  # odd length, partial last block
    assert packed.size == 35 and absmax.size == 2
    assert absmax[0] == 0.0 and absmax[1] == 3.0
    assert np.all(packed[:32] == 0x77)
    assert packed[-1] & 0xF == 7  # pad nibble
    deq = oracle.nf4_dequant(packed, absmax, 69)
    assert np.all(deq[:64] == 0.0) and deq[65] == -3.0


def test_blocks_straddle_rows_of_the_flattened_tensor():
    W = np.zeros((2, 96), np.float32)
    W[0, 64:] = 0.5
    W[0, 70] = 8.0          # in block 1, row 0
    W[1, :32] = 0.25        # also block 1 (row 1, cols 0..31)
    W[1, 32:] = 0.125
    packed, absmax = oracle.nf4_quantize(W)
    assert absmax.tolist() == [0.0, 8.0, 0.125]
    deq = oracle.nf4_dequant(packed, absmax, W.size).reshape(W.shape)
    assert deq[0, 70] == 8.0 and deq[1, 40] == 0.125
    # row 1 col 0 sits in block 1 with absmax 8: 0.25/8 = 0.03125 -> nearest code value
    c = oracle.nf4_codebook()
    expect = c[np.argmin(np.abs(c - 0.03125))] * np.float32(8.0)
    assert deq[1, 0] == np.float32(expect)


def test_quantize_is_idempotent_and_error_bounded():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal(64 * 500) * 0.02).astype(np.float32)
    w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    p1, a1 = oracle.nf4_quantize(w)
    d1 = oracle.nf4_dequant(p1, a1, w.size)
    p2, a2 = oracle.nf4_quantize(d1)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
    c = oracle.nf4_codebook().astype(np.float64)
    half_gap = np.max(np.diff(c)) / 2
    err = np.abs(w.astype(np.float64) - d1.astype(np.float64))
    bound = half_gap * np.repeat(a1, 64).astype(np.float64) * (1 + 1e-6) + 1e-30
    assert np.all(err <= bound)
    # absmax is the block's max |w| exactly
    assert np.array_equal(a1, np.abs(w.reshape(-1, 64)).max(1))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),        # subnormals
        np.array([0.0, -0.0, 3.3895314e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  -(1.0 + 2 ** -8), np.inf, -np.inf], np.float32),    # ties, overflow
    ])
    ours = oracle.bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.isnan(oracle.bf16_bits_to_f32(oracle.bf16_rne_bits(np.array([np.nan], np.float32))))[0]
