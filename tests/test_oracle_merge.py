"""Pins of the oracle's adapter merge (oracle/merge.py)."""
import numpy as np

import oracle
import synth


def _base(rows, cols, seed):
    w = synth.bf16_bits_to_f32(synth.to_bf16_bits(np.random.default_rng(seed).standard_normal((rows, cols)) * 0.02))
    return oracle.nf4_quantize(w)


def test_zero_B_gives_the_dequantized_base_and_requantizes_to_the_same_codes():
    rows, cols, r = 96, 128, 8
    packed, absmax = _base(rows, cols, 0)
    A = np.random.default_rng(1).standard_normal((r, cols))
    B = np.zeros((rows, r))
    merged = oracle.lora_merge(packed, absmax, rows, cols, A, B, 2.0)
    assert np.array_equal(merged, oracle.bf16_round(oracle.nf4_dequant(packed, absmax, rows * cols)).reshape(rows, cols))
    p2, a2 = oracle.lora_merge(packed, absmax, rows, cols, A, B, 2.0, to_nf4=True)
    assert np.array_equal(p2, packed) and np.array_equal(a2, absmax)


def test_merged_linear_equals_the_qlora_linear_up_to_bf16_rounding():
    rows, cols, r, s = 64, 192, 4, 0.25
    packed, absmax = _base(rows, cols, 2)
    g = np.random.default_rng(3)
    A, B = g.standard_normal((r, cols)) * 0.05, g.standard_normal((rows, r)) * 0.05
    x = g.standard_normal((16, cols))
    merged = oracle.lora_merge(packed, absmax, rows, cols, A, B, s)
    W = oracle.nf4_dequant(packed, absmax, rows * cols).reshape(rows, cols).astype(np.float64)
    y_ref = x @ W.T + s * (x @ A.T) @ B.T
    y = x @ merged.astype(np.float64).T
    # each merged weight carries at most half a bf16 ulp of relative error
    bound = 2.0 ** -9 * (np.abs(x) @ np.abs(W + s * B @ A).T)
    assert np.all(np.abs(y - y_ref) <= bound + 1e-12)


def test_rank_one_exact_sum():
    rows, cols = 2, 64
    packed, absmax = oracle.nf4_quantize(np.zeros((rows, cols), np.float32))    # all-zero base
    A = np.full((1, cols), 0.5)
    B = np.array([[2.0], [-4.0]])
    merged = oracle.lora_merge(packed, absmax, rows, cols, A, B, 0.25)
    assert np.array_equal(merged, np.stack([np.full(cols, 0.25), np.full(cols, -0.5)]).astype(np.float32))
