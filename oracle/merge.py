"""Adapter merge, the oracle's version: fold a trained LoRA adapter into its
NF4 base matrix.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: the tool merges the adapter into the base model (guillermodelpino.com
article, command list: `soup merge`; imasters article, closing section). The
merged weight is the weight the QLoRA linear computes with, written out:
    W_merged = W' + s * B A,   W' = fl32(c[code] * absmax),  s = alpha / r
(LoRA, Hu et al. 2021, section 4.1: for inference the low-rank product can
be added into the frozen weight once), computed in float64 here and rounded
to bf16 through fp32 (round to nearest even both times; bf16 is the
computation type the weights are used in). The NF4 output re-quantizes that
bf16 matrix with the ordinary quantizer (same blocks over the flattened
matrix).

Parity pins (tests/test_oracle_merge.py): B = 0 gives bf16 of the dequantized
base exactly, and then NF4 re-quantization returns the original codes and
absmax (quantize o dequant is the identity on quantized values); a merged
linear equals the QLoRA linear x W'^T + s (x A^T) B^T up to the bf16 rounding
of the merged weights; a rank-1 adapter with exactly representable values
gives the hand-computed sum.
"""
from __future__ import annotations

import numpy as np

from .nf4 import bf16_round, nf4_dequant, nf4_quantize


def lora_merge(packed, absmax, rows, cols, A, B, scale, to_nf4=False):
    """Returns bf16-rounded float32 [rows, cols], or (to_nf4) (packed, absmax)
    of that matrix re-quantized."""
    w = nf4_dequant(packed, absmax, rows * cols).reshape(rows, cols).astype(np.float64)
    merged = w + float(scale) * (np.asarray(B, np.float64) @ np.asarray(A, np.float64))
    merged = bf16_round(merged.astype(np.float64))
    if not to_nf4:
        return merged
    return nf4_quantize(merged)
