"""NF4 (4-bit NormalFloat) blockwise quantization, the oracle's version.

Pages: NF4, 4 bits per parameter, is how the frozen 8B base fits
(rug.gal article, "En detalle"; imasters article, "Como cabe um 8B em 4 GB",
config line ``quantization: 4bit  # NF4``). The pages give no construction,
so the published definition (QLoRA, Dettmers et al. 2023, NormalFloat section
and NF4 appendix) is followed:

codebook  16 values: 8 non-negative quantiles, 7 negative quantiles and an
          exact zero, normalised to [-1, 1]. The quantile probabilities are
          evenly spaced from p_max = 0.9677083 (the paper's offset) down to
          1/2 in fp32; the quantiles are the standard normal inverse CDF
          (fp64); the values are rounded to fp32 and then divided by their
          maximum in fp32. This reproduces the 16 values the QLoRA appendix
          prints, bit for bit (pinned in tests/golden/nf4_codebook_qlora.txt).
quantize  per block of 64 consecutive elements of the row-major flattened
          tensor: absmax a = max |w| (fp32), x = w / a (IEEE fp32 division),
          code = index of the nearest codebook value, decided by the 15
          fp32 midpoints m_i = fl((c_i + c_{i+1}) / 2): code = #{i : x > m_i}
          (an exact tie goes to the lower code). a = 0 gives x = 0 (code 7).
pack      two codes per byte, the even element in the high nibble. An odd
          element count pads the last low nibble with code 7.
dequant   w' = fl32(c[code] * a); the GEMM operand is that value rounded to
          bf16 (round-to-nearest-even).

Parity pins: codebook = published table; round trip of every code at
power-of-two scales; brute-force nearest value vs the midpoint rule;
idempotence of quantize(dequant(quantize(w))); error bound; bf16 rounding
vs torch's conversion.
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

BLOCK = 64


def _even_steps_f32(start: float, end: float, steps: int) -> np.ndarray:
    """fp32 points evenly spaced from start to end inclusive.

    The step is (end - start) / (steps - 1) in fp32; the first half of the
    points are start + i*step and the second half end - (steps-1-i)*step,
    so both end points are exact."""
    f = np.float32
    start, end = f(start), f(end)
    step = f((end - start) / f(steps - 1))
    out = np.empty(steps, np.float32)
    for i in range(steps):
        if i < steps // 2:
            out[i] = f(start + f(step * f(i)))
        else:
            out[i] = f(end - f(step * f(steps - 1 - i)))
    return out


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 values, ascending, float32."""
    inv = NormalDist().inv_cdf
    p_max = 0.9677083
    pos_p = _even_steps_f32(p_max, 0.5, 9)[:-1]   # 8 probabilities -> 8 positive quantiles
    neg_p = _even_steps_f32(p_max, 0.5, 8)[:-1]   # 7 probabilities -> 7 negative quantiles
    vals = [inv(float(p)) for p in pos_p] + [0.0] + [-inv(float(p)) for p in neg_p]
    v = np.sort(np.array(vals, dtype=np.float64)).astype(np.float32)
    v = (v / v.max()).astype(np.float32)
    return v


def nf4_midpoints(c: np.ndarray | None = None) -> np.ndarray:
    """The 15 decision thresholds m_i = fl32((c_i + c_{i+1}) / 2)."""
    c = nf4_codebook() if c is None else c
    return ((c[:-1] + c[1:]) * np.float32(0.5)).astype(np.float32)


def nf4_quantize(w, block: int = BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a tensor (any shape; flattened row-major) to NF4.

    Returns (packed uint8 [ceil(n/2)], absmax float32 [ceil(n/block)])."""
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    n = w.size
    nb = (n + block - 1) // block
    padded = np.zeros(nb * block, np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, block)
    absmax = np.abs(blocks).max(axis=1).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    x[absmax == 0] = np.float32(0.0)
    m = nf4_midpoints()
    # number of thresholds strictly below x  == #{i : x > m_i}
    codes = np.searchsorted(m, x.ravel(), side="left").astype(np.uint8)[:n]
    if n % 2:
        codes = np.concatenate([codes, np.array([7], np.uint8)])
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    return packed, absmax


def nf4_unpack(packed: np.ndarray, n: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    codes = np.empty(packed.size * 2, np.uint8)
    codes[0::2] = packed >> 4
    codes[1::2] = packed & 0xF
    return codes[:n]


def nf4_dequant(packed, absmax, n: int, block: int = BLOCK) -> np.ndarray:
    """w'[i] = fl32(c[code_i] * absmax[i // block]), float32 [n]."""
    c = nf4_codebook()
    codes = nf4_unpack(packed, n)
    a = np.repeat(np.asarray(absmax, np.float32), block)[:n]
    return (c[codes] * a).astype(np.float32)


def bf16_rne_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint32)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """fp32 value after a round trip through bf16 (RNE)."""
    return bf16_bits_to_f32(bf16_rne_bits(x))
