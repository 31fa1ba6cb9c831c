"""MXFP8 quantisation of activations (E4M3 elements, one e8m0 scale per 32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (DeepSeekv4 Flash for 1x Spark forum thread, second post on
v0.2.3, "experts moved to the source's own numerics", and the fourth post): at
prefill the MXFP4 experts run as fp4 weights times E4M3 activations, with the
activation scale computed dynamically.

Readings where the pages are silent (listed in the design notes):
  * scales are per 32 consecutive elements along the contraction axis, matching
    the MX block of the block-scaled matrix instruction;
  * the scale is the smallest power of two that keeps the block maximum within
    E4M3's finite range without clipping: with a = max |v| = m * 2^p,
    m in [0.5, 1): e = p - 9 if m <= 0.875 else p - 8, so a / 2^e <= 448;
    the e8m0 code is E = clamp(e + 127, 0, 254);
  * elements are rounded to nearest, ties to even, onto E4M3FN (subnormals kept,
    sign kept on values that round to zero, saturating at 448);
  * an all-zero block gets E = 0 and all element codes 0x00.
The same rule quantises the fp32 intermediate h before the down projection.
"""
from __future__ import annotations

import numpy as np

from .codecs import E4M3, E8M0, f64_to_e4m3fn_rne


def block_exponent_code(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(amax)
    e = np.where(m <= 0.875, p - 9, p - 8).astype(np.int64)
    E = np.clip(e + 127, 0, 254)
    return np.where(amax == 0, 0, E).astype(np.uint8)


def quantize(v: np.ndarray):
    """v: [rows, K] real values (K a multiple of 32). Returns (codes u8 [rows, K],
    e8m0 u8 [rows, K / 32])."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    blk = v.reshape(rows, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    E = block_exponent_code(amax)
    scale = np.ldexp(1.0, E.astype(np.int64) - 127)
    codes = f64_to_e4m3fn_rne(blk / scale[..., None])
    codes = np.where((amax == 0)[..., None], np.uint8(0), codes)
    return codes.reshape(rows, K).astype(np.uint8), E


def dequantize(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    s = E8M0[np.asarray(e8m0, dtype=np.uint8).reshape(rows, K // 32)]
    return E4M3[codes] * np.repeat(s, 32, axis=1)
