"""Lossless MXFP4 -> NVFP4 re-encode of an expert tensor, and its inverse.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (REAP K180 Mixed NVFP4 card, section on the lossless
MXFP4 -> NVFP4 conversion, and "How It Was Built", step 3): the e2m1 nibbles are
carried over unchanged; only the scales change, from one e8m0 per 32 weights to
one e4m3 per 16 weights plus one fp32 scale_2 per expert tensor; the re-encoded
weights equal the originals.

Reading where the pages are silent (listed in the design notes): scale_2 is
chosen so that the largest block exponent lands on e4m3's largest power of two,
2^8. With Emax the largest e8m0 code in the tensor:
    scale_2 = 2^(Emax - 127 - 8)
    e4m3 of both 16-halves of a block with code E = 2^(E - Emax + 8)
so e4m3 * scale_2 = 2^(E - 127) exactly. e4m3 holds every power of two from 2^-9
(smallest subnormal) to 2^8, so the re-encode is exact when Emax - E <= 17 for
every block; a wider span, or a NaN code (255), cannot be carried and is refused.

The inverse (NVFP4 -> MXFP4, so that an NVFP4 tensor can take a path built for
e8m0 block scales) is exact exactly when, in every 32-block, both 16-halves carry
the same e4m3 scale and that scale times scale_2 is a power of two 2^k with
-127 <= k <= 127 (then E = k + 127); otherwise it is refused. It undoes the
forward re-encode byte for byte.
"""
from __future__ import annotations

import numpy as np


class LossyConversion(ValueError):
    pass


def e4m3_code_of_pow2(k: int) -> int:
    """E4M3FN code of 2^k for -9 <= k <= 8."""
    if not -9 <= k <= 8:
        raise LossyConversion(f"2^{k} is not an e4m3 power of two")
    if k >= -6:
        return (k + 7) << 3                 # normal: exponent field k + 7, mantissa 0
    return 1 << (k + 9)                     # subnormal: (m / 8) * 2^-6 with m = 2^(k+9)


def mxfp4_to_nvfp4(nib, e8m0, rows: int, cols: int):
    """Returns (nibbles u8 [rows, cols/2], e4m3 u8 [rows, cols/16], scale_2 fp32)."""
    nib = np.asarray(nib, dtype=np.uint8).reshape(rows, cols // 2)
    e = np.asarray(e8m0, dtype=np.uint8).reshape(rows, cols // 32)
    if np.any(e == 255):
        raise LossyConversion("NaN e8m0 code")
    emax = int(e.max())
    if emax - int(e.min()) > 17:
        raise LossyConversion(f"exponent span {emax - int(e.min())} > 17")
    scale2 = np.float32(2.0 ** (emax - 127 - 8))
    codes32 = np.array([e4m3_code_of_pow2(int(E) - emax + 8) if 0 <= emax - int(E) <= 17 else 0
                        for E in range(256)], dtype=np.uint8)
    e4m3 = np.repeat(codes32[e], 2, axis=1)   # both 16-halves of each 32-block
    return nib.copy(), e4m3, scale2


def nvfp4_to_mxfp4(nib, e4m3, scale2, rows: int, cols: int):
    """Returns (nibbles u8 [rows, cols/2], e8m0 u8 [rows, cols/32]) or raises
    LossyConversion when some block has no exact e8m0 scale."""
    from fractions import Fraction

    from .codecs import E4M3

    nib = np.asarray(nib, dtype=np.uint8).reshape(rows, cols // 2)
    s = np.asarray(e4m3, dtype=np.uint8).reshape(rows, cols // 32, 2)
    if np.any(s[..., 0] != s[..., 1]):
        raise LossyConversion("the two 16-halves of a block carry different scales")
    s2 = Fraction(float(np.float32(scale2)))
    e8 = np.empty((rows, cols // 32), dtype=np.uint8)
    for code in np.unique(s[..., 0]):
        v = E4M3[int(code)]
        if not np.isfinite(v) or v <= 0:
            raise LossyConversion(f"e4m3 scale code {int(code):#x} is not a positive number")
        p = Fraction(float(v)) * s2
        k = p.numerator.bit_length() - 1 if p.denominator == 1 else -(p.denominator.bit_length() - 1)
        if p != Fraction(2) ** k or not -127 <= k <= 127:
            raise LossyConversion(f"scale {p} is not a power of two in e8m0's range")
        e8[s[..., 0] == code] = k + 127
    return nib.copy(), e8
