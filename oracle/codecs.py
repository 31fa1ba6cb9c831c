"""Element codecs, written from the definitions of each number format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats and where they are named:
  * e2m1 (FP4): the element type of the MXFP4 and NVFP4 blocks (REAP K180 Mixed
    NVFP4 model card, section on the lossless MXFP4 -> NVFP4 conversion). Bit
    layout from the OCP Microscaling Formats (MX) v1.0 specification: 1 sign bit,
    2 exponent bits with bias 1, 1 mantissa bit, no infinities or NaN.
  * e4m3fn (FP8): NVFP4 block scales, the FP8 block-128 dense weights (IQ2_XXS +
    Q2_K + FP8 hybrid model card, format table) and MXFP8 activations. 1 sign,
    4 exponent bits with bias 7, 3 mantissa bits; S.1111.111 is NaN; no infinities.
  * e8m0 (UE8M0): MXFP4 block scales and the FP8 block-128 tile scales. An
    unsigned power of two 2^(E-127); E = 255 is NaN.
  * fp16 (IEEE binary16): Q2_K d/dmin and IQ2_XXS d.
  * bf16: the activation vector.
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                       # subnormal: 2^(1-1) * (m / 2)
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e4m3fn_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6         # subnormal
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(code: int) -> float:
    if code == 255:
        return math.nan
    return 2.0 ** (code - 127)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):                # NaN payloads stay NaN
        return u.view(np.float32).astype(np.float64)


def f64_to_e4m3fn_rne(v: np.ndarray) -> np.ndarray:
    """Round to nearest, ties to even, onto E4M3FN codes, saturating at +-448.
    The sign is kept for values that round to zero. Inputs must not be NaN.

    Normal binade [2^e, 2^(e+1)) has quantum 2^(e-3); below 2^-6 the quantum is
    the subnormal step 2^-9. Scaling by a power of two is exact in float64, so
    ``np.rint`` (ties to even) performs the one rounding."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v).astype(np.uint8) << 7).astype(np.uint8)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    # Subnormal codes are the count of 2^-9 steps; a count of 8 is code 0x08,
    # the smallest normal 2^-6, so the same integer serves as the code.
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)

    nrm = ~sub
    _, p = np.frexp(a[nrm])
    e = p.astype(np.int64) - 1                      # a in [2^e, 2^(e+1))
    q = np.rint(a[nrm] / np.ldexp(1.0, e - 3)).astype(np.int64)   # 8..16
    up = q == 16
    e = np.where(up, e + 1, e)
    q = np.where(up, 8, q)
    c = ((e + 7) << 3) | (q - 8)
    code[nrm] = c

    code = np.where(a >= 448.0, 0x7E, code)
    code = np.where(code > 0x7E, 0x7E, code)        # rounding crossed 448: saturate
    return code.astype(np.uint8) | sign
