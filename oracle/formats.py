"""Exact decode of whole expert tensors, one function per block format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each decoder takes an expert tensor in its source layout (the layout the format
is published in; see below) and returns the exact real value of every weight as
float64, shape [rows, cols] (rows = output features, cols = input features, the
contraction axis). Every product here is exact in float64 (at most 30
significant bits), so these are the values the formats define, before any
rounding. ``to_f32`` then rounds once, to nearest even, for the bit-exact check
of a device dequantiser.

Formats and the passages that define them:
  * MXFP4 - e2m1 elements with one e8m0 scale per 32 along the input axis, 4.25
    bits per weight (DeepSeekv4 Flash for 1x Spark [REAP25] forum thread, first
    post, measured-KL format allocation; REAP K180 Mixed NVFP4 card, lossless
    MXFP4 -> NVFP4 conversion section). Source layout: nibbles u8 [rows, cols/2]
    with element 2j in the low nibble of byte j; e8m0 u8 [rows, cols/32].
  * NVFP4 - e2m1 elements, one e4m3 scale per 16, one fp32 scale_2 per expert
    tensor, 4.5 bits per weight (REAP K180 card, "Why this mix?" and the
    conversion section). Weight = e2m1 * e4m3 * scale_2.
  * Q2_K - ggml 256-weight superblock of 2-bit quants with a 4-bit scale and a
    4-bit min per 16 weights and fp16 d, dmin: 84 bytes, 2.625 bits per weight
    (IQ2_XXS + Q2_K + FP8 hybrid card, format table; DeepSeek-V4.1-Flash
    mixed-Q2 GGUF card, Recipe: 2.25 bits per weight averaged over IQ2_XXS
    gate/up and Q2_K down). Weight = d * (sc & 15) * q - dmin * (sc >> 4).
  * IQ2_XXS - ggml 256-weight superblock: fp16 d, 32 codebook indices of 8
    magnitudes, 32 seven-bit sign codes, 8 four-bit scales: 66 bytes, 2.0625 bits
    per weight (same two cards). The codebook is an input.
  * FP8 block-128 - E4M3 weights with one UE8M0 scale per 128 x 128 tile, 8 bits
    per weight (IQ2_XXS + Q2_K + FP8 hybrid card, format table; DeepSeek-V4-Flash
    W4A16-FP8 card, component precisions table: FP8 block 128 x 128).
  * FP8 block-32 - the same with one UE8M0 scale per 32 x 32 tile: the dense FP8
    weights of DeepSeek-V4.1 (DeepSeek-V4.1-Flash mixed-Q2 GGUF card, Recipe,
    second bullet: V4.1 uses 32 x 32 E8M0 block scales where V4 uses 128 x 128,
    and reading one with the other's tile size rescales every weight).
    8 + 8/1024 bits per weight.
  * MXFP8 - E4M3 elements with one e8m0 scale per 32 along the input axis, the
    checkpoint's own format for attention, shared experts and the head
    (DeepSeekv4 Flash for 1x Spark forum thread, first post; second post: the
    same bytes pre-stored in the matrix engine's layout). 8.25 bits per weight.
    Source layout: codes u8 [rows, cols], e8m0 u8 [rows, cols/32].

Readings where the pages are silent (each listed in the design notes):
  * Q2_K block = scales[16] u8, qs[64] u8, d fp16, dmin fp16 (little-endian).
    Sub-block j = i // 16 of weight i uses scales[j]: low nibble = scale, high
    nibble = min. The 2-bit quant of weight i: half h = i // 128, r = i % 128,
    byte qs[32 h + r % 32], bits 2 * (r // 32) and up.
  * IQ2_XXS block = d fp16, then for sub-block b = 0..7 (32 weights each) a
    little-endian u32 a0 (byte l = codebook index of group l) and u32 a1
    (bits 7l..7l+6 = sign code of group l, bits 28..31 = scale s). Group l holds
    weights 32 b + 8 l + j, j = 0..7. db = d * (0.5 + s) / 4. The 8-bit sign mask
    is the 7-bit code with bit 7 set to the parity of the code (so every group has
    an even number of negative weights); bit j set negates weight j.
  * FP8 tiles are 2-D 128 x 128 (8.0005 bits per weight; a 1 x 128 tiling would
    give 8.0625); the V4.1 tiles likewise 2-D 32 x 32.
  * MXFP8 elements and scales follow the OCP MX definition (E4M3FN elements, a
    shared power-of-two scale 2^(E-127), E = 255 NaN) with the block along the
    input axis, as for MXFP4 in the same checkpoint.
"""
from __future__ import annotations

import numpy as np

from .codecs import E2M1, E4M3, E8M0, fp16_to_f64

MXFP4, NVFP4, Q2_K, IQ2_XXS, FP8_B128, MXFP8, FP8_B32 = 1, 2, 3, 4, 5, 6, 7
BLOCK_K = {MXFP4: 32, NVFP4: 16, Q2_K: 256, IQ2_XXS: 256, FP8_B128: 128, MXFP8: 32, FP8_B32: 32}


def packed_bytes(fmt: int, rows: int, cols: int) -> int:
    """Bytes of one expert tensor [rows, cols], scales included (NVFP4's 4-byte
    scale_2 included). 0 for a shape the format cannot hold."""
    bk = BLOCK_K.get(fmt)
    if bk is None or rows <= 0 or cols <= 0 or cols % bk:
        return 0
    n = rows * cols
    if fmt == MXFP4:
        return n // 2 + n // 32
    if fmt == NVFP4:
        return n // 2 + n // 16 + 4
    if fmt == Q2_K:
        return rows * (cols // 256) * 84
    if fmt == IQ2_XXS:
        return rows * (cols // 256) * 66
    if fmt == FP8_B128:
        if rows % 128:
            return 0
        return n + (rows // 128) * (cols // 128)
    if fmt == FP8_B32:
        if rows % 32:
            return 0
        return n + (rows // 32) * (cols // 32)
    if fmt == MXFP8:
        return n + n // 32
    return 0


def _nibbles(nib: np.ndarray, rows: int, cols: int) -> np.ndarray:
    b = np.asarray(nib, dtype=np.uint8).reshape(rows, cols // 2)
    out = np.empty((rows, cols), dtype=np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def dequant_mxfp4(nib, e8m0, rows: int, cols: int) -> np.ndarray:
    n = _nibbles(nib, rows, cols)
    s = E8M0[np.asarray(e8m0, dtype=np.uint8).reshape(rows, cols // 32)]
    return E2M1[n] * np.repeat(s, 32, axis=1)


def dequant_nvfp4(nib, e4m3, scale2: float, rows: int, cols: int) -> np.ndarray:
    n = _nibbles(nib, rows, cols)
    s = E4M3[np.asarray(e4m3, dtype=np.uint8).reshape(rows, cols // 16)]
    return E2M1[n] * np.repeat(s, 16, axis=1) * np.float64(np.float32(scale2))


def dequant_q2_k(blocks, rows: int, cols: int) -> np.ndarray:
    nsb = cols // 256
    b = np.asarray(blocks, dtype=np.uint8).reshape(rows, nsb, 84)
    sc = b[:, :, 0:16]
    qs = b[:, :, 16:80]
    d = fp16_to_f64(b[:, :, 80:82].copy().view(np.uint16)[..., 0])
    dmin = fp16_to_f64(b[:, :, 82:84].copy().view(np.uint16)[..., 0])
    i = np.arange(256)
    j = i // 16
    h = i // 128
    r = i % 128
    q = (qs[:, :, 32 * h + r % 32] >> (2 * (r // 32)).astype(np.uint8)) & 3
    scale = (sc[:, :, j] & 15).astype(np.float64)
    mn = (sc[:, :, j] >> 4).astype(np.float64)
    w = d[..., None] * scale * q - dmin[..., None] * mn
    return w.reshape(rows, cols)


def iq2_sign_mask(code7: np.ndarray) -> np.ndarray:
    """8-bit sign mask from a 7-bit sign code: bit 7 = parity of the code."""
    c = np.asarray(code7, dtype=np.uint32) & 0x7F
    par = np.zeros_like(c)
    for k in range(7):
        par ^= (c >> k) & 1
    return c | (par << 7)


def dequant_iq2_xxs(blocks, grid, rows: int, cols: int) -> np.ndarray:
    nsb = cols // 256
    b = np.asarray(blocks, dtype=np.uint8).reshape(rows, nsb, 66)
    g = np.asarray(grid, dtype=np.uint8).reshape(256, 8).astype(np.float64)
    d = fp16_to_f64(b[:, :, 0:2].copy().view(np.uint16)[..., 0])
    sub = b[:, :, 2:66].copy().view(np.uint32).reshape(rows, nsb, 8, 2)
    a0 = sub[..., 0]
    a1 = sub[..., 1]
    s = (a1 >> 28).astype(np.float64)
    db = d[..., None] * (0.5 + s) / 4.0                      # [rows, nsb, 8]
    w = np.empty((rows, nsb, 8, 4, 8), dtype=np.float64)
    for l in range(4):
        gi = (a0 >> (8 * l)) & 0xFF
        mask = iq2_sign_mask((a1 >> (7 * l)) & 0x7F)
        mags = g[gi]                                          # [rows, nsb, 8, 8]
        for j in range(8):
            neg = ((mask >> j) & 1).astype(bool)
            w[..., l, j] = np.where(neg, -1.0, 1.0) * db * mags[..., j]
    return w.reshape(rows, cols)


def dequant_fp8_b128(q, s, rows: int, cols: int) -> np.ndarray:
    v = E4M3[np.asarray(q, dtype=np.uint8).reshape(rows, cols)]
    sc = E8M0[np.asarray(s, dtype=np.uint8).reshape(rows // 128, cols // 128)]
    return v * np.repeat(np.repeat(sc, 128, axis=0), 128, axis=1)


def dequant_fp8_b32(q, s, rows: int, cols: int) -> np.ndarray:
    v = E4M3[np.asarray(q, dtype=np.uint8).reshape(rows, cols)]
    sc = E8M0[np.asarray(s, dtype=np.uint8).reshape(rows // 32, cols // 32)]
    return v * np.repeat(np.repeat(sc, 32, axis=0), 32, axis=1)


def dequant_mxfp8(q, e8m0, rows: int, cols: int) -> np.ndarray:
    v = E4M3[np.asarray(q, dtype=np.uint8).reshape(rows, cols)]
    s = E8M0[np.asarray(e8m0, dtype=np.uint8).reshape(rows, cols // 32)]
    return v * np.repeat(s, 32, axis=1)


def dequant(fmt: int, planes, rows: int, cols: int, scale2: float = 1.0, grid=None) -> np.ndarray:
    """Dispatch on format; ``planes`` is the list of source-layout arrays."""
    if fmt == MXFP4:
        return dequant_mxfp4(planes[0], planes[1], rows, cols)
    if fmt == NVFP4:
        return dequant_nvfp4(planes[0], planes[1], scale2, rows, cols)
    if fmt == Q2_K:
        return dequant_q2_k(planes[0], rows, cols)
    if fmt == IQ2_XXS:
        return dequant_iq2_xxs(planes[0], grid, rows, cols)
    if fmt == FP8_B128:
        return dequant_fp8_b128(planes[0], planes[1], rows, cols)
    if fmt == FP8_B32:
        return dequant_fp8_b32(planes[0], planes[1], rows, cols)
    if fmt == MXFP8:
        return dequant_mxfp8(planes[0], planes[1], rows, cols)
    raise ValueError(fmt)


def to_f32(w: np.ndarray) -> np.ndarray:
    """Round exact values once, to nearest even, to float32."""
    return np.asarray(w, dtype=np.float64).astype(np.float32)
