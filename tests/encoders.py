"""Block encoders used to pin the oracle's decoders by round trip.

They run the layout readings in the other direction (field values -> bytes),
one weight at a time, so an index or shift mistake in a decoder does not cancel
against the same mistake here. Exact expected values are computed with
``fractions.Fraction`` from the chosen field values.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e2m1_frac(code: int) -> Fraction:
    m = E2M1_MAG[code & 7]
    return -m if code & 8 else m


def e4m3_frac(code: int) -> Fraction:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    assert not (e == 15 and m == 7)
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def pow2_frac(k: int) -> Fraction:
    return Fraction(2) ** k


def fp16_frac(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def put_nibble(buf: bytearray, k: int, code: int):
    if k % 2 == 0:
        buf[k // 2] = (buf[k // 2] & 0xF0) | code
    else:
        buf[k // 2] = (buf[k // 2] & 0x0F) | (code << 4)


def encode_mxfp4(codes, E, rows, cols):
    """codes [rows][cols] e2m1 codes, E [rows][cols/32] e8m0 codes."""
    nib = bytearray(rows * cols // 2)
    for r in range(rows):
        row = bytearray(cols // 2)
        for c in range(cols):
            put_nibble(row, c, int(codes[r][c]))
        nib[r * cols // 2:(r + 1) * cols // 2] = row
    exact = [[e2m1_frac(int(codes[r][c])) * pow2_frac(int(E[r][c // 32]) - 127) for c in range(cols)]
             for r in range(rows)]
    return np.frombuffer(bytes(nib), np.uint8), np.array(E, np.uint8).reshape(-1), exact


def encode_nvfp4(codes, S, scale2, rows, cols):
    nib = bytearray(rows * cols // 2)
    for r in range(rows):
        row = bytearray(cols // 2)
        for c in range(cols):
            put_nibble(row, c, int(codes[r][c]))
        nib[r * cols // 2:(r + 1) * cols // 2] = row
    s2 = Fraction(float(np.float32(scale2)))
    exact = [[e2m1_frac(int(codes[r][c])) * e4m3_frac(int(S[r][c // 16])) * s2 for c in range(cols)]
             for r in range(rows)]
    return np.frombuffer(bytes(nib), np.uint8), np.array(S, np.uint8).reshape(-1), exact


def encode_q2_k_block(q, sc, mn, d_bits, dmin_bits):
    """q[256] in 0..3; sc[16], mn[16] in 0..15; fp16 bit patterns for d and dmin."""
    blk = bytearray(84)
    for j in range(16):
        blk[j] = (mn[j] << 4) | sc[j]
    for i in range(256):
        h, r = divmod(i, 128)
        byte = 16 + 32 * h + r % 32
        shift = 2 * (r // 32)
        blk[byte] |= (q[i] & 3) << shift
    blk[80:82] = int(d_bits).to_bytes(2, "little")
    blk[82:84] = int(dmin_bits).to_bytes(2, "little")
    d, dmin = fp16_frac(d_bits), fp16_frac(dmin_bits)
    exact = [d * sc[i // 16] * q[i] - dmin * mn[i // 16] for i in range(256)]
    return bytes(blk), exact


def encode_iq2_xxs_block(gidx, neg, scales, d_bits, grid):
    """gidx[32] codebook indices (group g = 4 b + l); neg[256] booleans with an even
    count per group of 8; scales[8] in 0..15."""
    blk = bytearray(66)
    blk[0:2] = int(d_bits).to_bytes(2, "little")
    for b in range(8):
        a0 = 0
        a1 = scales[b] << 28
        for l in range(4):
            g = 4 * b + l
            a0 |= gidx[g] << (8 * l)
            bits = [bool(neg[32 * b + 8 * l + j]) for j in range(8)]
            assert sum(bits) % 2 == 0
            code = sum(1 << j for j in range(7) if bits[j])
            a1 |= code << (7 * l)
        blk[2 + 8 * b:6 + 8 * b] = a0.to_bytes(4, "little")
        blk[6 + 8 * b:10 + 8 * b] = a1.to_bytes(4, "little")
    d = fp16_frac(d_bits)
    exact = []
    for i in range(256):
        b, rem = divmod(i, 32)
        l, j = divmod(rem, 8)
        db = d * (Fraction(1, 2) + scales[b]) / 4
        v = db * int(grid[gidx[4 * b + l]][j])
        exact.append(-v if neg[i] else v)
    return bytes(blk), exact


def encode_fp8_b128(codes, S, rows, cols):
    q = np.array(codes, np.uint8).reshape(rows, cols)
    exact = [[e4m3_frac(int(q[r, c])) * pow2_frac(int(S[r // 128][c // 128]) - 127) for c in range(cols)]
             for r in range(rows)]
    return q.reshape(-1), np.array(S, np.uint8).reshape(-1), exact


def encode_mxfp8(codes, E, rows, cols):
    """codes [rows][cols] E4M3 codes, E [rows][cols/32] e8m0 codes."""
    q = np.array(codes, np.uint8).reshape(rows, cols)
    exact = [[e4m3_frac(int(q[r, c])) * pow2_frac(int(E[r][c // 32]) - 127) for c in range(cols)]
             for r in range(rows)]
    return q.reshape(-1), np.array(E, np.uint8).reshape(-1), exact


def encode_fp8_b32(codes, S, rows, cols):
    """codes [rows][cols] E4M3 codes, S [rows/32][cols/32] e8m0 codes of the tiles."""
    q = np.array(codes, np.uint8).reshape(rows, cols)
    exact = [[e4m3_frac(int(q[r, c])) * pow2_frac(int(S[r // 32][c // 32]) - 127) for c in range(cols)]
             for r in range(rows)]
    return q.reshape(-1), np.array(S, np.uint8).reshape(-1), exact
