"""Seeded synthetic inputs for the routed-MoE dequant path.

This module is input generation only: it draws bytes and numbers, and maps raw
random bytes onto the code ranges each workload uses. It decodes nothing and
computes nothing of the method. Both the CPU oracle's tests and the GPU path are
fed from it; the GPU fill kernel (``csrc/synth.hip``) implements the same
counter-based generator from the same definition, so full-size tensors can be
made on the device and any expert of them regenerated on the host.

Counter-based generator (SplitMix64, Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; finaliser constants as published
by Vigna for ``splitmix64.c``):

    mix64(z)  = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
                z *= 0x94D049BB133111EB; z ^= z >> 31          (all mod 2^64)
    key(S, s) = mix64(S * 2^32 + s)
    word(S, s, i) = mix64(key(S, s) + (i + 1) * 0x9E3779B97F4A7C15)

Byte j of stream ``s`` is byte ``j % 8`` (little-endian) of ``word(S, s, j // 8)``.

Source layouts produced here (the layouts the formats are published in):
  * MXFP4   nibbles u8 [rows, cols/2] (element 2j in the low nibble of byte j),
            e8m0 u8 [rows, cols/32]
  * NVFP4   nibbles u8 [rows, cols/2], e4m3 u8 [rows, cols/16], fp32 scale_2
  * Q2_K    u8 [rows, cols/256, 84]: scales[16], qs[64], d fp16, dmin fp16
  * IQ2_XXS u8 [rows, cols/256, 66]: d fp16, then 8 x (u32 a0, u32 a1)
  * FP8-B128 codes u8 [rows, cols], ue8m0 u8 [rows/128, cols/128]
  * FP8-B32  codes u8 [rows, cols], ue8m0 u8 [rows/32, cols/32]
  * MXFP8   codes u8 [rows, cols], e8m0 u8 [rows, cols/32]
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Field kinds: how raw random bytes are mapped to codes (integer maps only).
FIELD_RAW = 0          # bytes used as drawn
FIELD_E8M0_119_123 = 1  # e8m0 exponent codes 119..123 (2^-8 .. 2^-4)
FIELD_E4M3_08_28 = 2    # e4m3 codes 0x08..0x28 (33 codes, 2^-6 .. 2^-2)
FIELD_E4M3_FINITE = 3   # the 254 non-NaN e4m3 codes
FIELD_Q2K_BLOCK = 4     # 84-byte Q2_K blocks: d and dmin taken from D_TABLE
FIELD_IQ2_BLOCK = 5     # 66-byte IQ2_XXS blocks: d taken from D_TABLE

D_TABLE_SIZE = 4096


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * _M1
        z = z ^ (z >> np.uint64(27))
        z = z * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def stream_key(seed: int, stream: int) -> np.uint64:
    v = ((int(seed) & 0xFFFFFFFF) << 32) | (int(stream) & 0xFFFFFFFF)
    return mix64(np.array([v], dtype=np.uint64))[0]


def words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    key = stream_key(seed, stream)
    i = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + (i + np.uint64(1)) * GAMMA)


def raw_bytes(seed: int, stream: int, byte_offset: int, nbytes: int) -> np.ndarray:
    """Bytes [byte_offset, byte_offset + nbytes) of a stream."""
    if nbytes == 0:
        return np.zeros(0, dtype=np.uint8)
    w0 = byte_offset // 8
    w1 = (byte_offset + nbytes + 7) // 8
    b = words(seed, stream, w0, w1 - w0).view(np.uint8)  # little-endian host
    s = byte_offset - 8 * w0
    return b[s:s + nbytes].copy()


def d_table() -> np.ndarray:
    """fp16 codes for values spread uniformly over [1e-3, 1e-2] (4096 points,
    midpoint rule, rounded to nearest fp16). Used for Q2_K d/dmin and IQ2_XXS d."""
    i = np.arange(D_TABLE_SIZE, dtype=np.float64)
    v = 1e-3 + 9e-3 * (i + 0.5) / D_TABLE_SIZE
    return v.astype(np.float16).view(np.uint16)


def apply_field(b: np.ndarray, kind: int, byte_offset: int = 0) -> np.ndarray:
    """Map raw bytes to the code range of a field. ``byte_offset`` is the
    position of b[0] in its stream (block fields depend on the position)."""
    b = b.astype(np.uint8, copy=True)
    if kind == FIELD_RAW:
        return b
    if kind == FIELD_E8M0_119_123:
        return (119 + (b % 5)).astype(np.uint8)
    if kind == FIELD_E4M3_08_28:
        return (0x08 + (b % 33)).astype(np.uint8)
    if kind == FIELD_E4M3_FINITE:
        c = (b % 254).astype(np.uint16)
        c = np.where(c >= 0x7F, c + 1, c)
        return c.astype(np.uint8)
    if kind in (FIELD_Q2K_BLOCK, FIELD_IQ2_BLOCK):
        bs = 84 if kind == FIELD_Q2K_BLOCK else 66
        halves = [80, 82] if kind == FIELD_Q2K_BLOCK else [0]
        tab = d_table()
        n = b.size
        pos = (np.arange(n, dtype=np.int64) + byte_offset) % bs
        # A half-word field is rewritten as a whole: its two raw bytes give 16 random
        # bits, reduced mod 4096 to pick a table entry.
        out = b.copy()
        for h in halves:
            lo_idx = np.nonzero(pos == h)[0]
            lo_idx = lo_idx[lo_idx + 1 < n]
            raw = b[lo_idx].astype(np.uint16) | (b[lo_idx + 1].astype(np.uint16) << 8)
            code = tab[raw % D_TABLE_SIZE]
            out[lo_idx] = (code & 0xFF).astype(np.uint8)
            out[lo_idx + 1] = (code >> 8).astype(np.uint8)
        return out
    raise ValueError(f"unknown field kind {kind}")


def field_bytes(seed: int, stream: int, kind: int, byte_offset: int, nbytes: int) -> np.ndarray:
    """Bytes of a generated field. Block fields must start on a block boundary."""
    if kind in (FIELD_Q2K_BLOCK, FIELD_IQ2_BLOCK):
        bs = 84 if kind == FIELD_Q2K_BLOCK else 66
        assert byte_offset % bs == 0 and nbytes % bs == 0
    return apply_field(raw_bytes(seed, stream, byte_offset, nbytes), kind, byte_offset)


# ----------------------------------------------------------------------------
# Expert tensors: one stream per (layer, projection, plane); expert e occupies
# bytes [e * plane_bytes, (e + 1) * plane_bytes) of its stream.

PROJ_GATE, PROJ_UP, PROJ_DOWN, PROJ_LINEAR = 0, 1, 2, 3
FMT_MXFP4, FMT_NVFP4, FMT_Q2_K, FMT_IQ2_XXS, FMT_FP8_B128, FMT_MXFP8, FMT_FP8_B32 = 1, 2, 3, 4, 5, 6, 7
FMT_NAMES = {FMT_MXFP4: "mxfp4", FMT_NVFP4: "nvfp4", FMT_Q2_K: "q2_k",
             FMT_IQ2_XXS: "iq2_xxs", FMT_FP8_B128: "fp8_b128", FMT_MXFP8: "mxfp8", FMT_FP8_B32: "fp8_b32"}


def stream_id(layer: int, proj: int, plane: int) -> int:
    return (layer << 8) | (proj << 4) | plane


def source_planes(fmt: int, rows: int, cols: int):
    """[(plane_bytes_per_expert, field_kind)] of a format's source layout."""
    if fmt == FMT_MXFP4:
        return [(rows * cols // 2, FIELD_RAW), (rows * cols // 32, FIELD_E8M0_119_123)]
    if fmt == FMT_NVFP4:
        return [(rows * cols // 2, FIELD_RAW), (rows * cols // 16, FIELD_E4M3_08_28)]
    if fmt == FMT_Q2_K:
        return [(rows * (cols // 256) * 84, FIELD_Q2K_BLOCK)]
    if fmt == FMT_IQ2_XXS:
        return [(rows * (cols // 256) * 66, FIELD_IQ2_BLOCK)]
    if fmt == FMT_FP8_B128:
        return [(rows * cols, FIELD_E4M3_FINITE), ((rows // 128) * (cols // 128), FIELD_E8M0_119_123)]
    if fmt == FMT_FP8_B32:
        return [(rows * cols, FIELD_E4M3_FINITE), ((rows // 32) * (cols // 32), FIELD_E8M0_119_123)]
    if fmt == FMT_MXFP8:
        return [(rows * cols, FIELD_E4M3_FINITE), (rows * cols // 32, FIELD_E8M0_119_123)]
    raise ValueError(fmt)


def expert_source(seed: int, layer: int, proj: int, fmt: int, rows: int, cols: int, expert: int):
    """Source-layout planes (list of u8 arrays) of one expert tensor."""
    out = []
    for p, (nb, kind) in enumerate(source_planes(fmt, rows, cols)):
        out.append(field_bytes(seed, stream_id(layer, proj, p), kind, expert * nb, nb))
    return out


def scale2_values(seed: int, layer: int, proj: int, n_experts: int) -> np.ndarray:
    """NVFP4 per-expert fp32 scale_2 ~ U[0.5, 2] (from the top 24 bits of a word)."""
    w = words(seed, stream_id(layer, proj, 15), 0, n_experts)
    u = (w >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return (0.5 + 1.5 * u).astype(np.float32)


def iq2_standin_grid(seed: int = 0x1A2) -> np.ndarray:
    """A stand-in IQ2_XXS codebook: 256 distinct 8-tuples over a fixed 3-level
    alphabet of small positive integers. ggml's own table is not reproduced here."""
    rng = np.random.default_rng(seed)
    levels = np.array([5, 19, 41], dtype=np.uint8)
    picks = rng.choice(3 ** 8, size=256, replace=False)
    digits = np.zeros((256, 8), dtype=np.int64)
    v = picks.copy()
    for j in range(8):
        digits[:, j] = v % 3
        v //= 3
    return levels[digits]


# ----------------------------------------------------------------------------
# Activations and routing (host generated; small).

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + r) >> np.uint64(16)).astype(np.uint16)


def activations_bf16(seed: int, T: int, H: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))


def softmax_f32(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def uniform_routing(seed: int, T: int, n_experts: int, top_k: int):
    """Independent top-k per token: distinct uniform expert ids and softmax weights."""
    rng = np.random.default_rng(seed + 7919)
    ids = np.stack([rng.choice(n_experts, size=top_k, replace=False) for _ in range(T)]).astype(np.int32)
    w = softmax_f32(rng.standard_normal((T, top_k)))
    return ids, w


def cold_routing_sequence(seed: int, n_steps: int, n_experts: int, top_k: int):
    """bs=1 routing for a sequence of decode steps: each step's ids are a uniform
    random top_k-subset, drawn as consecutive groups of a fresh random permutation,
    so no expert repeats within n_experts // top_k consecutive steps."""
    rng = np.random.default_rng(seed + 104729)
    per = n_experts // top_k
    ids = np.zeros((n_steps, top_k), dtype=np.int32)
    for s0 in range(0, n_steps, per):
        p = rng.permutation(n_experts)
        for j in range(min(per, n_steps - s0)):
            ids[s0 + j] = p[j * top_k:(j + 1) * top_k]
    w = softmax_f32(rng.standard_normal((n_steps, top_k)))
    return ids, w


def zipf_token_ids(seed: int, T: int, vocab: int = 1 << 17, s: float = 1.1) -> np.ndarray:
    rng = np.random.default_rng(seed + 31337)
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return rng.choice(vocab, size=T, p=p).astype(np.int64)


def hash_routing(seed: int, token_ids: np.ndarray, n_experts: int, top_k: int):
    """Expert ids from a hash of the token id: SplitMix64 draws keyed by
    (seed, token id), reduced mod n_experts, duplicates rejected; route weights are a
    softmax of logits taken from the same draws. Repeated tokens repeat their route,
    which makes expert loads uneven."""
    T = token_ids.size
    ids = np.zeros((T, top_k), dtype=np.int32)
    logits = np.zeros((T, top_k), dtype=np.float64)
    cache = {}
    for t in range(T):
        tok = int(token_ids[t])
        if tok not in cache:
            chosen, lg = [], []
            i = 0
            while len(chosen) < top_k:
                w = words(seed, 0x7000_0000 | (tok & 0x0FFF_FFFF), i, 1)[0]
                i += 1
                e = int(w % np.uint64(n_experts))
                if e in chosen:
                    continue
                chosen.append(e)
                lg.append(float(w >> np.uint64(11)) * 2.0 ** -53 * 4.0 - 2.0)
            cache[tok] = (chosen, lg)
        ids[t], logits[t] = cache[tok]
    return ids, softmax_f32(logits)
