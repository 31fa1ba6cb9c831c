"""Pins of the CPU oracle against things other than itself: the pages' printed
figures, hand-worked blocks, library decoders (torch float8 / bfloat16 casts),
exact rational arithmetic on encoded blocks, closed forms and invariants."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, convert, formats, moe, mxfp8
from tests import encoders as enc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- element codecs

def test_e2m1_matches_ocp_table():
    g = load("e2m1_ocp.json")["magnitudes_by_code_0_to_7"]
    assert list(codecs.E2M1[:8]) == g
    assert list(codecs.E2M1[8:]) == [-v for v in g]
    assert math.copysign(1.0, codecs.E2M1[8]) == -1.0          # code 8 is -0


def test_e4m3_all_codes_match_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(codecs.E4M3), nan)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(codecs.E4M3[~nan], t[~nan])
    assert codecs.E4M3[0x7E] == 448.0 and codecs.E4M3[0x01] == 2.0 ** -9


def test_e8m0_all_codes_match_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(codecs.E8M0), nan) and nan[255] and nan.sum() == 1
    assert np.array_equal(codecs.E8M0[~nan], t[~nan])
    assert codecs.E8M0[127] == 1.0 and codecs.E8M0[0] == 2.0 ** -127


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    ours = codecs.bf16_to_f64(bits)
    fin = np.isfinite(t)
    assert np.array_equal(ours[fin], t[fin])


def test_e4m3_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000) * np.exp2(rng.uniform(-16, 9, 200000))
    v = v[np.abs(v) < 464]                                    # torch does not saturate above
    # exact ties between neighbouring codes, and -0 / small negatives
    fin = codecs.E4M3[np.isfinite(codecs.E4M3) & (codecs.E4M3 >= 0)]
    fin = np.unique(fin)
    ties = (fin[:-1] + fin[1:]) / 2
    v = np.concatenate([v, ties, -ties, [-0.0, -1e-9, 1e-9, 2.0 ** -10, 3 * 2.0 ** -11]])
    ours = codecs.f64_to_e4m3fn_rne(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_rne_saturates():
    assert codecs.f64_to_e4m3fn_rne(np.array([464.0, 1e6, -500.0])).tolist() == [0x7E, 0x7E, 0xFE]


# ---------------------------------------------------------------- sizes from the pages

def test_bits_per_weight_match_pages():
    g = load("page_figures.json")["bits_per_weight"]
    R, C = 2048, 4096
    for fmt, key in [(formats.MXFP4, "mxfp4"), (formats.NVFP4, "nvfp4"), (formats.Q2_K, "q2_k"),
                     (formats.IQ2_XXS, "iq2_xxs"), (formats.FP8_B128, "fp8_b128")]:
        nb = formats.packed_bytes(fmt, R, C)
        if fmt == formats.NVFP4:
            nb -= 4                                          # per-tensor scale_2, not per weight
        bpw = nb * 8 / (R * C)
        p = g[key]
        # the page prints the figure truncated or rounded to the stated decimals
        assert math.floor(bpw * 10 ** p["printed_decimals"] + 1e-9) / 10 ** p["printed_decimals"] == p["printed"] \
            or round(bpw, p["printed_decimals"]) == p["printed"], (key, bpw)
    assert formats.packed_bytes(formats.Q2_K, 1, 256) == 84
    assert formats.packed_bytes(formats.IQ2_XXS, 1, 256) == 66
    assert formats.packed_bytes(formats.MXFP4, 1, 32) == 17
    assert formats.packed_bytes(formats.NVFP4, 1, 16) == 9 + 4
    assert formats.packed_bytes(formats.FP8_B128, 128, 128) == 16385


def test_mixed_q2_payload_identity():
    g = load("page_figures.json")["mixed_q2_payload"]
    # gate, up in IQ2_XXS and down in Q2_K, three equal-sized matrices per expert
    n = 2048 * 4096
    bpw = (2 * formats.packed_bytes(formats.IQ2_XXS, 2048, 4096) + formats.packed_bytes(formats.Q2_K, 4096, 2048)) \
        * 8 / (3 * n)
    assert bpw == g["bits_per_weight"]
    assert round(g["routed_weights"] * bpw / 8 / 1e9, 2) == g["payload_gb"]


def test_model_shape_consistency():
    s = load("page_figures.json")["model_shape"]
    H, I, E, L, K = s["hidden_size"], 2048, s["routed_experts_per_layer"], s["decoder_layers"], s["top_k"]
    routed = 3 * H * I * E * L
    assert 270e9 < routed < 284e9                            # ~284 B total parameters
    assert 3 * H * I * K * L < 13e9                          # ~13 B active


def test_invalid_shapes_have_zero_size():
    assert formats.packed_bytes(formats.MXFP4, 4, 33) == 0
    assert formats.packed_bytes(formats.Q2_K, 4, 128) == 0
    assert formats.packed_bytes(formats.FP8_B128, 100, 128) == 0
    assert formats.packed_bytes(99, 4, 256) == 0


# ---------------------------------------------------------------- worked blocks

def test_worked_mxfp4():
    g = load("worked_blocks.json")["mxfp4"]
    nib = np.frombuffer(bytes.fromhex(g["nibble_bytes_hex"]), np.uint8)
    w = formats.dequant_mxfp4(nib, np.array(g["e8m0"], np.uint8), 1, 32)[0]
    assert w.tolist() == g["expected"]
    assert [math.copysign(1, v) for v in w] == [math.copysign(1, v) for v in g["expected"]]


def _blank_with(set_bytes, n):
    b = np.zeros(n, np.uint8)
    for k, v in set_bytes.items():
        b[int(k)] = v
    return b


def test_worked_nvfp4():
    g = load("worked_blocks.json")["nvfp4"]
    nib = bytearray(16)
    for k, c in enumerate(g["nibble_codes"]):
        enc.put_nibble(nib, k, c)
    w = formats.dequant_nvfp4(np.frombuffer(bytes(nib), np.uint8), np.array(g["e4m3"], np.uint8),
                              g["scale2"], 1, 32)[0]
    for k, v in g["expected_at"].items():
        assert w[int(k)] == v


def test_worked_q2_k():
    g = load("worked_blocks.json")["q2_k"]
    w = formats.dequant_q2_k(_blank_with(g["set_bytes"], 84), 1, 256)[0]
    for k, v in g["expected_at"].items():
        assert w[int(k)] == v, k


def test_worked_iq2_xxs():
    g = load("worked_blocks.json")["iq2_xxs"]
    grid = np.zeros((256, 8), np.uint8)
    for k, v in g["grid_entries"].items():
        grid[int(k)] = v
    w = formats.dequant_iq2_xxs(_blank_with(g["set_bytes"], 66), grid, 1, 256)[0]
    for k, v in g["expected_at"].items():
        assert w[int(k)] == v, k


def test_worked_fp8_b128():
    g = load("worked_blocks.json")["fp8_b128"]
    q = np.zeros((g["rows"], g["cols"]), np.uint8)
    for k, v in g["codes_at"].items():
        r, c = map(int, k.split(","))
        q[r, c] = v
    w = formats.dequant_fp8_b128(q, np.array(g["scales"], np.uint8), g["rows"], g["cols"])
    for k, v in g["expected_at"].items():
        r, c = map(int, k.split(","))
        assert w[r, c] == v


# ---------------------------------------------------------------- exact round trips

def _assert_exact(w, exact):
    w = np.asarray(w)
    flat = [x for row in exact for x in row] if isinstance(exact[0], list) else exact
    for a, b in zip(w.reshape(-1).tolist(), flat):
        assert Fraction(a) == b


@pytest.mark.parametrize("seed", range(3))
def test_roundtrip_mxfp4(seed):
    rng = np.random.default_rng(seed)
    rows, cols = 3, 64
    codes = rng.integers(0, 16, (rows, cols))
    E = rng.integers(0, 255, (rows, cols // 32))
    E[0, 0], E[1, 1] = 0, 254                                # subnormal and largest scales
    nib, e, exact = enc.encode_mxfp4(codes, E, rows, cols)
    _assert_exact(formats.dequant_mxfp4(nib, e, rows, cols), exact)


@pytest.mark.parametrize("seed", range(3))
def test_roundtrip_nvfp4(seed):
    rng = np.random.default_rng(seed)
    rows, cols = 2, 64
    codes = rng.integers(0, 16, (rows, cols))
    S = rng.integers(0, 0x7F, (rows, cols // 16))
    S[0, 0] = 0x01
    s2 = float(np.float32(rng.uniform(0.5, 2.0)))
    nib, s, exact = enc.encode_nvfp4(codes, S, s2, rows, cols)
    w = formats.dequant_nvfp4(nib, s, s2, rows, cols)
    _assert_exact(w, exact)
    # the one fp32 rounding of the device dequant
    f32 = formats.to_f32(w)
    for a, b in zip(f32.reshape(-1).tolist(), [x for r in exact for x in r]):
        assert a == float(np.float32(float(b)))


@pytest.mark.parametrize("seed", range(3))
def test_roundtrip_q2_k(seed):
    rng = np.random.default_rng(seed)
    blocks, exact = [], []
    for _ in range(2):
        q = rng.integers(0, 4, 256).tolist()
        sc = rng.integers(0, 16, 16).tolist()
        mn = rng.integers(0, 16, 16).tolist()
        d, dm = (np.array(rng.uniform(1e-3, 1e-2, 2), np.float16).view(np.uint16)).tolist()
        b, ex = enc.encode_q2_k_block(q, sc, mn, d, dm)
        blocks.append(b)
        exact.extend(ex)
    w = formats.dequant_q2_k(np.frombuffer(b"".join(blocks), np.uint8), 1, 512)
    _assert_exact(w, exact)


def test_q2_k_with_dmin_zero_is_scale_times_quant():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 4, 256).tolist()
    sc = rng.integers(0, 16, 16).tolist()
    mn = rng.integers(0, 16, 16).tolist()
    d = int(np.array([0.25], np.float16).view(np.uint16)[0])
    b, _ = enc.encode_q2_k_block(q, sc, mn, d, 0)
    w = formats.dequant_q2_k(np.frombuffer(b, np.uint8), 1, 256)[0]
    assert w.tolist() == [0.25 * sc[i // 16] * q[i] for i in range(256)]


@pytest.mark.parametrize("seed", range(3))
def test_roundtrip_iq2_xxs(seed):
    rng = np.random.default_rng(seed)
    grid = rng.integers(0, 256, (256, 8), dtype=np.uint8)
    gidx = rng.integers(0, 256, 32).tolist()
    neg = []
    for g in range(32):
        bits = rng.integers(0, 2, 8)
        if bits.sum() % 2:
            bits[rng.integers(0, 8)] ^= 1
        neg.extend(bool(x) for x in bits)
    scales = rng.integers(0, 16, 8).tolist()
    d = int(np.array([rng.uniform(1e-3, 1e-2)], np.float16).view(np.uint16)[0])
    b, exact = enc.encode_iq2_xxs_block(gidx, neg, scales, d, grid)
    w = formats.dequant_iq2_xxs(np.frombuffer(b, np.uint8), grid, 1, 256)
    _assert_exact(w, exact)


def test_iq2_sign_mask_has_even_weight():
    m = formats.iq2_sign_mask(np.arange(128))
    assert all(bin(int(x)).count("1") % 2 == 0 for x in m)
    assert len(set(m.tolist())) == 128


@pytest.mark.parametrize("seed", range(2))
def test_roundtrip_fp8_b128(seed):
    rng = np.random.default_rng(seed)
    rows, cols = 128, 256
    codes = rng.integers(0, 254, (rows, cols))
    codes = np.where(codes >= 0x7F, codes + 1, codes)
    S = rng.integers(0, 255, (1, 2))
    q, s, exact = enc.encode_fp8_b128(codes, S, rows, cols)
    w = formats.dequant_fp8_b128(q, s, rows, cols)
    # check a sample of rows exactly (the full Fraction table is slow)
    for r in (0, 1, 64, 127):
        _assert_exact(w[r:r + 1], [exact[r]])


# ---------------------------------------------------------------- MXFP4 -> NVFP4

@pytest.mark.parametrize("seed", range(4))
def test_mxfp4_to_nvfp4_is_lossless(seed):
    rng = np.random.default_rng(seed)
    rows, cols = 16, 256
    nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    lo = int(rng.integers(1, 200))
    e8 = rng.integers(lo, lo + 18, rows * cols // 32).astype(np.uint8)   # span <= 17
    nib2, e4, s2 = convert.mxfp4_to_nvfp4(nib, e8, rows, cols)
    assert nib2.tobytes() == nib.tobytes()
    a = formats.dequant_mxfp4(nib, e8, rows, cols)
    b = formats.dequant_nvfp4(nib2, e4, s2, rows, cols)
    assert np.array_equal(a, b) and np.array_equal(np.signbit(a), np.signbit(b))


def test_mxfp4_to_nvfp4_refuses_lossy():
    nib = np.zeros(16, np.uint8)
    with pytest.raises(convert.LossyConversion):                # span 18
        convert.mxfp4_to_nvfp4(np.zeros(32, np.uint8), np.array([100, 118], np.uint8), 1, 64)
    with pytest.raises(convert.LossyConversion):
        convert.mxfp4_to_nvfp4(nib, np.array([255], np.uint8), 1, 32)
    # a span of exactly 17 is still exact
    n2, e4, s2 = convert.mxfp4_to_nvfp4(np.full(32, 0x77, np.uint8), np.array([100, 117], np.uint8), 1, 64)
    assert np.array_equal(formats.dequant_nvfp4(n2, e4, s2, 1, 64),
                          formats.dequant_mxfp4(np.full(32, 0x77, np.uint8), np.array([100, 117], np.uint8), 1, 64))


# ---------------------------------------------------------------- MXFP8 activations

def test_mxfp8_codes_match_library_cast():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    codes, E = mxfp8.quantize(v)
    scale = np.ldexp(1.0, E.astype(np.int64) - 127)
    lib = torch.from_numpy(v / np.repeat(scale, 32, axis=1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, lib)


def test_mxfp8_scale_is_smallest_non_clipping_power_of_two():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((32, 512)) * np.exp2(rng.uniform(-30, 30, (32, 1)))
    _, E = mxfp8.quantize(v)
    amax = np.abs(v.reshape(32, 16, 32)).max(axis=2)
    s = np.ldexp(1.0, E.astype(np.int64) - 127)
    assert np.all(amax / s <= 448.0)
    assert np.all(amax / (s / 2) > 448.0)                     # one step smaller would clip
    assert np.all(amax / s >= 224.0)


def test_mxfp8_zero_block_and_dequant_error():
    v = np.zeros((1, 64))
    v[0, 32:] = np.linspace(-3, 5, 32)
    codes, E = mxfp8.quantize(v)
    assert E[0, 0] == 0 and np.all(codes[0, :32] == 0)
    back = mxfp8.dequantize(codes, E)
    s = 2.0 ** (int(E[0, 1]) - 127)
    big = np.abs(v[0, 32:]) >= 2.0 ** -6 * s
    rel = np.abs(back[0, 32:] - v[0, 32:])[big] / np.abs(v[0, 32:])[big]
    assert np.all(rel <= 2.0 ** -4)                           # half an e4m3 ulp


# ---------------------------------------------------------------- MoE layer

def test_silu_closed_forms():
    z = np.linspace(-30, 30, 601)
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(moe.silu(z) - moe.silu(-z), z, rtol=0, atol=1e-12)
    assert abs(moe.silu(np.array([50.0]))[0] - 50.0) < 1e-15
    assert abs(moe.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def _tiny_layer(seed, H=64, I=32, E=5):
    rng = np.random.default_rng(seed)
    mats = {}
    for p, (r, c) in enumerate([(I, H), (I, H), (H, I)]):
        for e in range(E):
            codes = rng.integers(0, 16, (r, c))
            S = rng.integers(120, 127, (r, c // 32))
            nib, s, exact = enc.encode_mxfp4(codes, S, r, c)
            mats[(p, e)] = (nib, s, exact, r, c)
    return mats


def test_moe_layer_matches_brute_force():
    mats = _tiny_layer(0)
    weight = moe.CachedWeights(lambda p, e: formats.dequant_mxfp4(mats[(p, e)][0], mats[(p, e)][1],
                                                                  mats[(p, e)][3], mats[(p, e)][4]))
    rng = np.random.default_rng(9)
    T, K = 2, 3
    x_bits = np.array(rng.standard_normal((T, 64)), np.float32).view(np.uint32) >> 16
    x_bits = x_bits.astype(np.uint16)
    ids = np.array([[0, 3, 4], [2, 2, 1]], np.int32)            # duplicate id in token 1
    rw = np.array([[0.5, 0.25, 0.25], [0.125, 0.375, 0.5]], np.float32)
    y, h = moe.moe_layer(x_bits, ids, rw, weight)

    def bf(b):
        return Fraction(float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]))

    for t in range(T):
        x = [bf(b) for b in x_bits[t]]
        yt = [0.0] * 64
        for k in range(K):
            e = int(ids[t, k])
            G, U, D = mats[(0, e)][2], mats[(1, e)][2], mats[(2, e)][2]
            g = [sum(G[i][j] * x[j] for j in range(64)) for i in range(32)]
            u = [sum(U[i][j] * x[j] for j in range(64)) for i in range(32)]
            hh = [float(g[i]) / (1.0 + math.exp(-float(g[i]))) * float(u[i]) for i in range(32)]
            assert np.allclose(h[t, k], hh, rtol=1e-13, atol=0)
            for i in range(64):
                yt[i] += float(rw[t, k]) * sum(float(D[i][j]) * hh[j] for j in range(32))
        assert moe.rel_err(y[t], np.array(yt)) < 1e-12


def test_one_hot_route_is_single_expert_ffn():
    mats = _tiny_layer(1)
    weight = moe.CachedWeights(lambda p, e: formats.dequant_mxfp4(mats[(p, e)][0], mats[(p, e)][1],
                                                                  mats[(p, e)][3], mats[(p, e)][4]))
    x = np.random.default_rng(2).standard_normal((1, 64)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y, _ = moe.moe_layer(xb, np.array([[3, 1, 0]], np.int32), np.array([[1, 0, 0]], np.float32), weight)
    X = codecs.bf16_to_f64(xb)[0]
    ref = weight(2, 3) @ (moe.silu(weight(0, 3) @ X) * (weight(1, 3) @ X))
    assert np.array_equal(y[0], ref)


def test_one_hot_activation_selects_a_column():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, (8, 64))
    S = rng.integers(120, 130, (8, 2))
    nib, s, exact = enc.encode_mxfp4(codes, S, 8, 64)
    W = formats.dequant_mxfp4(nib, s, 8, 64)
    for j in (0, 17, 63):
        xb = np.zeros((1, 64), np.uint16)
        xb[0, j] = 0x3F80                                       # bf16 1.0
        y = moe.linear(W, xb)[0]
        assert [Fraction(v) for v in y] == [exact[r][j] for r in range(8)]


def test_rel_err_floor():
    ref = np.array([1.0, -1.0, 1e-9])
    assert moe.rel_err(ref, ref) == 0.0
    assert abs(moe.rel_err(ref + np.array([0, 0, 1e-3]), ref) - 1e-3 / 1.0) < 1e-12 or \
        moe.rel_err(ref + np.array([0, 0, 1e-3]), ref) <= 1e-3 / np.sqrt(np.mean(ref ** 2)) + 1e-12


# ---------------------------------------------------------------- W4A8 prefill stages
# The prefill chain (1x Spark forum thread, second post: fp4 weights times E4M3
# activations) is checked stage by stage against moe.prefill_h / moe.prefill_y, so
# those two functions are pinned here against the layer (when quantisation is
# lossless) and against exact rational arithmetic.

def _mxfp8_exact_rows(rng, rows, K, e_lo=118, e_hi=132):
    """Random rows whose every 32-block is exactly E4M3 x 2^(E-127), with the block
    maximum in (224, 448] x 2^(E-127), so MXFP8 quantisation gives back exactly
    these codes and scales. Returns (codes, E, exact Fractions)."""
    codes = rng.integers(0, 0x7F, (rows, K)).astype(np.uint8)         # finite, both signs below
    codes[codes == 0x7F] = 0x7E
    codes |= (rng.integers(0, 2, (rows, K)) << 7).astype(np.uint8)
    codes[codes == 0x80] = 0                                          # -0 has no rational sign
    big = np.array([0x77, 0x78, 0x7A, 0x7C, 0x7E], np.uint8)          # 240, 256, 320, 384, 448
    for r in range(rows):
        for b in range(K // 32):
            blk = codes[r, 32 * b:32 * b + 32]
            mags = np.array([abs(enc.e4m3_frac(int(c))) for c in blk])
            if mags.max() <= 224:
                j = rng.integers(0, 32)
                blk[j] = big[rng.integers(0, big.size)] | (blk[j] & 0x80)
    E = rng.integers(e_lo, e_hi, (rows, K // 32)).astype(np.uint8)
    exact = [[enc.e4m3_frac(int(codes[r, c])) * enc.pow2_frac(int(E[r, c // 32]) - 127) for c in range(K)]
             for r in range(rows)]
    return codes, E, exact


def _frac_bf16_bits(v: Fraction) -> int:
    b = int(np.array([float(v)], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0 and Fraction(float(v)) == v
    return b >> 16


def test_prefill_h_equals_layer_h_on_exact_mxfp8_input():
    mats = _tiny_layer(5, E=6)
    weight = moe.CachedWeights(lambda p, e: formats.dequant_mxfp4(mats[(p, e)][0], mats[(p, e)][1],
                                                                  mats[(p, e)][3], mats[(p, e)][4]))
    rng = np.random.default_rng(21)
    T, K = 3, 2
    codes, E, exact = _mxfp8_exact_rows(rng, T, 64, 110, 118)
    x_bits = np.array([[_frac_bf16_bits(v) for v in row] for row in exact], np.uint16)
    xq, xs = mxfp8.quantize(codecs.bf16_to_f64(x_bits))
    assert np.array_equal(xq, codes) and np.array_equal(xs, E)        # lossless by construction
    ids = np.array([[0, 5], [3, 1], [4, 2]], np.int32)
    rw = np.array([[0.7, 0.3], [0.25, 0.75], [0.6, 0.4]], np.float32)
    _, h_ref = moe.moe_layer(x_bits, ids, rw, weight)
    h = moe.prefill_h(xq, xs, ids, weight)
    assert np.array_equal(h, h_ref)


def test_prefill_y_equals_layer_combine_on_exact_mxfp8_h():
    # With h exactly MXFP8, prefill_y is the layer's route-weighted down combine.
    mats = _tiny_layer(6, E=5)
    weight = moe.CachedWeights(lambda p, e: formats.dequant_mxfp4(mats[(p, e)][0], mats[(p, e)][1],
                                                                  mats[(p, e)][3], mats[(p, e)][4]))
    rng = np.random.default_rng(22)
    T, K = 3, 2
    hq, hs, _ = _mxfp8_exact_rows(rng, T * K, 32)
    Hh = mxfp8.dequantize(hq, hs)
    rq, rs = mxfp8.quantize(Hh)
    assert np.array_equal(rq, hq) and np.array_equal(rs, hs)
    ids = np.array([[1, 4], [0, 2], [3, 0]], np.int32)
    rw = np.array([[0.9, 0.1], [0.2, 0.8], [0.35, 0.65]], np.float32)
    y = moe.prefill_y(hq, hs, ids, rw, weight)
    ref = np.zeros((T, 64))
    for t in range(T):
        for k in range(K):
            ref[t] += float(rw[t, k]) * (weight(moe.DOWN, ids[t, k]) @ Hh[t * K + k])
    assert np.array_equal(y, ref)


def test_prefill_stages_match_exact_rationals():
    # T = 2 tokens, K = 2 distinct experts per token, asymmetric route weights: a
    # swapped gate/up, a k*T + t row order for h or a dropped route weight all move
    # the result far beyond the tolerance below.
    H, I = 64, 32
    mats = _tiny_layer(7, H=H, I=I, E=4)
    weight = moe.CachedWeights(lambda p, e: formats.dequant_mxfp4(mats[(p, e)][0], mats[(p, e)][1],
                                                                  mats[(p, e)][3], mats[(p, e)][4]))
    rng = np.random.default_rng(23)
    T, K = 2, 2
    xq, xs, xe = _mxfp8_exact_rows(rng, T, H, 110, 118)
    ids = np.array([[2, 0], [1, 3]], np.int32)
    rw = np.array([[0.8125, 0.1875], [0.375, 0.625]], np.float32)
    h = moe.prefill_h(xq, xs, ids, weight)
    for t in range(T):
        for k in range(K):
            G, U = mats[(0, int(ids[t, k]))][2], mats[(1, int(ids[t, k]))][2]
            for i in range(I):
                g = sum(G[i][j] * xe[t][j] for j in range(H))
                u = sum(U[i][j] * xe[t][j] for j in range(H))
                want = float(g) / (1.0 + math.exp(-float(g))) * float(u)
                assert abs(h[t, k, i] - want) <= 1e-13 * max(1.0, abs(want))
    hq, hs, he = _mxfp8_exact_rows(rng, T * K, I, 118, 126)
    y = moe.prefill_y(hq, hs, ids, rw, weight)
    for t in range(T):
        for r in range(H):
            want = Fraction(0)
            for k in range(K):
                D = mats[(2, int(ids[t, k]))][2]
                want += Fraction(float(rw[t, k])) * sum(D[r][j] * he[t * K + k][j] for j in range(I))
            assert abs(y[t, r] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))


# ---------------------------------------------------------------- MXFP8 and V4.1 FP8 tiles

def test_worked_fp8_b32():
    g = load("worked_blocks.json")["fp8_b32"]
    q = np.zeros((g["rows"], g["cols"]), np.uint8)
    for k, v in g["codes_at"].items():
        r, c = map(int, k.split(","))
        q[r, c] = v
    w = formats.dequant_fp8_b32(q, np.array(g["scales"], np.uint8), g["rows"], g["cols"])
    for k, v in g["expected_at"].items():
        r, c = map(int, k.split(","))
        assert w[r, c] == v, k


def test_worked_mxfp8():
    g = load("worked_blocks.json")["mxfp8"]
    q = np.zeros((g["rows"], g["cols"]), np.uint8)
    for k, v in g["codes_at"].items():
        r, c = map(int, k.split(","))
        q[r, c] = v
    w = formats.dequant_mxfp8(q, np.array(g["scales"], np.uint8), g["rows"], g["cols"])
    for k, v in g["expected_at"].items():
        r, c = map(int, k.split(","))
        assert w[r, c] == v, k


def test_fp8_tile_sizes_and_bits_per_weight():
    t = load("page_figures.json")["fp8_tile_sizes"]
    H = 4096
    assert formats.packed_bytes(formats.FP8_B128, H, H) == H * H + (H // t["v4"]) ** 2
    assert formats.packed_bytes(formats.FP8_B32, H, H) == H * H + (H // t["v4_1"]) ** 2
    assert formats.packed_bytes(formats.FP8_B32, 4096, 2048) * 8 / (4096 * 2048) == 8 + 8 / 1024
    # MXFP8: an 8-bit element plus an 8-bit shared scale per 32 elements
    assert formats.packed_bytes(formats.MXFP8, 2048, 4096) * 8 / (2048 * 4096) == 8.25
    assert formats.packed_bytes(formats.FP8_B32, 48, 64) == 0       # rows not a multiple of 32
    assert formats.packed_bytes(formats.MXFP8, 3, 48) == 0          # cols not a multiple of 32


@pytest.mark.parametrize("seed", range(2))
def test_roundtrip_mxfp8(seed):
    rng = np.random.default_rng(40 + seed)
    rows, cols = 4, 96
    codes = rng.integers(0, 254, (rows, cols))
    codes = np.where(codes >= 0x7F, codes + 1, codes)           # skip 0x7f (NaN)
    E = rng.integers(0, 255, (rows, cols // 32))
    q, s, exact = enc.encode_mxfp8(codes, E, rows, cols)
    _assert_exact(formats.dequant_mxfp8(q, s, rows, cols), exact)


@pytest.mark.parametrize("seed", range(2))
def test_roundtrip_fp8_b32(seed):
    rng = np.random.default_rng(50 + seed)
    rows, cols = 64, 96
    codes = rng.integers(0, 254, (rows, cols))
    codes = np.where(codes >= 0x7F, codes + 1, codes)
    S = rng.integers(0, 255, (rows // 32, cols // 32))
    q, s, exact = enc.encode_fp8_b32(codes, S, rows, cols)
    w = formats.dequant_fp8_b32(q, s, rows, cols)
    for r in (0, 31, 32, 63):
        _assert_exact(w[r:r + 1], [exact[r]])


def test_fp8_b32_reduces_to_b128_when_tiles_agree():
    rng = np.random.default_rng(60)
    q = rng.integers(0, 0x7F, (256, 256)).astype(np.uint8)
    S128 = rng.integers(110, 140, (2, 2)).astype(np.uint8)
    S32 = np.repeat(np.repeat(S128, 4, axis=0), 4, axis=1)
    assert np.array_equal(formats.dequant_fp8_b32(q, S32, 256, 256), formats.dequant_fp8_b128(q, S128, 256, 256))
    # the page's hazard: the same scale bytes read with the other tile size rescale weights
    S32b = rng.integers(110, 140, (8, 8)).astype(np.uint8)
    as128 = formats.dequant_fp8_b128(q, S32b[:2, :2], 256, 256)
    assert not np.array_equal(formats.dequant_fp8_b32(q, S32b, 256, 256), as128)


def test_mxfp8_equals_fp8_tiles_with_per_row_scales():
    # an FP8 block-32 tensor is an MXFP8 tensor whose scales repeat over 32 rows
    rng = np.random.default_rng(61)
    q = rng.integers(0, 0x7F, (64, 128)).astype(np.uint8)
    S = rng.integers(100, 150, (2, 4)).astype(np.uint8)
    E = np.repeat(S, 32, axis=0)
    assert np.array_equal(formats.dequant_fp8_b32(q, S, 64, 128), formats.dequant_mxfp8(q, E, 64, 128))


# ---------------------------------------------------------------- NVFP4 -> MXFP4

@pytest.mark.parametrize("seed", range(4))
def test_nvfp4_to_mxfp4_inverts_the_forward_conversion(seed):
    rng = np.random.default_rng(70 + seed)
    rows, cols = 8, 256
    nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    lo = int(rng.integers(1, 200))
    e8 = rng.integers(lo, lo + 18, rows * cols // 32).astype(np.uint8)
    n2, e4, s2 = convert.mxfp4_to_nvfp4(nib, e8, rows, cols)
    n3, e8b = convert.nvfp4_to_mxfp4(n2, e4, s2, rows, cols)
    assert n3.tobytes() == nib.tobytes() and e8b.tobytes() == e8.tobytes()
    assert np.array_equal(formats.dequant_mxfp4(n3, e8b, rows, cols), formats.dequant_nvfp4(n2, e4, s2, rows, cols))


def test_nvfp4_to_mxfp4_refuses_what_e8m0_cannot_hold():
    nib = np.zeros(16, np.uint8)
    ok = np.full(2, 0x38, np.uint8)                                  # 1.0 on both halves
    n, e = convert.nvfp4_to_mxfp4(nib, ok, 0.25, 1, 32)
    assert e.tolist() == [[125]]                                     # 1.0 * 2^-2
    for e4, s2 in [(np.array([0x38, 0x40], np.uint8), 1.0),         # halves differ
                   (np.full(2, 0x3C, np.uint8), 1.0),               # 1.5: not a power of two
                   (ok, 1.5),                                        # scale_2 not a power of two
                   (np.zeros(2, np.uint8), 1.0),                     # zero scale
                   (np.full(2, 0xB8, np.uint8), 1.0),                # negative scale
                   (ok, 2.0 ** -128)]:                               # below e8m0's range
        with pytest.raises(convert.LossyConversion):
            convert.nvfp4_to_mxfp4(nib, e4, s2, 1, 32)
