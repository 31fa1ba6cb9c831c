"""GPU parity of the dense FP8 formats with power-of-two block scales (MXFP8,
MXFP8 pre-stored in the matrix instruction's operand order, FP8 with 32 x 32
tiles) and of the device MXFP4 <-> NVFP4 re-encodes, against the CPU oracle:
dequantised weights bit-exact, linear outputs within the projection tolerance,
conversions byte-exact (including the tensors they must refuse)."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth
from oracle import convert, formats, moe
from tests.helpers import TOL, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_tensor(bits):
    return cuda(bits.view(np.int16)).view(torch.bfloat16)


def f32_bits_equal(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))


def fp8_planes(fmt, rows, cols, seed, codes=None, scales=None):
    """Row-major source planes: E4M3 codes over the 254 finite codes, e8m0 scales in
    119..123 (2^-8 .. 2^-4) unless given."""
    rng = np.random.default_rng(seed)
    if codes is None:
        codes = synth.field_bytes(seed, 1, synth.FIELD_E4M3_FINITE, 0, rows * cols)
    if scales is None:
        n = rows * cols // 32 if fmt in (mq.FMT_MXFP8, mq.FMT_MXFP8_TILED) else (rows // 32) * (cols // 32)
        scales = rng.integers(119, 124, n).astype(np.uint8)
    return np.ascontiguousarray(codes, np.uint8), np.ascontiguousarray(scales, np.uint8)


def device_weight(fmt, rows, cols, planes_per_expert):
    """A device Weight; MXFP8_TILED is made on the device from the row-major planes."""
    src = mq.FMT_MXFP8 if fmt == mq.FMT_MXFP8_TILED else fmt
    E = len(planes_per_expert)
    W = mq.Weight.empty(src, rows, cols, E)
    for e, (q, s) in enumerate(planes_per_expert):
        W.data[e * W.expert_stride:e * W.expert_stride + q.size].copy_(torch.from_numpy(q))
        W.scales[e * W.scale_expert_stride:e * W.scale_expert_stride + s.size].copy_(torch.from_numpy(s))
    if fmt != mq.FMT_MXFP8_TILED:
        return W
    assert W.expert_stride == rows * cols and W.scale_expert_stride == rows * cols // 32
    td, ts = mq.mxfp8_to_tiled(W.data, W.scales, rows, cols, E)
    return mq.Weight(mq.FMT_MXFP8_TILED, rows, cols, E, td, ts, expert_stride=W.expert_stride,
                     scale_expert_stride=W.scale_expert_stride)


def oracle_fmt(fmt):
    return formats.MXFP8 if fmt in (mq.FMT_MXFP8, mq.FMT_MXFP8_TILED) else formats.FP8_B32


@pytest.mark.parametrize("fmt", [mq.FMT_MXFP8, mq.FMT_MXFP8_TILED, mq.FMT_FP8_B32])
def test_dense_fp8_dequant_bit_exact(fmt):
    """Every E4M3 code and e8m0 codes 0, 1, 127, 254 and 255 (NaN), on a 2-expert
    tensor (the second expert is read)."""
    say("dense fp8 dequant", fmt)
    rows, cols = 64, 1024
    rng = np.random.default_rng(fmt)
    planes = []
    for e in range(2):
        q = np.tile(np.arange(256, dtype=np.uint8), rows * cols // 256)
        rng.shuffle(q)
        _, s = fp8_planes(fmt, rows, cols, 10 + e)
        s = s.copy()
        s[:5] = [0, 1, 127, 254, 255]
        planes.append((q, s))
    W = device_weight(fmt, rows, cols, planes)
    got = mq.dequant(W, 1).cpu().numpy()
    want = formats.to_f32(formats.dequant(oracle_fmt(fmt), list(planes[1]), rows, cols))
    assert f32_bits_equal(got, want)


@pytest.mark.parametrize("fmt,rows,cols", [(mq.FMT_MXFP8, 4096, 4096), (mq.FMT_MXFP8_TILED, 4096, 4096),
                                           (mq.FMT_FP8_B32, 4096, 4096), (mq.FMT_MXFP8, 48, 640),
                                           (mq.FMT_MXFP8_TILED, 32, 1536), (mq.FMT_FP8_B32, 64, 384),
                                           (mq.FMT_MXFP8, 128, 8192), (mq.FMT_MXFP8_TILED, 16, 512),
                                           (mq.FMT_FP8_B32, 96, 128)])
def test_dense_fp8_linear(fmt, rows, cols):
    """y = W x on the block-scaled FP8 instruction: token counts that fill part of
    one 8-token pass, exactly one, one plus one token, several (and at K = 8192,
    where a pass holds four tokens); K from one 128-wide step (fewer steps than
    waves) to 64 steps."""
    say("dense fp8 linear", fmt, rows, cols)
    planes = [fp8_planes(fmt, rows, cols, 100 + e + rows) for e in range(2)]
    W = device_weight(fmt, rows, cols, planes)
    Wd = formats.dequant(oracle_fmt(fmt), list(planes[1]), rows, cols)
    rng = np.random.default_rng(rows + cols + fmt)
    for T in (1, 2, 7, 8, 9, 17, 64):
        x = synth.activations_bf16(int(rng.integers(1 << 30)), T, cols)
        y = mq.linear(W, 1, x_tensor(x)).cpu().numpy()
        err = rel_err(y, moe.linear(Wd, x))
        assert err < TOL, (fmt, rows, cols, T, err)


def test_tiled_and_row_major_agree_bitwise_with_outliers():
    """The pre-stored order changes only where the bytes are read from: outputs are
    bit-identical to the row-major layout's. x holds one outlier 2^8 .. 2^20 times
    the rest in each 32-block, which the two-term split must still carry."""
    say("tiled vs row-major")
    rows, cols = 1024, 4096
    planes = [fp8_planes(mq.FMT_MXFP8, rows, cols, 300)]
    Wr = device_weight(mq.FMT_MXFP8, rows, cols, planes)
    Wt = device_weight(mq.FMT_MXFP8_TILED, rows, cols, planes)
    Wd = formats.dequant(formats.MXFP8, list(planes[0]), rows, cols)
    rng = np.random.default_rng(301)
    x = synth.activations_bf16(302, 12, cols)
    xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
    for t in range(12):
        for b in range(cols // 32):
            j = 32 * b + int(rng.integers(32))
            xf[t, j] = np.float32(np.sign(xf[t, j] or 1.0) * 2.0 ** (8 + (b + t) % 13))
    xo = synth.bf16_bits_from_f32(xf)
    for xb in (x, xo):
        yr = mq.linear(Wr, 0, x_tensor(xb)).cpu().numpy()
        yt = mq.linear(Wt, 0, x_tensor(xb)).cpu().numpy()
        assert np.array_equal(yr.view(np.uint32), yt.view(np.uint32))
        assert rel_err(yr, moe.linear(Wd, xb)) < TOL


def test_dense_fp8_shapes_refused():
    say("dense fp8 refusals")
    W = device_weight(mq.FMT_MXFP8, 48, 640, [fp8_planes(mq.FMT_MXFP8, 48, 640, 5)])
    bad = mq.Weight(mq.FMT_MXFP8_TILED, 48, 640, 1, W.data, W.scales)     # cols not a multiple of 512
    with pytest.raises(mq.MoeqError):
        mq.linear(bad, 0, x_tensor(synth.activations_bf16(1, 1, 640)))
    # a routed layer cannot use the dense-only formats
    g = device_weight(mq.FMT_MXFP8, 512, 1024, [fp8_planes(mq.FMT_MXFP8, 512, 1024, 6)])
    d = device_weight(mq.FMT_MXFP8, 1024, 512, [fp8_planes(mq.FMT_MXFP8, 1024, 512, 7)])
    layer = mq.Layer(1024, 512, 1, 1, g, g, d)
    with pytest.raises((mq.MoeqError, ValueError)):
        mq.expert_forward(layer, x_tensor(synth.activations_bf16(1, 1, 1024)), cuda(np.zeros((1, 1), np.int32)),
                          cuda(np.ones((1, 1), np.float32)))


def test_device_mxfp4_nvfp4_round_trip_and_refusals():
    """Four tensors: two convertible, one with an exponent span of 18, one with a NaN
    scale. The convertible ones must match the oracle byte for byte (and convert
    back to the original bytes); the others keep their outputs untouched."""
    say("device mxfp4 <-> nvfp4")
    rows, cols, n = 256, 1024, 4
    rng = np.random.default_rng(77)
    nib = rng.integers(0, 256, n * rows * cols // 2, dtype=np.uint8)
    e8 = rng.integers(110, 128, n * rows * cols // 32).astype(np.uint8)   # span 17
    nb = rows * cols // 32
    e8[2 * nb + 5] = 92                                                      # tensor 2: span 35
    e8[3 * nb + 9] = 255                                                     # tensor 3: NaN
    nib_o, e4, s2, st = mq.mxfp4_to_nvfp4_device(cuda(nib), cuda(e8), rows, cols, n)
    nib_o, e4, s2, st = nib_o.cpu().numpy(), e4.cpu().numpy(), s2.cpu().numpy(), st.cpu().numpy()
    assert st.tolist() == [0, 0, 1, 1]
    for t in range(2):
        want_n, want_e4, want_s2 = convert.mxfp4_to_nvfp4(nib[t * rows * cols // 2:(t + 1) * rows * cols // 2],
                                                           e8[t * nb:(t + 1) * nb], rows, cols)
        assert nib_o[t * rows * cols // 2:(t + 1) * rows * cols // 2].tobytes() == want_n.tobytes()
        assert e4[t * 2 * nb:(t + 1) * 2 * nb].tobytes() == want_e4.tobytes()
        assert np.float32(s2[t]).tobytes() == np.float32(want_s2).tobytes()
    for t in (2, 3):
        with pytest.raises(convert.LossyConversion):
            convert.mxfp4_to_nvfp4(nib[:rows * cols // 2], e8[t * nb:(t + 1) * nb], rows, cols)
        assert not e4[t * 2 * nb:(t + 1) * 2 * nb].any() and s2[t] == 0
        assert not nib_o[t * rows * cols // 2:(t + 1) * rows * cols // 2].any()
    # back to MXFP4: tensors 0 and 1 return to their original bytes; a tensor whose
    # halves differ and one whose scale_2 is not a power of two are refused
    e4b = e4.copy()
    e4b[2 * 2 * nb:3 * 2 * nb] = e4[:2 * nb]
    e4b[3 * 2 * nb:] = e4[:2 * nb]
    e4b[2 * 2 * nb + 7] ^= 0x08                                              # tensor 2: halves differ
    s2b = s2.copy()
    s2b[2] = s2[0]
    s2b[3] = np.float32(1.5)                                                 # tensor 3: scale_2 not 2^k
    nib_m, e8m, st2 = mq.nvfp4_to_mxfp4_device(cuda(nib_o), cuda(e4b), cuda(s2b), rows, cols, n)
    nib_m, e8m, st2 = nib_m.cpu().numpy(), e8m.cpu().numpy(), st2.cpu().numpy()
    assert st2.tolist() == [0, 0, 1, 1]
    for t in range(2):
        assert e8m[t * nb:(t + 1) * nb].tobytes() == e8[t * nb:(t + 1) * nb].tobytes()
        assert nib_m[t * rows * cols // 2:(t + 1) * rows * cols // 2].tobytes() == \
            nib[t * rows * cols // 2:(t + 1) * rows * cols // 2].tobytes()
        on, oe = convert.nvfp4_to_mxfp4(nib_o[:rows * cols // 2], e4b[t * 2 * nb:(t + 1) * 2 * nb], s2b[t], rows, cols)
        assert oe.tobytes() == e8m[t * nb:(t + 1) * nb].tobytes()
    for t in (2, 3):
        with pytest.raises(convert.LossyConversion):
            convert.nvfp4_to_mxfp4(nib_o[:rows * cols // 2], e4b[t * 2 * nb:(t + 1) * 2 * nb], s2b[t], rows, cols)
        assert not e8m[t * nb:(t + 1) * nb].any()
    # in place: the nibble plane is left as it is
    buf = cuda(nib[:rows * cols // 2].copy())
    out, _, _, st3 = mq.mxfp4_to_nvfp4_device(buf, cuda(e8[:nb]), rows, cols, 1, nib_out=buf)
    assert int(st3.item()) == 0 and out.data_ptr() == buf.data_ptr()
    assert buf.cpu().numpy().tobytes() == nib[:rows * cols // 2].tobytes()
