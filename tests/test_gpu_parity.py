"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: dequantised weights bit-exact (the format's exact value rounded once to
fp32); MXFP8 codes and scales bit-exact; projections (h and y) within max
relative error 2e-3 of the float64 oracle (elementwise, floored at the output
RMS). Every input is seeded and synthetic.
"""
import sys

import numpy as np
import pytest

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from oracle import formats, moe, mxfp8
from tests.helpers import TOL, oracle_weight_fn, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def f32_bits_equal(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))


def upload_weight(fmt, rows, cols, planes_per_expert, scale2=None, grid=None):
    E = len(planes_per_expert)
    W = mq.Weight.empty(fmt, rows, cols, E)
    for e, planes in enumerate(planes_per_expert):
        if fmt in (mq.FMT_Q2_K, mq.FMT_IQ2_XXS):
            d, s = mq.pack_ggml(fmt, planes[0], rows, cols)
        else:
            d, s = planes[0].reshape(-1), planes[1].reshape(-1)
        W.data[e * W.expert_stride:e * W.expert_stride + d.size].copy_(torch.from_numpy(d))
        W.scales[e * W.scale_expert_stride:e * W.scale_expert_stride + s.size].copy_(torch.from_numpy(s))
    if fmt == mq.FMT_NVFP4:
        W.scale2.copy_(torch.from_numpy(np.asarray(scale2, np.float32)))
    if fmt == mq.FMT_IQ2_XXS:
        W.grid = torch.from_numpy(np.ascontiguousarray(grid, np.uint8).reshape(-1)).cuda()
    return W


def upload_layer(spec):
    """Device layer from host-generated source planes (no device fill involved)."""
    grid = workloads.host_grid()
    ws = []
    for p in range(3):
        fmt, rows, cols = spec.proj(p)
        planes = [workloads.host_source_planes(spec, p, e) for e in range(spec.n_experts)]
        ws.append(upload_weight(fmt, rows, cols, planes, workloads.host_scale2(spec, p), grid))
    return mq.Layer(spec.hidden, spec.inter, spec.n_experts, spec.top_k, *ws)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_tensor(bits):
    return cuda(bits.view(np.int16)).view(torch.bfloat16)


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("field", [0, 1, 2, 3, 4, 5])
def test_device_fill_matches_host_generator(field):
    say("fill", field)
    bs = {4: 84, 5: 66}.get(field, 1)
    tab = cuda(synth.d_table().astype(np.int16))
    for off, n in [(0, 84 * 66 * 40), (bs * 1000, bs * 977), (13 * (bs == 1), 5000 * bs)]:
        dev = torch.empty(n, dtype=torch.uint8, device="cuda")
        mq.synth_fill(dev, 77, 0x123, off, field, tab)
        torch.cuda.synchronize()
        host = synth.field_bytes(77, 0x123, field, off, n)
        assert np.array_equal(dev.cpu().numpy(), host), (field, off, n)


# ---------------------------------------------------------------- dequant

def _edge_planes(fmt, rows, cols, rng):
    if fmt == mq.FMT_MXFP4:
        nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
        e = rng.integers(0, 256, rows * cols // 32, dtype=np.uint8)
        e[:6] = [0, 1, 127, 254, 255, 2]
        return [nib, e]
    if fmt == mq.FMT_NVFP4:
        nib = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
        e = np.arange(rows * cols // 16, dtype=np.int64) % 256
        return [nib, e.astype(np.uint8)]
    if fmt == mq.FMT_FP8_B128:
        q = (np.arange(rows * cols) % 256).astype(np.uint8)
        rng.shuffle(q)
        s = rng.integers(100, 150, (rows // 128) * (cols // 128), dtype=np.uint8)
        s[0] = 0
        if s.size > 1:
            s[1] = 255
        return [q, s]
    bs = 84 if fmt == mq.FMT_Q2_K else 66
    b = rng.integers(0, 256, rows * (cols // 256) * bs, dtype=np.uint8).reshape(-1, bs)
    dpos = [80, 82] if fmt == mq.FMT_Q2_K else [0]
    for p in dpos:   # finite fp16 d / dmin
        v = rng.uniform(-0.05, 0.05, b.shape[0]).astype(np.float16).view(np.uint8).reshape(-1, 2)
        b[:, p:p + 2] = v
    return [b.reshape(-1)]


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_dequant_bit_exact_edge_codes(fmt):
    say("dequant edge", fmt)
    rng = np.random.default_rng(fmt)
    rows, cols = (256, 512)
    grid = rng.integers(0, 256, (256, 8), dtype=np.uint8)
    planes = [_edge_planes(fmt, rows, cols, rng) for _ in range(2)]
    s2 = np.array([0.7, 1.9], np.float32)
    W = upload_weight(fmt, rows, cols, planes, s2, grid)
    for e in range(2):
        got = mq.dequant(W, e).cpu().numpy()
        ref = formats.to_f32(formats.dequant(fmt, planes[e], rows, cols, scale2=float(s2[e]), grid=grid))
        assert f32_bits_equal(got, ref), (fmt, e)


WORKLOAD_DEQ = [("mxfp4_layer", (0, 1, 2)), ("nvfp4_q2k", (0, 2)), ("iq2_q2k_43", (0, 2))]


@pytest.mark.parametrize("name,projs", WORKLOAD_DEQ)
def test_dequant_full_size_device_filled(name, projs):
    """Full-size layer filled on the device; sampled experts bit-exact vs the oracle
    decoding host-regenerated bytes (pins the device fill and repack too)."""
    say("dequant full", name)
    spec = workloads.WORKLOADS[name].spec
    grid = workloads.host_grid()
    for p in projs:
        fmt, rows, cols = spec.proj(p)
        W = workloads.fill_weight(mq, spec, p, fmt, rows, cols, spec.n_experts)
        s2 = workloads.host_scale2(spec, p)
        for e in (0, 137, spec.n_experts - 1):
            got = mq.dequant(W, e).cpu().numpy()
            planes = workloads.host_source_planes(spec, p, e)
            ref = formats.to_f32(formats.dequant(fmt, planes, rows, cols, scale2=float(s2[e]), grid=grid))
            assert f32_bits_equal(got, ref), (name, p, e)
        del W
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- MXFP8 quantisation

@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_quantize_mxfp8_bit_exact(kind):
    say("mxfp8", kind)
    rng = np.random.default_rng(11)
    T, K = 37, 512
    v = (rng.standard_normal((T, K)) * np.exp2(rng.integers(-30, 30, (T, 1)))).astype(np.float32)
    v[0, :32] = 0.0                       # all-zero block
    v[1, :32] = -0.0
    v[2, 32:64] = 448.0                   # max exactly representable
    v[3, :32] = np.float32(2.0 ** -130)   # subnormal block maximum
    v[4, 5] = -1e-30                      # tiny negative in a normal block
    v[5, :32] = 2.0 ** 120                # large scale
    # block maximum 448 (scale 1): exact halfway points between E4M3 neighbours, which
    # round to the even code (1.0625 -> 1, 1.1875 -> 1.25, 17 -> 16, 19 -> 20, and
    # the subnormal 3 2^-10 -> 2^-8), with their negatives
    ties = np.array([1.0625, 1.1875, 17.0, 19.0, 3.0 * 2.0 ** -10, 0.5 + 2.0 ** -5], np.float32)
    v[6, :32] = 0.0
    v[6, 0] = 448.0
    v[6, 1:1 + ties.size] = ties
    v[6, 1 + ties.size:1 + 2 * ties.size] = -ties
    if kind == "bf16":
        bits = synth.bf16_bits_from_f32(v)
        x = x_tensor(bits)
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        x = cuda(v)
        vals = v.astype(np.float64)
    q, e = mq.quantize_mxfp8(x)
    rq, re_ = mxfp8.quantize(vals)
    assert np.array_equal(e.cpu().numpy(), re_)
    assert np.array_equal(q.cpu().numpy(), rq)


# ---------------------------------------------------------------- decode layer parity

SMALL = [
    # (fmt gate/up, fmt down, H, I, E, K)
    (1, 1, 1024, 512, 8, 3),
    (1, 1, 1056, 288, 5, 2),    # 33 and 9 chunks per row: masked lanes, ragged row tiles
    (2, 3, 1024, 512, 6, 3),
    (4, 3, 768, 512, 6, 3),
    (3, 4, 512, 768, 4, 2),
    (5, 5, 512, 256, 4, 2),
    (2, 2, 640, 384, 4, 4),
    (1, 1, 1536, 256, 4, 2),    # bs=1 MXFP4 gate/up on the matrix unit: the fourth wave gets no K step
    (1, 1, 512, 128, 3, 2),     # ... and a single wave of K steps
    (1, 1, 1024, 512, 16, 8),   # bs=1 MXFP4 down on the matrix unit with its largest work-group (8 slots)
    (1, 1, 1024, 512, 16, 10),  # more slots than it takes: the GEMV path
    (1, 1, 1024, 512, 12, 6),   # bs=1 MXFP4 matrix-unit kernels at the full layer's top-6
    (1, 1, 2048, 1024, 8, 2),   # ... and with two slots
    (2, 3, 2048, 1024, 4, 2),   # NVFP4 gate/up + Q2_K down, intermediate 1024
    (2, 1, 1536, 288, 4, 2),    # bs=1 NVFP4 gate/up on the matrix unit: the fourth wave gets no K step
    (2, 1, 512, 128, 3, 2),     # ... and a single wave of K steps
    (2, 3, 4096, 256, 4, 2),    # K = 4096 in NVFP4: two chunks per lane; at T = 16 the 2-token gate/up tiles
    (1, 1, 4096, 256, 4, 2),    # ... and in MXFP4
    (1, 1, 8192, 128, 4, 2),    # K = 8192: four chunks per lane (one-token gate/up tiles at any T)
]


@pytest.mark.parametrize("case", SMALL)
@pytest.mark.parametrize("T", [1, 3, 16])
def test_forward_small_layers(case, T):
    fg, fd, H, I, E, K = case
    say("forward small", case, T)
    spec = workloads.LayerSpec(H, I, E, K, fg, fd, seed=1234 + H + I + fg * 7 + fd)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(spec.seed + T, T, E, K)
    x = synth.activations_bf16(spec.seed + 5 * T, T, H)
    ref_y, ref_h = moe.moe_layer(x, ids, rw, oracle_weight_fn(spec))
    xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, xt, it, rt, ws=ws).cpu().numpy()
    if T > 1:
        mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, xt, it, ws=ws).cpu().numpy()
    y2 = mq.down(layer, torch.from_numpy(h).cuda(), it, rt, ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    assert rel_err(h.reshape(T, K, I), ref_h) < TOL
    assert rel_err(y, ref_y) < TOL
    assert rel_err(y2, ref_y) < TOL
    assert rel_err(y, y2) < 1e-5          # the layer call vs its stages called one by one


@pytest.mark.parametrize("T,I", [(40, 224), (7, 64), (20, 96), (64, 128), (65, 96)])
def test_iq2_grouped_gate_up(T, I):
    """IQ2_XXS gate/up for T > 1 (the matrix-instruction path): with two experts and
    top-2 every expert gets all T tokens (one fewer for the expert that loses the
    out-of-range id). T = 7 and 20 (below 28 pairs per expert) run the one-tile
    kernel, T = 20 over two 16-token tiles; from 28 the wide kernel: T = 40 spans
    three 16-token tiles of one pass, T = 64 gives passes of exactly 64 and 63 tokens
    and T = 65 a second pass of one token;
    I = 224 leaves the last 64-row work-group half empty; one out-of-range id puts
    a pair in the invalid bucket, whose h must be zero."""
    say("iq2 grouped", T, I)
    spec = workloads.LayerSpec(512, I, 2, 2, mq.FMT_IQ2_XXS, mq.FMT_MXFP4, seed=4400 + T)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 2, 2)
    ids = ids.copy()
    ids[1, 0] = 99
    x = synth.activations_bf16(spec.seed + 1, T, 512)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(ids)
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, x_tensor(x), it, ws=ws).cpu().numpy().reshape(T, 2, I)
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    assert np.all(h[1, 0] == 0.0)
    ids2 = ids.copy()
    ids2[1, 0] = 0
    _, ref_h = moe.moe_layer(x, ids2, rw, oracle_weight_fn(spec))
    ok = np.ones((T, 2), bool)
    ok[1, 0] = False
    assert rel_err(h[ok], ref_h[ok]) < TOL


@pytest.mark.parametrize("T,H", [(40, 544), (9, 512)])
def test_q2k_grouped_down(T, H):
    """Q2_K down for T > 1 (the matrix-instruction path, taken from 8 pairs per
    expert): with two experts and top-2 every expert gets all T tokens, so T = 40
    spans three 16-token tiles (the last partial) and T = 9 one partial tile;
    H = 544 leaves the last 64-row work-group half empty; one out-of-range
    id puts a pair in the invalid bucket, which must add nothing to y. The down stage
    is fed the oracle's own h, so y is compared with the oracle's y directly."""
    say("q2k grouped down", T, H)
    spec = workloads.LayerSpec(H, 256, 2, 2, mq.FMT_MXFP4, mq.FMT_Q2_K, seed=4600 + T)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 2, 2)
    x = synth.activations_bf16(spec.seed + 1, T, H)
    rw0 = rw.copy()
    rw0[1, 0] = 0.0  # the pair whose id goes out of range contributes nothing
    ref_y, ref_h = moe.moe_layer(x, ids, rw0, oracle_weight_fn(spec))
    bad = ids.copy()
    bad[1, 0] = 99
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(bad)
    mq.route(layer, it, ws=ws)
    h = torch.from_numpy(np.ascontiguousarray(ref_h, dtype=np.float32)).cuda()
    y = mq.down(layer, h, it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    assert rel_err(y, ref_y) < TOL


@pytest.mark.parametrize("fmt", [mq.FMT_MXFP4, mq.FMT_NVFP4])
def test_fp4_gate_up_scale_alignment(fmt):
    """Single-token MXFP4 / NVFP4 gate/up reads its block scales 16 bytes at a time
    on the matrix-instruction path; scale planes only 4-byte aligned (the minimum the
    ABI asks for) take the GEMV path instead. Both must match the oracle."""
    say("fp4 scale alignment", fmt)
    spec = workloads.LayerSpec(1024, 512, 8, 3, fmt, mq.FMT_MXFP4, seed=4501)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(spec.seed, 1, 8, 3)
    x = synth.activations_bf16(spec.seed + 1, 1, 1024)
    ref, ref_h = moe.moe_layer(x, ids, rw, oracle_weight_fn(spec))
    y16 = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw)).cpu().numpy()
    for w in (layer.gate, layer.up):
        buf = torch.empty(w.scales.numel() + 4, dtype=torch.uint8, device="cuda")
        buf[4:].copy_(w.scales)
        w.scales = buf[4:]
        assert w.scales.data_ptr() % 16 == 4
    h4 = mq.gate_up(layer, x_tensor(x), cuda(ids)).cpu().numpy()
    y4 = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw)).cpu().numpy()
    assert rel_err(y16, ref) < TOL
    assert rel_err(y4, ref) < TOL
    assert rel_err(h4.reshape(1, 3, 512), ref_h) < TOL


def test_layer_repeats_exactly():
    """Every sum runs in a fixed order (no float atomics, the combine walks the
    slots in order), so fifty calls in a row on one workspace agree bit for bit."""
    say("layer repeats")
    spec = workloads.LayerSpec(2048, 1024, 32, 6, 1, 1, seed=5)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(6, 1, 32, 6)
    x = x_tensor(synth.activations_bf16(7, 1, 2048))
    ws = layer.workspace(1)
    mq.check_device_error(ws)
    ys = [mq.expert_forward(layer, x, cuda(ids), cuda(rw), ws=ws).clone() for _ in range(50)]
    assert mq.check_device_error(ws) == 0
    ref = ys[0].cpu().numpy()
    for y in ys[1:]:
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    oref, _ = moe.moe_layer(synth.activations_bf16(7, 1, 2048), ids, rw, oracle_weight_fn(spec))
    assert rel_err(ref, oref) < TOL


def test_forward_is_deterministic():
    say("determinism")
    spec = workloads.LayerSpec(1024, 512, 16, 6, 4, 3, seed=99)
    layer = upload_layer(spec)
    for T in (1, 16):
        ids, rw = synth.uniform_routing(3, T, 16, 6)
        x = x_tensor(synth.activations_bf16(4, T, 1024))
        a = mq.expert_forward(layer, x, cuda(ids), cuda(rw)).cpu().numpy()
        b = mq.expert_forward(layer, x, cuda(ids), cuda(rw)).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("T", [1, 5])
def test_out_of_range_expert_ids(T):
    say("bad ids", T)
    spec = workloads.LayerSpec(512, 256, 8, 3, 1, 1, seed=7)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(8, T, 8, 3)
    ids = ids.copy()
    ids[0, 1] = 300
    if T > 1:
        ids[T - 1, 0] = -2
    x = synth.activations_bf16(9, T, 512)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    # reference: skipped pairs contribute nothing
    rw2 = rw.copy()
    ids2 = ids.copy()
    bad = (ids < 0) | (ids >= 8)
    rw2[bad] = 0
    ids2[bad] = 0
    ref, _ = moe.moe_layer(x, ids2, rw2, oracle_weight_fn(spec))
    assert rel_err(y, ref) < TOL


def test_out_of_range_expert_ids_matrix_path():
    """bs=1 with MXFP4 gate/up and down both on the block-scaled matrix instruction
    (K a multiple of 512): an out-of-range id contributes nothing and sets the
    error bit."""
    say("bad ids, matrix path")
    spec = workloads.LayerSpec(1024, 512, 8, 3, 1, 1, seed=77)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(8, 1, 8, 3)
    ids = ids.copy()
    ids[0, 1] = 300
    x = synth.activations_bf16(9, 1, 1024)
    ws = layer.workspace(1)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    rw2 = rw.copy()
    ids2 = ids.copy()
    rw2[0, 1] = 0
    ids2[0, 1] = 0
    ref, _ = moe.moe_layer(x, ids2, rw2, oracle_weight_fn(spec))
    assert rel_err(y, ref) < TOL


def test_single_expert_workload():
    say("single_expert")
    wl = workloads.WORKLOADS["single_expert"]
    layer = workloads.build_layer(mq, wl.spec)
    ids, rw = workloads.routing(wl, 1)
    x = workloads.activations(wl, 1)
    ref, ref_h = moe.moe_layer(x, ids, rw, oracle_weight_fn(wl.spec))
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw)).cpu().numpy()
    assert rel_err(y, ref) < TOL


@pytest.mark.parametrize("name,T,sample", [("mxfp4_layer", 1, None), ("nvfp4_q2k", 1, None),
                                            ("nvfp4_q2k", 16, [0, 7, 15]), ("iq2_q2k_43", 1, None),
                                            ("iq2_q2k_43", 16, [0, 8, 15]),
                                            ("iq2_q2k_43", 64, [0, 31, 63])])
def test_full_size_layer(name, T, sample):
    """Full-size layer (device-filled), the launch configuration the benchmark
    times; tokens sampled at bs 16 and 64 and checked against the oracle."""
    say("full layer", name, T)
    wl = workloads.WORKLOADS[name]
    layer = workloads.build_layer(mq, wl.spec)
    ids, rw = workloads.routing(wl, T)
    x = workloads.activations(wl, T)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    toks = list(range(T)) if sample is None else sample
    ref, _ = moe.moe_layer(x[toks], ids[toks], rw[toks], oracle_weight_fn(wl.spec))
    assert rel_err(y[toks], ref) < TOL
    del layer
    torch.cuda.empty_cache()


def test_iq2_q2k_layers_0_21_42():
    """Three of the 43 layers (distinct weights per layer), bs 1."""
    wl = workloads.WORKLOADS["iq2_q2k_43"]
    for l in (21, 42):
        say("iq2 layer", l)
        spec = workloads.LayerSpec(**{**wl.spec.__dict__, "layer": l})
        layer = workloads.build_layer(mq, spec)
        ids, rw = workloads.routing(wl, 1, step=l)
        x = workloads.activations(wl, 1, layer=l)
        y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw)).cpu().numpy()
        ref, _ = moe.moe_layer(x, ids, rw, oracle_weight_fn(spec))
        assert rel_err(y, ref) < TOL
        del layer
        torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 16])
def test_fp8_linear_full_size(T):
    say("fp8 linear", T)
    wl = workloads.WORKLOADS["nvfp4_q2k"]
    rows, cols = wl.linear
    W = workloads.build_linear(mq, wl.spec.seed, rows, cols)
    x = synth.activations_bf16(wl.spec.seed + 77 + T, T, cols)
    y = mq.linear(W, 0, x_tensor(x)).cpu().numpy()
    planes = workloads.host_linear_planes(wl.spec.seed, rows, cols)
    Wd = formats.dequant(mq.FMT_FP8_B128, planes, rows, cols)
    ref = moe.linear(Wd, x)
    assert rel_err(y, ref) < TOL


@pytest.mark.parametrize("fmt,rows,cols", [(1, 1000, 1024), (3, 333, 768), (5, 384, 640), (4, 200, 512),
                                           (2, 97, 96)])
def test_linear_ragged(fmt, rows, cols):
    say("linear ragged", fmt, rows, cols)
    rng = np.random.default_rng(rows)
    if fmt == 5:
        planes = [synth.field_bytes(3, 1, synth.FIELD_E4M3_FINITE, 0, rows * cols),
                  synth.field_bytes(3, 2, synth.FIELD_E8M0_119_123, 0, (rows // 128) * (cols // 128))]
    else:
        planes = synth.expert_source(5, 0, 0, fmt, rows, cols, 0)
    grid = workloads.host_grid()
    W = upload_weight(fmt, rows, cols, [planes], [1.25], grid)
    for T in (1, 6):
        x = synth.activations_bf16(int(rng.integers(1 << 30)), T, cols)
        y = mq.linear(W, 0, x_tensor(x)).cpu().numpy()
        ref = moe.linear(formats.dequant(fmt, planes, rows, cols, scale2=1.25, grid=grid), x)
        assert rel_err(y, ref) < TOL, (fmt, T)


@pytest.mark.parametrize("rows,cols", [(128, 256), (384, 768), (256, 4608), (128, 8192)])
def test_fp8_linear_token_batches(rows, cols):
    """FP8 block-128 linear for T >= 2 (the matrix-instruction path): one K step,
    fewer steps than waves, more steps than waves (4608 = 18 steps of 256 over 16
    waves) and a long K; T spans a ragged single tile, several tiles and more than
    one pass of four tiles over the weights. Expert 1 of two, so the expert offsets
    are exercised; scale codes span 2^-27 .. 2^22."""
    say("fp8 linear batches", rows, cols)
    rng = np.random.default_rng(rows * 7 + cols)
    planes = []
    for e in range(2):
        codes = synth.field_bytes(11 + e, 1, synth.FIELD_E4M3_FINITE, 0, rows * cols)
        sc = rng.integers(100, 150, size=(rows // 128) * (cols // 128), dtype=np.uint8)
        planes.append([codes, sc])
    W = upload_weight(5, rows, cols, planes)
    Wd = formats.dequant(5, planes[1], rows, cols)
    for T in (2, 5, 16, 17, 64, 70):
        x = synth.activations_bf16(int(rng.integers(1 << 30)), T, cols)
        y = mq.linear(W, 1, x_tensor(x)).cpu().numpy()
        ref = moe.linear(Wd, x)
        assert rel_err(y, ref) < TOL, (rows, cols, T)
