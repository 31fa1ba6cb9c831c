"""GPU parity at the edges of the decode kernels' numerics and tiling:

* the token-grouped 2-bit kernels at full depth (16 IQ2_XXS superblocks along the
  gate/up contraction, 8 Q2_K superblocks along the down contraction), with enough
  pairs per expert for the wide IQ2_XXS kernel and several token tiles per pass;
* single-token MXFP4 / NVFP4 gate/up and MXFP4 down, whose activations enter the
  block-scaled matrix instruction as E4M3 terms with one e8m0 scale per 32, fed
  blocks that each hold one outlier 2^8 .. 2^20 times the other values;
* the Q2_K down fed an fp32 h with full 24-bit mantissas, at one and sixteen
  tokens, against a bound much tighter than the projection tolerance;
* full forwards of a layer with IQ2_XXS gate/up and MXFP4 down (mixed formats) at
  decode sizes.

Every expected value comes from the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from oracle import moe
from tests.helpers import TOL, oracle_weight_fn, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_tensor(bits):
    return cuda(bits.view(np.int16)).view(torch.bfloat16)


def with_outliers(v, factors, rng):
    """One element of every 32-block of each row scaled by the block's factor
    (cycled over the blocks), sign kept: a block max 2^k times its other values."""
    v = np.array(v, dtype=np.float64, copy=True)
    rows, K = v.shape
    for r in range(rows):
        for b in range(K // 32):
            j = 32 * b + int(rng.integers(32))
            f = factors[b % len(factors)]
            v[r, j] = np.sign(v[r, j] or 1.0) * max(abs(v[r, j]), 0.5) * f
    return v


# factors 2^12 and 2^13 sit on either side of the range in which the two-term
# split of a bf16 value is exact; 2^20 is far past it
OUTLIER_FACTORS = [2.0 ** 8, 2.0 ** 12, 2.0 ** 13, 2.0 ** 16, 2.0 ** 20, 1.0]


@pytest.mark.parametrize("fmt", [mq.FMT_MXFP4, mq.FMT_NVFP4])
def test_single_token_activation_outliers(fmt):
    """bs=1 gate/up (x as two E4M3 terms) and MXFP4 down (h as three terms), with
    one outlier per 32-block: compared element by element with the oracle."""
    say("outliers", fmt)
    spec = workloads.LayerSpec(1024, 512, 8, 6, fmt, mq.FMT_MXFP4, seed=5100 + fmt)
    layer = workloads.build_layer(mq, spec)
    rng = np.random.default_rng(spec.seed)
    ids, rw = synth.uniform_routing(spec.seed, 1, 8, 6)
    x = synth.activations_bf16(spec.seed + 1, 1, 1024)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xo = synth.bf16_bits_from_f32(with_outliers(xf, OUTLIER_FACTORS, rng).astype(np.float32))
    wfn = oracle_weight_fn(spec)
    ws = layer.workspace(1)
    for label, xb in (("plain", x), ("outliers", xo)):
        ref_y, ref_h = moe.moe_layer(xb, ids, rw, wfn)
        h = mq.gate_up(layer, x_tensor(xb), cuda(ids), ws=ws).cpu().numpy()
        y = mq.expert_forward(layer, x_tensor(xb), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
        eh, ey = rel_err(h, ref_h), rel_err(y, ref_y)
        say(label, "h err", eh, "y err", ey)
        assert eh < TOL and ey < TOL, (label, eh, ey)
    # the down stage alone, on an h with one outlier per 32-block of every slot
    _, ref_h = moe.moe_layer(x, ids, rw, wfn)
    ho = with_outliers(ref_h.reshape(6, 512), OUTLIER_FACTORS, rng).astype(np.float32)
    ref = np.zeros((1, 1024))
    for k in range(6):
        ref[0] += float(rw[0, k]) * (wfn(moe.DOWN, int(ids[0, k])) @ ho[k].astype(np.float64))
    y = mq.down(layer, cuda(ho.reshape(1, 6, 512)), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    err = rel_err(y, ref)
    say("down outliers err", err)
    assert err < TOL
    assert mq.check_device_error(ws) == 0


@pytest.mark.parametrize("T", [1, 16])
def test_q2k_down_on_oracle_h_is_tight(T):
    """Q2_K down (the block-scaled kernel, one grid row per token at T=16) fed an
    fp32 h of silu(g) * u values: four E4M3 terms keep about 16 significant bits
    of h, and the min term takes the exact sub-block sums of h, so the error stays
    far below the projection tolerance."""
    say("q2k down tight", T)
    spec = workloads.LayerSpec(4096, 2048, 256, 6, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=5200 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 256, 6)
    wfn = oracle_weight_fn(spec)
    toks = list(range(T)) if T == 1 else [0, 9, 15]
    # h shaped like silu(g) * u (fp32 with full 24-bit mantissas)
    rng = np.random.default_rng(spec.seed)
    g, u = rng.standard_normal((2, T, 6, 2048)) * 2.0
    h = (moe.silu(g) * u).astype(np.float32)
    ref_y = np.zeros((len(toks), 4096))
    for i, t in enumerate(toks):
        for k in range(6):
            ref_y[i] += float(rw[t, k]) * (wfn(moe.DOWN, int(ids[t, k])) @ h[t, k].astype(np.float64))
    ws = layer.workspace(T)
    it = cuda(ids)
    if T > 1:
        mq.route(layer, it, ws=ws)
    y = mq.down(layer, cuda(h), it, cuda(rw), ws=ws).cpu().numpy()
    err = rel_err(y[toks], ref_y)
    say("err", err)
    assert err < 1e-4
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt_dn", [mq.FMT_Q2_K, mq.FMT_IQ2_XXS])
def test_grouped_2bit_kernels_full_depth(fmt_dn):
    """IQ2_XXS gate/up + Q2_K or IQ2_XXS down at hidden 4096 / intermediate 2048
    with 4 experts and top-3: about 75 pairs per expert, so the wide IQ2_XXS kernel
    decodes each of the 16 superblocks along K once for a 64-token pass and a short
    second pass, and the grouped down runs 8 superblocks along K over five 16-token
    tiles."""
    say("grouped 2-bit full depth", fmt_dn)
    T = 100
    spec = workloads.LayerSpec(4096, 2048, 4, 3, mq.FMT_IQ2_XXS, fmt_dn, seed=5300 + fmt_dn)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 4, 3)
    loads = np.bincount(ids.reshape(-1), minlength=4)
    assert loads.min() >= 64, loads
    x = synth.activations_bf16(spec.seed + 1, T, 4096)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(ids)
    y = mq.expert_forward(layer, x_tensor(x), it, cuda(rw), ws=ws).cpu().numpy()
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, x_tensor(x), it, ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    toks = [0, 1, 50, 63, 64, 99]
    ref_y, ref_h = moe.moe_layer(x[toks], ids[toks], rw[toks], oracle_weight_fn(spec))
    eh, ey = rel_err(h[toks], ref_h), rel_err(y[toks], ref_y)
    say("h err", eh, "y err", ey)
    assert eh < TOL and ey < TOL
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,sample", [(16, None), (96, [0, 50, 95])])
def test_mixed_iq2_gate_up_mxfp4_down_forward(T, sample):
    """A layer whose gate/up is IQ2_XXS and whose down is MXFP4, end to end through
    moeq_expert_forward at decode sizes (routing, grouped IQ2_XXS gate/up, MXFP4
    down, combine) against the exact layer. From 128 tokens the MXFP4 down takes
    the W4A8 prefill GEMM instead (MXFP8 h), checked stage by stage in
    test_gpu_prefill_mixed.py."""
    say("mixed iq2/mxfp4", T)
    spec = workloads.LayerSpec(1024, 512, 32, 6, mq.FMT_IQ2_XXS, mq.FMT_MXFP4, seed=5400 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 32, 6)
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    toks = list(range(T)) if sample is None else sample
    ref, _ = moe.moe_layer(x[toks], ids[toks], rw[toks], oracle_weight_fn(spec))
    err = rel_err(y[toks], ref)
    say("err", err)
    assert err < TOL


@pytest.mark.parametrize("T,E,K", [(48, 64, 6), (40, 2, 2), (130, 2, 2)])
def test_iq2_grouped_down_tiles(T, E, K):
    """The token-grouped IQ2_XXS down fed the oracle's own h: T = 48 over 64 experts
    (4.5 pairs per touched expert: one partial 16-token tile each), T = 40 and 130
    over two experts with top-2 (three and nine tiles per expert, the last partial).
    One out-of-range id must add nothing."""
    say("iq2 grouped down", T, E, K)
    spec = workloads.LayerSpec(1024, 512, E, K, mq.FMT_MXFP4, mq.FMT_IQ2_XXS, seed=5500 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    rw0 = rw.copy()
    rw0[1, 0] = 0.0  # the pair whose id goes out of range contributes nothing
    wfn = oracle_weight_fn(spec)
    toks = list(range(T)) if T <= 48 else [0, 1, 47, 48, 96, 129]
    ref_y, ref_h = moe.moe_layer(x[toks], ids[toks], rw0[toks], wfn)
    _, h_all = moe.moe_layer(x, ids, rw, wfn)
    bad = ids.copy()
    bad[1, 0] = 999
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(bad)
    mq.route(layer, it, ws=ws)
    h = torch.from_numpy(np.ascontiguousarray(h_all, dtype=np.float32)).cuda()
    y = mq.down(layer, h, it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    err = rel_err(y[toks], ref_y)
    say("err", err)
    assert err < TOL
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,T", [(256, 2), (256, 3), (64, 8)])
def test_iq2_direct_few_tokens(E, T):
    """IQ2_XXS gate/up + Q2_K down for a few tokens. Over 256 experts at T = 2 and 3
    (1.01 and 1.02 pairs per touched expert) both projections run over every
    (token, slot) pair without routing; over 64 experts at T = 8 (1.36 pairs) the
    gate/up is token-grouped and the Q2_K down grouped on the FP8 instruction. One
    out-of-range id must give zero h and add nothing."""
    say("iq2 few tokens", E, T)
    spec = workloads.LayerSpec(1024, 512, E, 6, mq.FMT_IQ2_XXS, mq.FMT_Q2_K, seed=5600 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, 6)
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    bad = ids.copy()
    bad[T - 1, 4] = -3
    rw0 = rw.copy()
    rw0[T - 1, 4] = 0.0
    wfn = oracle_weight_fn(spec)
    ref_y, ref_h = moe.moe_layer(x, ids, rw0, wfn)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    xt, it = x_tensor(x), cuda(bad)
    y = mq.expert_forward(layer, xt, it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, xt, it, ws=ws).cpu().numpy().reshape(T, 6, 512)
    assert np.all(h[T - 1, 4] == 0.0)
    ok = np.ones((T, 6), bool)
    ok[T - 1, 4] = False
    eh, ey = rel_err(h[ok], ref_h[ok]), rel_err(y, ref_y)
    say("h err", eh, "y err", ey)
    assert eh < TOL and ey < TOL


@pytest.mark.parametrize("fmt_dn,T", [(mq.FMT_Q2_K, 1), (mq.FMT_Q2_K, 8), (mq.FMT_MXFP4, 8)])
def test_down_rejects_unaligned_h(fmt_dn, T):
    """h 4 bytes past a 16-byte boundary is refused before any launch (the down
    kernels read h 16 bytes at a time; the C ABI documents 16-byte alignment)."""
    say("down unaligned h", fmt_dn, T)
    spec = workloads.LayerSpec(1024, 512, 8, 6, mq.FMT_NVFP4, fmt_dn, seed=5900 + T + fmt_dn)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 8, 6)
    buf = torch.zeros(T * 6 * 512 + 4, dtype=torch.float32, device="cuda")
    ht = buf[1:1 + T * 6 * 512].view(T, 6, 512)
    assert ht.data_ptr() % 16 == 4
    ws = layer.workspace(T)
    it = cuda(ids)
    if T > 1:
        mq.route(layer, it, ws=ws)
    with pytest.raises(mq.MoeqError):
        mq.down(layer, ht, it, cuda(rw), ws=ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,E", [(1, 64), (3, 64), (8, 8)])
def test_q2k_down_intermediate_beyond_2048(T, E):
    """A Q2_K down with intermediate 2560 (ten superblocks, past the FP8 kernels'
    2048): the dequantize + GEMV at one token, GEMV partials at three tokens over 64
    experts, and the bf16 matrix-instruction grouped down at six pairs per expert."""
    say("q2k down I=2560", T, E)
    K, I = 6, 2560
    spec = workloads.LayerSpec(512, I, E, K, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=5950 + T + E)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    rng = np.random.default_rng(spec.seed)
    h = (moe.silu(rng.standard_normal((T, K, I)) * 2.0) * rng.standard_normal((T, K, I)) * 2.0).astype(np.float32)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(ids)
    if T > 1:
        mq.route(layer, it, ws=ws)
    y = mq.down(layer, cuda(h), it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    wfn = oracle_weight_fn(spec)
    ref = np.array([sum(float(rw[t, k]) * (wfn(moe.DOWN, int(ids[t, k])) @ h[t, k].astype(np.float64))
                        for k in range(K)) for t in range(T)])
    e = rel_err(y, ref)
    say("err", e)
    assert e < TOL
