"""Prefill (T >= 128) of layers that mix MXFP4 with IQ2_XXS or Q2_K projections
(DeepSeekv4 Flash for 1x Spark forum thread: an IQ2_XXS floor with MXFP4 promoted
on gate/up in early layers and on down in late ones; second post: one grouped
GEMM per projection). The MXFP4 projection runs the W4A8 grouped GEMM (MXFP8
activations), the other one the grouped decode kernels on exact activations.
Every stage is checked against the oracle on the GPU's own input to that stage,
so rounding-boundary flips in the MXFP8 quantisation of h cannot fail a test, and
the layer call must reproduce the stages bit for bit."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from oracle import moe, mxfp8
from tests.helpers import TOL, oracle_weight_fn, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_tensor(bits):
    return cuda(bits.view(np.int16)).view(torch.bfloat16)


def bits32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("H,I,E,T,sample", [(1024, 512, 16, 256, None), (4096, 2048, 256, 2048, [0, 1337])])
def test_iq2_gate_up_mxfp4_down_prefill(H, I, E, T, sample):
    say("prefill iq2 gate/up + mxfp4 down", H, I, E, T)
    spec = workloads.LayerSpec(H, I, E, 6, mq.FMT_IQ2_XXS, mq.FMT_MXFP4, seed=7100 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, 6)
    x = synth.activations_bf16(spec.seed + 1, T, H)
    xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y_fwd = mq.expert_forward(layer, xt, it, rt, ws=ws)
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, xt, it, ws=ws)                                # grouped IQ2_XXS, fp32
    hq, hs = mq.quantize_mxfp8(h.reshape(T * 6, I))
    y = mq.prefill_down(layer, hq, hs, it, rt, ws=ws)
    assert mq.check_device_error(ws) == 0
    h, hq, hs, y, y_fwd = (t.cpu().numpy() for t in (h, hq, hs, y, y_fwd))
    assert np.array_equal(bits32(y), bits32(y_fwd))                  # the layer call is these stages
    toks = list(range(T)) if sample is None else sample
    wfn = oracle_weight_fn(spec)
    _, ref_h = moe.moe_layer(x[toks], ids[toks], rw[toks], wfn)
    assert rel_err(h[toks], ref_h) < TOL
    rows = [t * 6 + k for t in toks for k in range(6)]
    oq, os_ = mxfp8.quantize(h.reshape(T * 6, I)[rows].astype(np.float64))
    assert np.array_equal(oq, hq[rows]) and np.array_equal(os_, hs[rows])
    ref_y = moe.prefill_y(hq[rows], hs[rows], ids[toks], rw[toks], wfn)
    err = rel_err(y[toks], ref_y)
    say("y err", err)
    assert err < TOL
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt_dn", [mq.FMT_Q2_K, mq.FMT_IQ2_XXS])
def test_mxfp4_gate_up_2bit_down_prefill(fmt_dn):
    say("prefill mxfp4 gate/up + 2-bit down", fmt_dn)
    H, I, E, T = 1024, 512, 16, 256
    spec = workloads.LayerSpec(H, I, E, 6, mq.FMT_MXFP4, fmt_dn, seed=7200 + fmt_dn)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, 6)
    x = synth.activations_bf16(spec.seed + 1, T, H)
    xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y_fwd = mq.expert_forward(layer, xt, it, rt, ws=ws)
    xq, xs = mq.quantize_mxfp8(xt)
    mq.route(layer, it, ws=ws)
    h = torch.empty((T * 6, I), dtype=torch.float32, device="cuda")
    mq.prefill_gate_up(layer, xq, xs, it, h_f32=h, ws=ws)                # W4A8
    y = mq.down(layer, h.reshape(T, 6, I), it, rt, ws=ws)              # grouped 2-bit down, exact h
    assert mq.check_device_error(ws) == 0
    h, xq, xs, y, y_fwd = (t.cpu().numpy() for t in (h, xq, xs, y, y_fwd))
    assert np.array_equal(bits32(y), bits32(y_fwd))
    wfn = oracle_weight_fn(spec)
    ref_h = moe.prefill_h(xq, xs, ids, wfn)
    assert rel_err(h.reshape(T, 6, I), ref_h) < TOL
    ref_y = np.zeros((T, H))
    for t in range(T):
        for k in range(6):
            ref_y[t] += float(rw[t, k]) * (wfn(moe.DOWN, int(ids[t, k])) @ h[t * 6 + k].astype(np.float64))
    err = rel_err(y, ref_y)
    say("y err", err)
    assert err < TOL


def test_mixed_prefill_stage_checks():
    """The W4A8 stage entry points take a mixed layer when their own projection is
    MXFP4 and refuse it (MOEQ_E_FMT) otherwise."""
    spec = workloads.LayerSpec(512, 256, 4, 2, mq.FMT_IQ2_XXS, mq.FMT_MXFP4, seed=7300)
    layer = workloads.build_layer(mq, spec)
    T = 4
    x = x_tensor(synth.activations_bf16(1, T, 512))
    ids, rw = synth.uniform_routing(2, T, 4, 2)
    xq, xs = mq.quantize_mxfp8(x)
    with pytest.raises(mq.MoeqError) as ei:
        mq.prefill_gate_up(layer, xq, xs, cuda(ids))
    assert ei.value.status == -2
    hq = torch.zeros((T * 2, 256), dtype=torch.uint8, device="cuda")
    hs = torch.full((T * 2, 8), 127, dtype=torch.uint8, device="cuda")
    mq.route(layer, cuda(ids))
    y = mq.prefill_down(layer, hq, hs, cuda(ids), cuda(rw)).cpu().numpy()
    assert not y.any()                                                   # all-zero h gives y = 0
