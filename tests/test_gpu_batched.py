"""Batched MXFP4 and NVFP4 decode (T > 1) on the block-scaled matrix instruction
against the CPU oracle. Up to 8 tokens (4 for the NVFP4 gate/up) the
single-token kernels run over every (token, slot) pair; beyond, the grouped
kernels take each routed expert's pairs in staged tiles of two (MXFP4 gate/up and
down, and the NVFP4 gate/up, one pair per instruction). Cases: experts
with several tiles of pairs, K of 1024 and 4096 (one and eight steps per wave),
out-of-range ids on both paths, and the full DeepSeek-V4-Flash-shaped layers at
16 and 64 tokens (co-scheduled decode sessions)."""
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


@pytest.mark.parametrize("T,E,K", [(2, 8, 6), (5, 8, 6), (40, 8, 6), (9, 3, 2), (17, 2, 1), (33, 2, 1), (8, 8, 6),
                                   (9, 8, 6), (32, 8, 6)])
def test_batched_mxfp4_tiles(T, E, K):
    """T = 40 over 8 experts gives about 30 pairs per expert: fifteen two-pair
    tiles each for gate/up and down; T = 33, one slot, two experts: an odd expert
    ends on a one-pair tile; T = 8 is the largest batch of the direct path and
    T = 9 the smallest of the grouped one."""
    say("batched mxfp4", T, E, K)
    spec = workloads.LayerSpec(1024, 512, E, K, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=6100 + T + E)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    ref_y, ref_h = moe.moe_layer(x, ids, rw, oracle_weight_fn(spec))
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
    y = mq.expert_forward(layer, xt, it, rt, ws=ws).cpu().numpy()
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, xt, it, ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    eh, ey = rel_err(h, ref_h), rel_err(y, ref_y)
    say("h err", eh, "y err", ey)
    assert eh < TOL and ey < TOL


@pytest.mark.parametrize("T", [8, 40])
def test_batched_mxfp4_out_of_range_id(T):
    """T = 8 runs the single-token kernels over every pair, T = 40 the grouped
    kernels (the out-of-range ids form a bucket of their own there)."""
    say("batched mxfp4 bad id", T)
    E, K = 8, 6
    spec = workloads.LayerSpec(1024, 512, E, K, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=6200)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    bad = ids.copy()
    bad[3, 2] = -1
    bad[7, 5] = E
    rw0 = rw.copy()
    rw0[3, 2] = rw0[7, 5] = 0.0
    ref_y, _ = moe.moe_layer(x := synth.activations_bf16(spec.seed + 1, T, 1024), ids, rw0, oracle_weight_fn(spec))
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(bad), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    assert rel_err(y, ref_y) < TOL


@pytest.mark.parametrize("T,sample", [(8, [0, 3, 7]), (16, [0, 5, 15]), (64, [0, 31, 63])])
def test_batched_mxfp4_full_layer(T, sample):
    """T = 8 on the single-token kernels over every pair, T = 16 and 64 on the grouped
    kernels."""
    say("batched mxfp4 full layer", T)
    wl = workloads.WORKLOADS["mxfp4_layer"]
    layer = workloads.build_layer(mq, wl.spec)
    ids, rw = synth.uniform_routing(wl.spec.seed + 900 + T, T, 256, 6)
    x = synth.activations_bf16(wl.spec.seed + 901 + T, T, 4096)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    ref, _ = moe.moe_layer(x[sample], ids[sample], rw[sample], oracle_weight_fn(wl.spec))
    err = rel_err(y[sample], ref)
    say("err", err)
    assert err < TOL
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,T,E,K", [(1024, 17, 8, 6), (1024, 40, 8, 6), (1024, 22, 2, 1), (4096, 24, 8, 6),
                                     (1024, 33, 64, 6), (1024, 20, 256, 6), (1024, 4, 8, 6), (1024, 5, 8, 6)])
def test_batched_nvfp4_gate_up_tiles(H, T, E, K):
    """NVFP4 gate/up on the grouped kernel (from 5 tokens): 12.75 and 30 pairs per
    expert (two-pair tiles, the last partial), two experts of 11 pairs, hidden 4096
    (eight K steps per wave), about 3.2 pairs per expert over 64 experts, 1.2 over
    256 experts (T = 20), and T = 5, the smallest grouped batch; T = 4 is the largest
    batch of the direct path."""
    say("batched nvfp4", H, T, E, K)
    spec = workloads.LayerSpec(H, 512, E, K, mq.FMT_NVFP4, mq.FMT_MXFP4, seed=6300 + T + E + H)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    x = synth.activations_bf16(spec.seed + 1, T, H)
    ref_y, ref_h = moe.moe_layer(x, ids, rw, oracle_weight_fn(spec))
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
    y = mq.expert_forward(layer, xt, it, rt, ws=ws).cpu().numpy()
    mq.route(layer, it, ws=ws)
    h = mq.gate_up(layer, xt, it, ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    eh, ey = rel_err(h, ref_h), rel_err(y, ref_y)
    say("h err", eh, "y err", ey)
    assert eh < TOL and ey < TOL


def test_batched_nvfp4_out_of_range_id():
    say("batched nvfp4 bad id")
    E, K, T = 8, 6, 40
    spec = workloads.LayerSpec(1024, 512, E, K, mq.FMT_NVFP4, mq.FMT_MXFP4, seed=6400)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    bad = ids.copy()
    bad[3, 2] = -1
    bad[7, 5] = E
    rw0 = rw.copy()
    rw0[3, 2] = rw0[7, 5] = 0.0
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    ref_y, _ = moe.moe_layer(x, ids, rw0, oracle_weight_fn(spec))
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(bad), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    assert rel_err(y, ref_y) < TOL


@pytest.mark.parametrize("T,sample", [(16, [0, 5, 15]), (64, [0, 31, 63])])
def test_batched_nvfp4_q2k_full_layer(T, sample):
    """The NVFP4 + Q2_K layer of the DeepSeek-V4-Flash shape at 64 co-scheduled
    tokens: grouped NVFP4 gate/up and grouped Q2_K down."""
    say("batched nvfp4 + q2k full layer", T)
    wl = workloads.WORKLOADS["nvfp4_q2k"]
    layer = workloads.build_layer(mq, wl.spec)
    ids, rw = synth.uniform_routing(wl.spec.seed + 900 + T, T, 256, 6)
    x = synth.activations_bf16(wl.spec.seed + 901 + T, T, 4096)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    y = mq.expert_forward(layer, x_tensor(x), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    ref, _ = moe.moe_layer(x[sample], ids[sample], rw[sample], oracle_weight_fn(wl.spec))
    err = rel_err(y[sample], ref)
    say("err", err)
    assert err < TOL
    del layer
    torch.cuda.empty_cache()
