"""moeq_expert_forward_noalloc (the forward for callers that cannot allocate)
against moeq_expert_forward on the same inputs: two calls in a row on the shared
scratch, the second with fewer tokens, on the decode paths (single-token
matrix-unit kernels, grouped GEMVs) and the MXFP4 prefill path; a call that needs
more than the scratch is refused before any launch; out-of-range ids reach the
caller's error word."""
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


def bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("fmts,Ts", [((mq.FMT_MXFP4, mq.FMT_MXFP4), (16, 1)),
                                     ((mq.FMT_MXFP4, mq.FMT_MXFP4), (160, 3)),
                                     ((mq.FMT_NVFP4, mq.FMT_Q2_K), (64, 1))])
def test_noalloc_matches_workspace_forward(fmts, Ts):
    spec = workloads.LayerSpec(4096, 2048, 256, 6, fmts[0], fmts[1], seed=5600 + fmts[0] + Ts[0])
    layer = workloads.build_layer(mq, spec)
    wfn = oracle_weight_fn(spec)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for T in Ts:                                   # second call smaller than the first
        say("noalloc", fmts, T)
        ids, rw = synth.uniform_routing(spec.seed + T, T, 256, 6)
        x = synth.activations_bf16(spec.seed + 7 * T, T, 4096)
        xt, it, rt = x_tensor(x), cuda(ids), cuda(rw)
        y_na = torch.full((T, 4096), np.nan, dtype=torch.float32, device="cuda")
        mq.expert_forward_noalloc(layer, xt, it, rt, y=y_na, dev_err=err)
        y_ws = mq.expert_forward(layer, xt, it, rt)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y_na), bits(y_ws)), T
        assert int(err.item()) == 0
        if T <= 16:                                # decode path: against the oracle too
            toks = list(range(min(T, 3)))
            ref, _ = moe.moe_layer(x[toks], ids[toks], rw[toks], wfn)
            assert rel_err(y_na.cpu().numpy()[toks], ref) < TOL
    del layer
    torch.cuda.empty_cache()


def test_noalloc_limits_and_errors():
    spec = workloads.LayerSpec(1024, 512, 8, 6, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=5700)
    layer = workloads.build_layer(mq, spec)
    # out-of-range id: skipped, its bit set in the caller's word
    T = 5
    ids, rw = synth.uniform_routing(spec.seed, T, 8, 6)
    bad = ids.copy()
    bad[2, 3] = 8
    rw0 = rw.copy()
    rw0[2, 3] = 0.0
    x = synth.activations_bf16(spec.seed + 1, T, 1024)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("noalloc bad id")
    y = mq.expert_forward_noalloc(layer, x_tensor(x), cuda(bad), cuda(rw), dev_err=err).cpu().numpy()
    assert int(err.item()) & mq.DEVERR_EXPERT_ID
    ok_ids = ids.copy()
    ref, _ = moe.moe_layer(x, ok_ids, rw0, oracle_weight_fn(spec))
    assert rel_err(y, ref) < TOL
    # the same call without an error word, then a single token
    y2 = mq.expert_forward_noalloc(layer, x_tensor(x), cuda(bad), cuda(rw)).cpu().numpy()
    assert np.array_equal(y2.view(np.uint32), y.view(np.uint32))
    y1 = mq.expert_forward_noalloc(layer, x_tensor(x[:1]), cuda(ids[:1]), cuda(rw[:1])).cpu().numpy()
    ref1, _ = moe.moe_layer(x[:1], ids[:1], rw[:1], oracle_weight_fn(spec))
    assert rel_err(y1, ref1) < TOL
    # too many tokens for the scratch: refused before any launch, y untouched
    T = 4096
    need = mq.workspace_bytes(layer, T)
    assert need > mq.NOALLOC_SCRATCH_BYTES
    xs = x_tensor(synth.activations_bf16(3, T, 1024))
    ids_b, rw_b = synth.uniform_routing(9, T, 8, 6)
    y_big = torch.full((T, 1024), 7.0, dtype=torch.float32, device="cuda")
    say("noalloc too large")
    with pytest.raises(mq.MoeqError) as ei:
        mq.expert_forward_noalloc(layer, xs, cuda(ids_b), cuda(rw_b), y=y_big)
    assert ei.value.status == mq.MOEQ_E_SCRATCH
    assert bool(torch.all(y_big == 7.0))
