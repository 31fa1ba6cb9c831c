"""Q2_K down on the block-scaled FP8 matrix instruction (2-bit codes as E4M3
subnormals, h as four integer digits per 16-value sub-block) against the CPU oracle:
the single-token layer and the direct path of a few tokens (one grid row per token),
fed an fp32 h with full 24-bit mantissas and compared against a bound much tighter
than the projection tolerance (the digits keep 17 bits of h relative to each
sub-block's maximum, and every product is exact). Shapes cover one, three and eight superblocks along K (waves with no
superblock, and with fewer than the others), 544 output rows (a partial last
16-row tile), out-of-range ids, h with one outlier per 32-block, and top-8, which
the kernel does not take (the GEMV runs instead)."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from oracle import moe
from tests.helpers import TOL, oracle_weight_fn, rel_err

pytestmark = pytest.mark.gpu

TIGHT = 1e-4


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def oracle_down(wfn, h, ids, rw, toks, n_experts):
    K = ids.shape[1]
    out = []
    for t in toks:
        y = 0.0
        for k in range(K):
            e = int(ids[t, k])
            if 0 <= e < n_experts:
                y = y + float(rw[t, k]) * (wfn(moe.DOWN, e) @ h[t, k].astype(np.float64))
        out.append(y)
    return np.array(out)


def silu_like_h(seed, T, K, I):
    rng = np.random.default_rng(seed)
    g, u = rng.standard_normal((2, T, K, I)) * 2.0
    return (moe.silu(g) * u).astype(np.float32)


@pytest.mark.parametrize("H,I,E,K,T", [
    (1024, 256, 8, 2, 1),      # one superblock: the second wave of each slot has none
    (544, 768, 8, 6, 1),       # three superblocks (2 + 1 per slot's waves), partial row tile
    (4096, 2048, 256, 6, 1),   # the DeepSeek-V4-Flash down
    (1024, 2048, 256, 6, 6),   # direct path, 1.06 pairs per touched expert
    (4096, 2048, 256, 6, 8),
    (512, 512, 16, 8, 1),      # top-8: the GEMV path
])
def test_q2k_down_matches_oracle(H, I, E, K, T):
    say("q2k down", H, I, E, K, T)
    spec = workloads.LayerSpec(H, I, E, K, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8100 + I + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    wfn = oracle_weight_fn(spec)
    h = silu_like_h(spec.seed, T, K, I)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(ids)
    if T > 1:
        mq.route(layer, it, ws=ws)
    y = mq.down(layer, cuda(h), it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) == 0
    toks = list(range(T)) if T <= 8 else [0, 7, 15]
    ref = oracle_down(wfn, h, ids, rw, toks, E)
    err = rel_err(y[toks], ref)
    say("err", err)
    assert err < TIGHT
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 3])
def test_q2k_down_out_of_range_ids(T):
    """An out-of-range id adds nothing and sets the error bit; the other slots of the
    same token are unaffected."""
    say("q2k down bad id", T)
    spec = workloads.LayerSpec(1024, 512, 64, 6, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8200 + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, 64, 6)
    bad = ids.copy()
    bad[0, 2] = -1
    bad[T - 1, 5] = 64
    h = silu_like_h(spec.seed, T, 6, 512)
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(bad)
    if T > 1:
        mq.route(layer, it, ws=ws)
    y = mq.down(layer, cuda(h), it, cuda(rw), ws=ws).cpu().numpy()
    assert mq.check_device_error(ws) & mq.DEVERR_EXPERT_ID
    ref = oracle_down(oracle_weight_fn(spec), h, bad, rw, list(range(T)), 64)
    assert rel_err(y, ref) < TIGHT


def test_q2k_down_h_outliers():
    """h with one value per 32-block 2^8 .. 2^20 times the others: the small values
    of such a block lose bits below the fourth term's range, far below the outlier's
    own contribution."""
    from tests.test_gpu_edges import OUTLIER_FACTORS, with_outliers
    say("q2k down outliers")
    spec = workloads.LayerSpec(1024, 1024, 8, 6, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8300)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, 1, 8, 6)
    rng = np.random.default_rng(spec.seed)
    h = with_outliers(silu_like_h(spec.seed, 1, 6, 1024).reshape(6, 1024), OUTLIER_FACTORS, rng)
    h = h.astype(np.float32).reshape(1, 6, 1024)
    ws = layer.workspace(1)
    y = mq.down(layer, cuda(h), cuda(ids), cuda(rw), ws=ws).cpu().numpy()
    ref = oracle_down(oracle_weight_fn(spec), h, ids, rw, [0], 8)
    err = rel_err(y, ref)
    say("err", err)
    assert err < TOL
