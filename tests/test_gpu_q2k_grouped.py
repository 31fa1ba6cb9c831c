"""Token-grouped Q2_K down (T > 1) on the block-scaled FP8 matrix instruction against
the CPU oracle: each expert's weights read once for all of its pairs, h as four
digits per 32-value block made once per pair. The layer shapes are chosen so the
grouped path runs; they cover experts of one pass of four pairs and of many passes
over the same weight registers (up to nine), one, three and eight superblocks along
K, a partial last 64-row tile, out-of-range ids, h with one outlier per
32-block, and the full DeepSeek-V4-Flash down at T = 256 (sampled tokens). The bound
is much tighter than the projection tolerance: four digits keep 19 bits of h
relative to each block's maximum and every product is exact."""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from tests.helpers import TOL, oracle_weight_fn, rel_err
from tests.test_gpu_q2k_mfma import TIGHT, cuda, oracle_down, silu_like_h

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def run_down(layer, h, ids, rw, T):
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    it = cuda(ids)
    mq.route(layer, it, ws=ws)
    y = mq.down(layer, cuda(h), it, cuda(rw), ws=ws).cpu().numpy()
    return y, mq.check_device_error(ws)


def bucket_sizes(ids, E):
    return np.bincount(ids[(ids >= 0) & (ids < E)].ravel(), minlength=E)


@pytest.mark.parametrize("H,I,E,K,T", [
    (1024, 256, 16, 2, 24),    # one superblock; about 3 pairs per expert: one group per pass
    (544, 768, 16, 2, 40),     # three superblocks, partial 64-row tile, up to 9+ pairs (passes)
    (1024, 2048, 8, 6, 8),     # eight superblocks, 6 pairs per expert: two groups per pass
    (512, 512, 8, 6, 48),      # 36 pairs per expert: nine passes
    (512, 256, 2, 1, 40),      # one superblock, 20 pairs per expert: five passes
    (1024, 2048, 4, 4, 20),    # eight superblocks, 20 pairs per expert
])
def test_q2k_grouped_down_matches_oracle(H, I, E, K, T):
    say("q2k grouped down", H, I, E, K, T)
    spec = workloads.LayerSpec(H, I, E, K, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8400 + I + T)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    say("pairs per expert", bucket_sizes(ids, E).tolist())
    wfn = oracle_weight_fn(spec)
    h = silu_like_h(spec.seed, T, K, I)
    y, err = run_down(layer, h, ids, rw, T)
    assert err == 0
    toks = list(range(T)) if T <= 24 else list(range(0, T, 3))
    ref = oracle_down(wfn, h, ids, rw, toks, E)
    e = rel_err(y[toks], ref)
    say("err", e)
    assert e < TIGHT
    del layer
    torch.cuda.empty_cache()


def test_q2k_grouped_down_full_size():
    """The DeepSeek-V4-Flash down (hidden 4096, intermediate 2048, 256 experts, top-6)
    at T = 256: about six pairs per touched expert, sampled tokens."""
    say("q2k grouped down full size")
    spec = workloads.LayerSpec(4096, 2048, 256, 6, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8500)
    layer = workloads.build_layer(mq, spec)
    T = 256
    ids, rw = synth.uniform_routing(spec.seed, T, 256, 6)
    h = silu_like_h(spec.seed, T, 6, 2048)
    y, err = run_down(layer, h, ids, rw, T)
    assert err == 0
    toks = [0, 77, 255]
    ref = oracle_down(oracle_weight_fn(spec), h, ids, rw, toks, 256)
    e = rel_err(y[toks], ref)
    say("err", e)
    assert e < TIGHT
    del layer
    torch.cuda.empty_cache()


def test_q2k_grouped_down_out_of_range_ids():
    """Out-of-range ids go to their own bucket: those pairs add nothing, the error bit
    is set, and every other pair of the same tokens is unaffected."""
    say("q2k grouped down bad ids")
    E, K, T = 8, 6, 10
    spec = workloads.LayerSpec(1024, 512, E, K, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8600)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    bad = ids.copy()
    bad[0, 2] = -1
    bad[4, 0] = E
    bad[9, 5] = 1000
    h = silu_like_h(spec.seed, T, K, 512)
    y, err = run_down(layer, h, bad, rw, T)
    assert err & mq.DEVERR_EXPERT_ID
    ref = oracle_down(oracle_weight_fn(spec), h, bad, rw, list(range(T)), E)
    assert rel_err(y, ref) < TIGHT


def test_q2k_grouped_down_h_outliers():
    """h with one value per 32-block 2^8 .. 2^20 times the others: the block's small
    values lose the bits below the fourth digit, far below the outlier's own share."""
    from tests.test_gpu_edges import OUTLIER_FACTORS, with_outliers
    say("q2k grouped down outliers")
    E, K, T = 8, 6, 8
    spec = workloads.LayerSpec(1024, 1024, E, K, mq.FMT_NVFP4, mq.FMT_Q2_K, seed=8700)
    layer = workloads.build_layer(mq, spec)
    ids, rw = synth.uniform_routing(spec.seed, T, E, K)
    rng = np.random.default_rng(spec.seed)
    h = silu_like_h(spec.seed, T, K, 1024).reshape(T * K, 1024)
    h = with_outliers(h, OUTLIER_FACTORS, rng).astype(np.float32).reshape(T, K, 1024)
    y, err = run_down(layer, h, ids, rw, T)
    assert err == 0
    ref = oracle_down(oracle_weight_fn(spec), h, ids, rw, list(range(T)), E)
    e = rel_err(y, ref)
    say("err", e)
    assert e < TOL
