"""GPU parity of the W4A8 prefill path (MXFP4 weights x MXFP8 activations on the
block-scaled matrix instruction), stage by stage, each given identical inputs:

1. MXFP8 quantisation of x: bit-exact against the oracle;
2. h (fp32, before quantisation) within 2e-3 of the oracle fed the same Xq;
3. MXFP8 quantisation of the GPU's h: bit-exact against the oracle quantising it;
4. y within 2e-3 of the oracle fed the GPU's Hq;
5. reported only: y against the unquantised float64 chain (the cost of W4A8).
"""
import sys

import numpy as np
import pytest

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from oracle import moe, mxfp8
from tests.helpers import TOL, oracle_weight_fn, rel_err
from tests.test_gpu_parity import cuda, upload_layer, x_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def run_stages(layer, x_bits, ids, rw):
    T = x_bits.shape[0]
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    xt = x_tensor(x_bits)
    it = cuda(ids)
    xq, xs = mq.quantize_mxfp8(xt)
    mq.route(layer, it, ws=ws)
    P = T * layer.top_k
    h = torch.empty((P, layer.inter), dtype=torch.float32, device="cuda")
    hq, hs = mq.prefill_gate_up(layer, xq, xs, it, h_f32=h, ws=ws)
    y = mq.prefill_down(layer, hq, hs, it, cuda(rw), ws=ws)
    y_fwd = mq.expert_forward(layer, xt, it, cuda(rw), ws=ws)
    err = mq.check_device_error(ws, clear=True)
    return dict(xq=xq.cpu().numpy(), xs=xs.cpu().numpy(), h=h.cpu().numpy(), hq=hq.cpu().numpy(),
                hs=hs.cpu().numpy(), y=y.cpu().numpy(), y_fwd=y_fwd.cpu().numpy(), err=err)


def pair_h(weight, xq, xs, t, e):
    xh = mxfp8.dequantize(xq[t:t + 1], xs[t:t + 1])[0]
    return moe.swiglu(weight(0, e) @ xh, weight(1, e) @ xh)


@pytest.mark.parametrize("case", [
    # (H, I, E, K, T, seed)
    (512, 256, 8, 3, 40, 1),       # several experts with 1..30 tokens
    (1024, 512, 4, 2, 150, 2),     # > 64 tokens per expert: several passes of token tiles
    (512, 768, 16, 6, 129, 3),     # T >= 128: expert_forward takes the prefill path; 3 row groups
    (1280, 512, 8, 2, 200, 4),     # K = 1280: five 256-chunks, a partial second group of staged scales
])
def test_prefill_stages_small(case):
    H, I, E, K, T, seed = case
    say("prefill small", case)
    spec = workloads.LayerSpec(H, I, E, K, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=4000 + seed)
    layer = upload_layer(spec)
    ids, rw = synth.uniform_routing(seed, T, E, K)
    x = synth.activations_bf16(seed + 11, T, H)
    out = run_stages(layer, x, ids, rw)
    assert out["err"] == 0
    weight = oracle_weight_fn(spec)
    # 1. MXFP8 of x
    rq, rs = mxfp8.quantize((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    assert np.array_equal(out["xq"], rq) and np.array_equal(out["xs"], rs)
    # 2. h against the oracle on the same Xq
    ref_h = moe.prefill_h(out["xq"], out["xs"], ids, weight).reshape(T * K, I)
    assert rel_err(out["h"], ref_h) < TOL
    # 3. MXFP8 of the GPU's h
    q2, s2 = mxfp8.quantize(out["h"].astype(np.float64))
    assert np.array_equal(out["hs"], s2)
    assert np.array_equal(out["hq"], q2)
    # 4. y against the oracle fed the GPU's Hq
    ref_y = moe.prefill_y(out["hq"], out["hs"], ids, rw, weight)
    assert rel_err(out["y"], ref_y) < TOL
    if T >= 128:
        assert np.array_equal(out["y_fwd"], out["y"])
    # 5. reported: W4A8 against the unquantised chain
    full, _ = moe.moe_layer(x, ids, rw, weight)
    say(f"W4A8 vs bf16/fp64 chain: rel err {rel_err(out['y'], full):.3e}")


def test_prefill_out_of_range_ids():
    say("prefill bad ids")
    spec = workloads.LayerSpec(512, 256, 8, 2, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=4100)
    layer = upload_layer(spec)
    T = 130
    ids, rw = synth.uniform_routing(5, T, 8, 2)
    ids = ids.copy()
    ids[3, 0] = 99
    ids[77, 1] = -1
    x = synth.activations_bf16(6, T, 512)
    out = run_stages(layer, x, ids, rw)
    assert out["err"] & mq.DEVERR_EXPERT_ID
    bad = (ids < 0) | (ids >= 8)
    ids2, rw2 = ids.copy(), rw.copy()
    ids2[bad], rw2[bad] = 0, 0
    weight = oracle_weight_fn(spec)
    hq = out["hq"].reshape(T, 2, -1)
    assert np.all(hq[3, 0] == 0) and np.all(hq[77, 1] == 0)
    ref_y = moe.prefill_y(out["hq"], out["hs"], ids2, rw2, weight)
    assert rel_err(out["y"], ref_y) < TOL


def test_prefill_full_size_sampled():
    """2048 prompt tokens routed by a hash of the token id over 256 MXFP4 experts
    (the launch configuration of the prefill workload); sampled pairs and tokens
    checked against the oracle."""
    say("prefill full size")
    wl = workloads.WORKLOADS["prefill_mxfp4"]
    spec = wl.spec
    T = 2048
    layer = workloads.build_layer(mq, spec)
    ids, rw = workloads.routing(wl, T)
    x = workloads.activations(wl, T)
    out = run_stages(layer, x, ids, rw)
    assert out["err"] == 0
    weight = oracle_weight_fn(spec)
    loads = np.bincount(ids.reshape(-1), minlength=256)
    say(f"expert loads: min {loads.min()} mean {loads.mean():.1f} max {loads.max()}")
    rq, rs = mxfp8.quantize((x[:64].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    assert np.array_equal(out["xq"][:64], rq) and np.array_equal(out["xs"][:64], rs)
    busiest = int(np.argmax(loads))
    toks = [0, 1, 1000, 2047] + [int(t) for t in np.nonzero((ids == busiest).any(1))[0][-2:]]
    K = spec.top_k
    for t in toks:
        for k in range(K):
            p = t * K + k
            ref = pair_h(weight, out["xq"], out["xs"], t, int(ids[t, k]))
            assert rel_err(out["h"][p], ref) < TOL, (t, k)
            q2, s2 = mxfp8.quantize(out["h"][p:p + 1].astype(np.float64))
            assert np.array_equal(out["hq"][p:p + 1], q2) and np.array_equal(out["hs"][p:p + 1], s2)
    ref_y = moe.prefill_y(out["hq"].reshape(T, K, -1)[toks].reshape(len(toks) * K, -1),
                          out["hs"].reshape(T, K, -1)[toks].reshape(len(toks) * K, -1),
                          ids[toks], rw[toks], weight)
    assert rel_err(out["y"][toks], ref_y) < TOL
    assert np.array_equal(out["y_fwd"], out["y"])
    del layer
    torch.cuda.empty_cache()


def test_prefill_item_boundaries():
    """Expert loads chosen at the work-item edges: 1, 32 (one token tile), 33 (a
    second tile), 64 (one full item), 65 (a second item of one pair) and 128 (two
    full items); the other pairs go to the remaining experts."""
    say("prefill item boundaries")
    H, I, E, K, T = 512, 256, 8, 2, 200
    spec = workloads.LayerSpec(H, I, E, K, mq.FMT_MXFP4, mq.FMT_MXFP4, seed=4200)
    layer = upload_layer(spec)
    loads = [1, 32, 33, 64, 65, 128]
    flat = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(loads)])
    rest = T * K - flat.size
    flat = np.concatenate([flat, 6 + (np.arange(rest) % 2).astype(np.int32)])
    rng = np.random.default_rng(4201)
    ids = rng.permutation(flat).reshape(T, K).astype(np.int32)   # duplicates within a token allowed
    _, rw = synth.uniform_routing(4202, T, E, K)
    x = synth.activations_bf16(4203, T, H)
    assert list(np.bincount(ids.reshape(-1), minlength=E)[:6]) == loads
    out = run_stages(layer, x, ids, rw)
    assert out["err"] == 0
    weight = oracle_weight_fn(spec)
    ref_h = moe.prefill_h(out["xq"], out["xs"], ids, weight).reshape(T * K, I)
    assert rel_err(out["h"], ref_h) < TOL
    q2, s2 = mxfp8.quantize(out["h"].astype(np.float64))
    assert np.array_equal(out["hq"], q2) and np.array_equal(out["hs"], s2)
    ref_y = moe.prefill_y(out["hq"], out["hs"], ids, rw, weight)
    assert rel_err(out["y"], ref_y) < TOL
    assert np.array_equal(out["y_fwd"], out["y"])
