#!/usr/bin/env python3
"""Benchmark of the routed-MoE dequant path on one MI355X.

Metric: routed-MoE layer weight-stream GB/s (and us/layer) at bs=1 decode, on the
DeepSeek-V4-Flash-shaped MXFP4 layer (hidden 4096, 256 experts, intermediate
2048, top-6; gate, up and down in MXFP4). One step = one pass of the decode hot
path (gate/up dequant-GEMV with SwiGLU, down dequant-GEMV with the top-6
route-weighted combine) for one token, with a fresh uniform top-6 of the 256
experts per step (no expert repeats within 42 steps, so the weights stream from
HBM rather than from the 256 MB last-level cache). Weights are seeded synthetic
packed blocks resident in HBM before the timed region. Steps are captured in a
HIP graph and replayed, so the host's launch cost does not pace the GPU.

Printed: one JSON line with the metric, a `roofline` object for the dominant
kernel (the gate/up dequant-GEMV, timed with HIP events on its stream) and a
`cpu_baseline` object (the CPU oracle timed on a bounded sample of the same
workload on this host).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --workload iq2_q2k_43 --tokens 2048   # a batched layer: us/layer only
    python bench.py --workload iq2_q2k_43 --layers 43 [--tokens 64]   # 43 distinct layers per step
    python bench.py --workload dense_linear --fmt mxfp8_tiled [--tokens 16]   # a dense FP8 linear
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published peak
# Dense MFMA peak for an FP8 operand (v_mfma_scale_f32_32x32x64_f8f6f4 runs at the
# FP8 rate unless both operands are FP6/FP4): 5.0 PFLOP/s on MI355X.
MFMA_FP8_PEAK_TFLOPS = 5000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Sources the dominant kernel of each workload is compiled from (its own file and
# the device header it includes; moeq_kernels.h holds declarations and parameter
# blocks only): a traffic measurement stays valid while these are unchanged.
KERNEL_SOURCES = {
    "mxfp4_layer": ("moeq_gu_mx4.hip", "moeq_device.h"),
    "prefill_mxfp4": ("moeq_prefill.hip", "moeq_device.h"),
}


def source_digest(workload: str) -> str:
    """Digest of the kernel sources a traffic measurement of `workload` belongs to."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_moe_dequant_amd", "csrc")
    names = KERNEL_SOURCES.get(workload) or sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h")))
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None if absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest(workload):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, ids, rw, x_bits, budget_s: float):
    """The CPU oracle (exact decode + float64 layer) on the first steps of the same
    routing sequence, until the time budget is spent."""
    from threadpoolctl import threadpool_info

    from oracle import formats, moe
    from bit_quantized_moe_dequant_amd import workloads

    spec = wl.spec
    per_step_bytes = None
    done, spent = 0, 0.0
    while spent < budget_s and done < ids.shape[0]:
        e_list = [int(e) for e in ids[done]]
        planes = {(p, e): workloads.host_source_planes(spec, p, e) for p in range(3) for e in e_list}
        t0 = time.perf_counter()

        def weight(p, e):
            fmt, rows, cols = spec.proj(p)
            return formats.dequant(fmt, planes[(p, e)], rows, cols)

        moe.moe_layer(x_bits, ids[done:done + 1], rw[done:done + 1], moe.CachedWeights(weight))
        spent += time.perf_counter() - t0
        done += 1
        if per_step_bytes is None:
            per_step_bytes = sum(formats.packed_bytes(*spec.proj(p)) for p in range(3)) * spec.top_k
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {
        "value": round(per_step_bytes * done / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(max(blas) if blas else 1),
        "kind": "oracle",
        "sample": (f"{done} bs=1 decode steps of the same workload and routing sequence "
                   f"({spent:.1f} s): exact decode of the 6 routed experts' MXFP4 gate/up/down "
                   f"(numpy, one thread) and the float64 layer (BLAS threads = cores); "
                   f"host has {len(os.sched_getaffinity(0))} cores"),
        "us_per_layer": round(spent / done * 1e6, 1),
    }


def cpu_baseline_prefill(wl, ids, rw, x_bits, budget_s: float):
    """The CPU oracle on the prefill workload, expert by expert (bounded memory):
    exact decode of expert e's three MXFP4 matrices, then the W4A8 chain for the
    tokens routed to e (MXFP8 x, h, MXFP8 h, route-weighted down partials)."""
    from threadpoolctl import threadpool_info

    from oracle import formats, moe, mxfp8
    from bit_quantized_moe_dequant_amd import workloads

    spec = wl.spec
    X = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xq, xs = mxfp8.quantize(X)
    pairs = experts = 0
    spent = 0.0
    for e in range(spec.n_experts):    # id order: hashed routing makes loads unrelated to ids
        if spent >= budget_s:
            break
        planes = [workloads.host_source_planes(spec, p, e) for p in range(3)]
        tok, slot = np.nonzero(ids == e)
        t0 = time.perf_counter()
        w = [formats.dequant(spec.proj(p)[0], planes[p], *spec.proj(p)[1:]) for p in range(3)]

        def weight(p, _e, w=w):
            return w[p]

        sub = np.full((tok.size, 1), e, np.int32)
        h = moe.prefill_h(xq[tok], xs[tok], sub, weight).reshape(tok.size, -1)
        hq, hs = mxfp8.quantize(h)
        moe.prefill_y(hq, hs, sub, rw[tok, slot].reshape(-1, 1), weight)
        spent += time.perf_counter() - t0
        pairs += tok.size
        experts += 1
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    per_expert = sum(formats.packed_bytes(*spec.proj(p)) for p in range(3))
    return {
        "value": round(pairs / spec.top_k / spent, 2),
        "unit": "tokens/s",
        "cores": int(max(blas) if blas else 1),
        "kind": "oracle",
        "sample": (f"{experts} of {spec.n_experts} experts (in id order, {pairs} of {ids.size} token-expert "
                   f"pairs, {spent:.1f} s): exact MXFP4 decode (numpy, one thread) and the float64 W4A8 "
                   f"chain (BLAS threads = cores); tokens/s = pairs / top_k / s; "
                   f"host has {len(os.sched_getaffinity(0))} cores"),
        "weight_GBps": round(per_expert * experts / spent / 1e9, 4),
    }


def run_prefill(args, wl):
    """The prefill workload: one step = one MoE layer over T prompt tokens (MXFP8
    quantisation of x, routing, the W4A8 gate/up and down grouped GEMMs, combine)."""
    import torch

    import bit_quantized_moe_dequant_amd as mq
    from bit_quantized_moe_dequant_amd import workloads

    spec = wl.spec
    T = wl.token_counts[0]
    K, W = args.steps, args.warmup
    log(f"workload {wl.name}: building layer ({spec.n_experts} experts) on the device")
    layer = workloads.build_layer(mq, spec)
    ids, rw = workloads.routing(wl, T)
    x_bits = workloads.activations(wl, T)
    loads = np.bincount(ids.reshape(-1), minlength=spec.n_experts)
    touched = int((loads > 0).sum())
    P = T * spec.top_k
    ids_t = torch.from_numpy(ids).cuda()
    rw_t = torch.from_numpy(rw).cuda()
    x_t = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty((T, spec.hidden), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    step_bytes = touched * layer.expert_bytes()
    gu_bytes = touched * (layer.gate.algorithmic_bytes() + layer.up.algorithmic_bytes())
    gu_flop = 2 * P * 2 * spec.inter * spec.hidden
    step_flop = gu_flop + 2 * P * spec.hidden * spec.inter

    def step():
        mq.expert_forward(layer, x_t, ids_t, rw_t, y=y, ws=ws)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(K):
                step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / K
    log(f"{K} steps: wall {wall_s * 1e3:.2f} ms -> {ms_per_step * 1e3:.1f} us/layer (events)")

    # dominant kernel: the gate/up grouped GEMM (route and x quantisation done once)
    xq, xs = mq.quantize_mxfp8(x_t)
    mq.route(layer, ids_t, ws=ws)
    hq = torch.empty((P, spec.inter), dtype=torch.uint8, device="cuda")
    hs = torch.empty((P, spec.inter // 32), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    graph_gu = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph_gu, stream=cap):
            for _ in range(K):
                mq.prefill_gate_up(layer, xq, xs, ids_t, hq=hq, hs=hs, ws=ws)
        graph_gu.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(cap)
        graph_gu.replay()
        g1.record(cap)
    torch.cuda.synchronize()
    gu_us = g0.elapsed_time(g1) * 1e3 / K
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    gu_tflops = gu_flop / (gu_us * 1e-6) / 1e12
    err = mq.check_device_error(ws)
    if err:
        sys.exit(f"device error word {err:#x}")
    value = T / (ms_per_step * 1e-3)
    out = {
        "metric": "routed-MoE layer prefill tokens/s (T=2048, W4A8 grouped GEMM) + weight-stream GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": "DeepSeek-V4-Flash-shaped routed-MoE layer, prefill of 2048 tokens routed by a "
                           "seeded hash of Zipf token ids: hidden 4096, 256 experts, intermediate 2048, "
                           "top-6, MXFP4 weights x MXFP8 activations, fp32 accumulate",
            "tokens_per_step": T,
            "experts_touched": touched,
            "expert_load_min_mean_max": [int(loads.min()), round(float(loads.mean()), 1), int(loads.max())],
            "weight_bytes_per_step": step_bytes,
            "flop_per_step": step_flop,
            "launch": "HIP graph of the timed steps",
            "parallelism": "single GPU",
        },
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "weight_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "pct_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "layer_tflops": round(step_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": {
            "kernel": "prefill gate/up grouped GEMM (block-scaled FP8xFP4 MFMA) + SwiGLU + MXFP8 of h",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl.name),
            "launch_us": round(gu_us, 3),
            "algorithmic_bytes_per_launch": gu_bytes,
            "mfma_tflops": round(gu_tflops, 2),
            "mfma_peak_tflops": MFMA_FP8_PEAK_TFLOPS,
            "mfma_frac": round(gu_tflops / MFMA_FP8_PEAK_TFLOPS, 4),
            "flop_per_launch": gu_flop,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline_prefill(wl, ids, rw, x_bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)


FMT_LABEL = {1: "MXFP4 (e2m1 + e8m0/32)", 2: "NVFP4 (e2m1 + e4m3/16 + fp32 scale_2)", 3: "Q2_K", 4: "IQ2_XXS",
             5: "FP8 E4M3 + UE8M0/128x128"}
GU_KERNEL = {
    1: "gate/up + SwiGLU: MXFP4 weights straight into v_mfma_scale_f32_16x16x128_f8f6f4 (bf16 token as two E4M3 terms)",
    2: "gate/up + SwiGLU: NVFP4 weights into v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 scale per 16 on the results",
    4: "gate/up + SwiGLU: IQ2_XXS dequant-GEMV (codebook in LDS, exact bf16 weights, v_dot2_f32_bf16)",
}


def run_layers(args, wl):
    """Decode through N distinct layers back to back (--layers N, e.g. the 43 MoE
    layers of the 2-bit hybrid model): N layers are built with their own weights
    (43 x 1.8 GB for IQ2_XXS + Q2_K, far beyond the 256 MB MALL), and one step is one
    forward of every layer at T tokens, each layer with its own activations and a
    fresh uniform top-k per token. K steps are captured in one HIP graph and timed
    with HIP events; it prints us per layer, us per step and tokens/s through the
    stack. Not the headline metric."""
    import torch

    import bit_quantized_moe_dequant_amd as mq
    from bit_quantized_moe_dequant_amd import synth, workloads

    N, T, K, W = args.layers, args.tokens, args.steps, args.warmup
    base = wl.spec
    log(f"workload {wl.name}: building {N} layers ({base.n_experts} experts each) on the device")
    layers = []
    for li in range(N):
        spec = workloads.LayerSpec(base.hidden, base.inter, base.n_experts, base.top_k, base.fmt_gate_up,
                                   base.fmt_down, base.seed, li)
        layers.append(workloads.build_layer(mq, spec))
    torch.cuda.synchronize()
    all_bytes = sum(l.expert_bytes() * l.n_experts for l in layers)
    log(f"built: {all_bytes / 1e9:.1f} GB of weights")
    xs = [torch.from_numpy(synth.activations_bf16(base.seed + 11 * li, T, base.hidden).view(np.int16)).cuda().view(
        torch.bfloat16) for li in range(N)]
    routes = [[synth.uniform_routing(base.seed + 1000 * li + 7 * i, T, base.n_experts, base.top_k)
               for li in range(N)] for i in range(W + K)]
    ids_t = [[torch.from_numpy(r[0]).cuda() for r in step] for step in routes]
    rw_t = [[torch.from_numpy(r[1]).cuda() for r in step] for step in routes]
    y = torch.empty((T, base.hidden), dtype=torch.float32, device="cuda")
    ws = layers[0].workspace(T)
    touched = float(np.mean([np.unique(r[0]).size for step in routes[W:] for r in step]))
    step_bytes = N * touched * layers[0].expert_bytes()

    def step(i):
        for li in range(N):
            mq.expert_forward(layers[li], xs[li], ids_t[i][li], rw_t[i][li], y=y, ws=ws)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / K
    err = mq.check_device_error(ws)
    if err:
        sys.exit(f"device error word {err:#x}")
    log(f"{K} steps through {N} layers at T={T}: {ms_per_step * 1e3:.1f} us/step, "
        f"{ms_per_step * 1e3 / N:.2f} us/layer")
    print(json.dumps({
        "metric": f"routed-MoE decode through {N} layers at T={T}: us/layer (not the headline)",
        "value": round(ms_per_step * 1e3 / N, 3),
        "unit": "us/layer",
        "higher_is_better": False,
        "steps": K,
        "warmup": W,
        "us_per_step": round(ms_per_step * 1e3, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "experts_touched_per_layer": round(touched, 1),
        "weight_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": N, "tokens_per_step": T,
                   "weight_bytes_all_layers": all_bytes,
                   "routing": "uniform top-k per token, fresh per step and layer",
                   "launch": "HIP graph of the timed steps"},
    }), flush=True)


def run_batch(args, wl):
    """A decode workload at T > 1 tokens per step (--tokens): one step = one MoE layer
    over T tokens with a fresh uniform top-k per token (routing, gate/up, down,
    combine), K steps captured in one HIP graph. Not the headline metric: it prints
    us/layer, tokens/s and the weight bytes of the touched experts per second."""
    import torch

    import bit_quantized_moe_dequant_amd as mq
    from bit_quantized_moe_dequant_amd import synth, workloads

    spec = wl.spec
    T, K, W = args.tokens, args.steps, args.warmup
    log(f"workload {wl.name} at T={T}: building layer ({spec.n_experts} experts) on the device")
    layer = workloads.build_layer(mq, spec)
    routes = [synth.uniform_routing(spec.seed + 77 * i, T, spec.n_experts, spec.top_k) for i in range(W + K)]
    ids_t = [torch.from_numpy(r[0]).cuda() for r in routes]
    rw_t = [torch.from_numpy(r[1]).cuda() for r in routes]
    x_t = torch.from_numpy(synth.activations_bf16(spec.seed + 5, T, spec.hidden).view(np.int16)).cuda().view(
        torch.bfloat16)
    y = torch.empty((T, spec.hidden), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    touched = float(np.mean([np.unique(r[0]).size for r in routes[W:]]))
    step_bytes = touched * layer.expert_bytes()

    def step(i):
        mq.expert_forward(layer, x_t, ids_t[i], rw_t[i], y=y, ws=ws)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / K
    err = mq.check_device_error(ws)
    if err:
        sys.exit(f"device error word {err:#x}")
    log(f"{K} steps at T={T}: {ms_per_step * 1e3:.1f} us/layer")
    print(json.dumps({
        "metric": f"routed-MoE layer us/layer at T={T} (batched decode / prefill, not the headline)",
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/layer",
        "higher_is_better": False,
        "steps": K,
        "warmup": W,
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "experts_touched": round(touched, 1),
        "weight_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": T, "routing": "uniform top-k per token, fresh per step",
                   "launch": "HIP graph of the timed steps"},
    }), flush=True)


def run_dense_linear(args):
    """A dense FP8 linear (the pages' 4096 x 4096 shared-expert / attention size) in
    one format, T tokens per step: y = W x with W rotating over 40 stored copies
    (672 MB, so every step reads its weights from HBM, not from the 256 MB
    last-level cache). Not the headline metric: prints us per linear and GB/s."""
    import torch

    import bit_quantized_moe_dequant_amd as mq
    from bit_quantized_moe_dequant_amd import synth, workloads

    fmt = mq.FMT_BY_NAME[args.fmt]
    rows = cols = 4096
    T, K, W = args.tokens, args.steps, args.warmup
    n_copies = 40
    log(f"dense linear {args.fmt} {rows}x{cols}, T={T}: building {n_copies} copies")
    Wt = workloads.build_dense(mq, fmt, 20262, rows, cols, n_copies)
    x = torch.from_numpy(synth.activations_bf16(20262 + T, T, cols).view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty((T, rows), dtype=torch.float32, device="cuda")
    nbytes = mq.packed_bytes(fmt, rows, cols)

    def step(i):
        mq.linear(Wt, i % n_copies, x, y=y)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    log(f"{K} linears: {us:.2f} us each")
    print(json.dumps({
        "metric": f"dense FP8 linear {rows}x{cols} us per call at T={T} (not the headline)",
        "value": round(us, 3), "unit": "us", "higher_is_better": False, "steps": K, "warmup": W,
        "weight_GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 /
                                                                                  HBM_PEAK_GBS, 2),
        "weight_bytes": nbytes, "data": "synthetic",
        "config": {"workload": "dense_linear", "format": args.fmt, "rows": rows, "cols": cols, "tokens": T,
                   "copies_rotated": n_copies, "launch": "HIP graph of the timed steps"},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 2000 decode, 100 prefill)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mxfp4_layer")
    ap.add_argument("--tokens", type=int, default=1,
                    help="decode workloads: tokens per step (T > 1 prints a separate us/layer line)")
    ap.add_argument("--fmt", default="mxfp8_tiled",
                    help="dense_linear workload: fp8_b128, fp8_b32, mxfp8 or mxfp8_tiled")
    ap.add_argument("--layers", type=int, default=1,
                    help="decode through this many distinct layers per step (e.g. 43 for iq2_q2k_43)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)")

    import torch

    import bit_quantized_moe_dequant_amd as mq
    from bit_quantized_moe_dequant_amd import synth, workloads

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "copies": 3}))
        return
    if args.workload == "dense_linear":
        if args.steps is None:
            args.steps = 2000
        return run_dense_linear(args)
    wl = workloads.WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = 100 if wl.prefill else (20 if args.tokens > 1 or args.layers > 1 else 2000)
    if wl.prefill:
        return run_prefill(args, wl)
    if args.layers > 1:
        return run_layers(args, wl)
    if args.tokens > 1:
        return run_batch(args, wl)
    spec = wl.spec
    K, W = args.steps, args.warmup
    log(f"workload {wl.name}: building layer ({spec.n_experts} experts) on the device")
    layer = workloads.build_layer(mq, spec)
    torch.cuda.synchronize()

    ids, rw = synth.cold_routing_sequence(spec.seed, W + K, spec.n_experts, spec.top_k)
    x_bits = workloads.activations(wl, 1)
    ids_t = torch.from_numpy(ids).cuda()
    rw_t = torch.from_numpy(rw).cuda()
    x_t = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty((1, spec.hidden), dtype=torch.float32, device="cuda")
    h = torch.empty((1, spec.top_k, spec.inter), dtype=torch.float32, device="cuda")
    ws = layer.workspace(1)
    step_bytes = spec.top_k * layer.expert_bytes()
    gu_bytes = spec.top_k * (layer.gate.algorithmic_bytes() + layer.up.algorithmic_bytes())

    def step(i):
        mq.expert_forward(layer, x_t, ids_t[i:i + 1], rw_t[i:i + 1], y=y, ws=ws)

    # warmup (eager), then capture the timed steps into one graph
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log(f"capturing {K} steps")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
    torch.cuda.synchronize()
    graph.replay()                                   # first replay uploads the graph
    torch.cuda.synchronize()

    # timed region: K steps
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    # Time per step from the HIP events around the replay: the GPU's own clock over
    # the K steps, without the host's launch and synchronisation latency.
    ms_per_step = gpu_ms / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"{K} steps: wall {wall_s * 1e3:.2f} ms, events {gpu_ms:.2f} ms -> {ms_per_step * 1e3:.2f} us/layer")

    # Dominant kernel: the gate/up dequant-GEMV, timed in the same regime as the
    # steps (a graph of K launches over the same routing sequence, replayed on its
    # capture stream, bracketed by HIP events on that stream). Inside a graph the
    # launches run back to back, so the average per launch is the kernel's time.
    graph_gu = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph_gu, stream=cap):
            for i in range(K):
                mq.gate_up(layer, x_t, ids_t[W + i:W + i + 1], h=h, ws=ws)
        graph_gu.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(cap)
        graph_gu.replay()
        g1.record(cap)
    torch.cuda.synchronize()
    gu_us = g0.elapsed_time(g1) * 1e3 / K
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic = measured_traffic(wl.name)
    err = mq.check_device_error(ws)
    if err:
        sys.exit(f"device error word {err:#x}")

    out = {
        "metric": "routed-MoE layer weight-stream GB/s (% of HBM peak) + us/layer, bs=1 decode",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": f"DeepSeek-V4-Flash-shaped routed-MoE layer, bs=1 decode: hidden {spec.hidden}, "
                           f"{spec.n_experts} experts, intermediate {spec.inter}, top-{spec.top_k}, "
                           f"gate/up {FMT_LABEL[spec.fmt_gate_up]}, down {FMT_LABEL[spec.fmt_down]}",
            "tokens_per_step": 1,
            "weight_bytes_per_step": step_bytes,
            "routing": "uniform top-6 per step, no expert repeated within 42 steps (cold)",
            "launch": "HIP graph of the timed steps",
            "parallelism": "single GPU",
        },
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "moe_tokens_per_s_43_layers": round(1e3 / (ms_per_step * 43), 1),
        "roofline": {
            "kernel": GU_KERNEL.get(spec.fmt_gate_up, "gate/up + SwiGLU dequant-GEMV"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "launch_us": round(gu_us, 3),
            "algorithmic_bytes_per_launch": gu_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(wl, ids[W:], rw[W:], x_bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
