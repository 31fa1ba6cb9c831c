"""The forward captured in a HIP graph: every replay equals the eager result bit for
bit (the forward has no float atomics, so eager runs are deterministic too). Replays
are interleaved with unrelated eager work and synchronisations, so state that a
graph would only set up on its first replay (cleared counters, the routing tables in
the workspace) is exercised on every replay.

Covers the three launch sequences of the forward: bs=1 (gate/up + single-token
down), T=16 (routing, grouped GEMVs, combine) and T=256 prefill (MXFP8 of x,
routing, the two grouped GEMMs, combine)."""
import sys

import numpy as np
import pytest

import bit_quantized_moe_dequant_amd as mq
from bit_quantized_moe_dequant_amd import synth, workloads
from tests.test_gpu_parity import cuda, upload_layer, x_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("case", [
    # (H, I, E, K, gate/up format, down format, T, calls per graph)
    (1024, 512, 16, 6, mq.FMT_MXFP4, mq.FMT_MXFP4, 1, 3),
    (1024, 512, 16, 6, mq.FMT_NVFP4, mq.FMT_Q2_K, 16, 2),
    (1024, 512, 16, 6, mq.FMT_NVFP4, mq.FMT_MXFP4, 1, 3),   # NVFP4 gate/up on the matrix unit
    (512, 256, 4, 2, mq.FMT_IQ2_XXS, mq.FMT_Q2_K, 32, 2),   # 16 pairs per expert: the two-tile IQ2_XXS gate/up and grouped Q2_K down
    (512, 256, 8, 2, mq.FMT_MXFP4, mq.FMT_MXFP4, 256, 2),   # prefill path (T >= 128, MXFP4)
])
def test_graph_replays_match_eager(case):
    H, I, E, K, fg, fd, T, n_calls = case
    say("graph", case)
    spec = workloads.LayerSpec(H, I, E, K, fg, fd, seed=7100 + T)
    layer = upload_layer(spec)
    calls = []
    for c in range(n_calls):
        ids, rw = synth.uniform_routing(70 + c, T, E, K)
        x = synth.activations_bf16(80 + c, T, H)
        calls.append((x_tensor(x), cuda(ids), cuda(rw)))
    ws = layer.workspace(T)
    mq.check_device_error(ws)
    outs = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(n_calls)]

    def forward_all():
        for (x, ids, rw), y in zip(calls, outs):
            mq.expert_forward(layer, x, ids, rw, y=y, ws=ws)

    forward_all()
    torch.cuda.synchronize()
    eager = [y.clone() for y in outs]

    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            forward_all()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for y in outs:
            y.fill_(float("nan"))
        # unrelated eager work between replays (it also dirties the workspace's routing
        # area for the grouped paths: the graph must rebuild it on every replay)
        if T > 1:
            other_ids, _ = synth.uniform_routing(900 + rep, T, E, K)
            mq.route(layer, cuda(other_ids), ws=ws)
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for c, (y, ref) in enumerate(zip(outs, eager)):
            assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), (rep, c)
    assert mq.check_device_error(ws) == 0
    del graph
