"""The five workloads and builders of their synthetic device tensors.

Shapes follow the DeepSeek-V4-Flash base model (W4A16-FP8 card, base-model
table: hidden 4096, 256 routed experts, top-6, 43 layers); the intermediate size
2048 is an assumption (the pages do not print it). Weight bytes are drawn by the
seeded generator (``synth``) on the device and can be regenerated per expert on
the host; activations and routing are drawn on the host.

  single_expert   one MXFP4 expert, H 1024, I 512, 1 token
  mxfp4_layer     MXFP4 layer, bs 1 (the decode metric's workload)
  nvfp4_q2k       NVFP4 gate/up + Q2_K down, bs 1 and 16, plus an FP8 block-128
                  4096 x 4096 dense linear
  iq2_q2k_43      IQ2_XXS gate/up + Q2_K down, 43 layers, bs 1 and 64
  prefill_mxfp4   MXFP4 layer, 2048 prompt tokens routed by a hash of the token id
  iq2_mxfp4       IQ2_XXS gate/up + MXFP4 down (a late layer of the measured-KL mix)
  mxfp4_iq2       MXFP4 gate/up + IQ2_XXS down (an early layer of the mix)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

from . import synth

FMT = synth.FMT_NAMES


@dataclass
class LayerSpec:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    fmt_gate_up: int
    fmt_down: int
    seed: int
    layer: int = 0

    def proj(self, p: int) -> Tuple[int, int, int]:
        """(fmt, rows, cols) of projection p (0 gate, 1 up, 2 down)."""
        if p in (0, 1):
            return self.fmt_gate_up, self.inter, self.hidden
        return self.fmt_down, self.hidden, self.inter


@dataclass
class Workload:
    name: str
    spec: LayerSpec
    token_counts: List[int]
    n_layers: int = 1
    linear: Tuple[int, int] | None = None      # (rows, cols) of an FP8 block-128 dense linear
    prefill: bool = False
    notes: str = ""
    extra: dict = field(default_factory=dict)


def _seed(i):
    return 20260 + i


WORKLOADS = {
    "single_expert": Workload("single_expert", LayerSpec(1024, 512, 1, 1, synth.FMT_MXFP4, synth.FMT_MXFP4, _seed(0)),
                              [1]),
    "mxfp4_layer": Workload("mxfp4_layer", LayerSpec(4096, 2048, 256, 6, synth.FMT_MXFP4, synth.FMT_MXFP4, _seed(1)),
                            [1]),
    "nvfp4_q2k": Workload("nvfp4_q2k", LayerSpec(4096, 2048, 256, 6, synth.FMT_NVFP4, synth.FMT_Q2_K, _seed(2)),
                          [1, 16], linear=(4096, 4096)),
    "iq2_q2k_43": Workload("iq2_q2k_43", LayerSpec(4096, 2048, 256, 6, synth.FMT_IQ2_XXS, synth.FMT_Q2_K, _seed(3)),
                           [1, 64], n_layers=43),
    # layers of the measured-KL mix (IQ2_XXS floor, MXFP4 promoted per projection):
    # MXFP4 on down in late layers, on gate/up in early ones
    "iq2_mxfp4": Workload("iq2_mxfp4", LayerSpec(4096, 2048, 256, 6, synth.FMT_IQ2_XXS, synth.FMT_MXFP4, _seed(5)),
                          [1, 2048]),
    "mxfp4_iq2": Workload("mxfp4_iq2", LayerSpec(4096, 2048, 256, 6, synth.FMT_MXFP4, synth.FMT_IQ2_XXS, _seed(6)),
                          [1, 2048]),
    "prefill_mxfp4": Workload("prefill_mxfp4",
                              LayerSpec(4096, 2048, 256, 6, synth.FMT_MXFP4, synth.FMT_MXFP4, _seed(4)),
                              [2048], prefill=True),
}

_FIELDS = {
    synth.FMT_MXFP4: [synth.FIELD_RAW, synth.FIELD_E8M0_119_123],
    synth.FMT_NVFP4: [synth.FIELD_RAW, synth.FIELD_E4M3_08_28],
    synth.FMT_FP8_B128: [synth.FIELD_E4M3_FINITE, synth.FIELD_E8M0_119_123],
    synth.FMT_FP8_B32: [synth.FIELD_E4M3_FINITE, synth.FIELD_E8M0_119_123],
    synth.FMT_MXFP8: [synth.FIELD_E4M3_FINITE, synth.FIELD_E8M0_119_123],
    synth.FMT_Q2_K: [synth.FIELD_Q2K_BLOCK],
    synth.FMT_IQ2_XXS: [synth.FIELD_IQ2_BLOCK],
}


def host_source_planes(spec: LayerSpec, proj: int, expert: int):
    """Source-layout planes of one expert tensor, regenerated on the host."""
    fmt, rows, cols = spec.proj(proj)
    return synth.expert_source(spec.seed, spec.layer, proj, fmt, rows, cols, expert)


def host_scale2(spec: LayerSpec, proj: int) -> np.ndarray:
    return synth.scale2_values(spec.seed, spec.layer, proj, spec.n_experts)


def host_grid() -> np.ndarray:
    return synth.iq2_standin_grid()


def fill_weight(mq, spec: LayerSpec, proj: int, fmt: int, rows: int, cols: int, n_experts: int,
                layer_index: int | None = None):
    """A device Weight for (fmt, rows, cols) filled from the generator streams of
    (seed, layer, proj): expert e is bytes [e * plane, (e + 1) * plane) of each stream."""
    import torch
    layer = spec.layer if layer_index is None else layer_index
    W = mq.Weight.empty(fmt, rows, cols, n_experts)
    if fmt in (synth.FMT_Q2_K, synth.FMT_IQ2_XXS):
        bs = 84 if fmt == synth.FMT_Q2_K else 66
        per = rows * (cols // 256) * bs
        tab = torch.from_numpy(synth.d_table().astype(np.int16)).cuda()
        p0 = mq.plane_bytes(fmt, rows, cols, 0)
        p1 = mq.plane_bytes(fmt, rows, cols, 1)
        # generate a few experts at a time to bound the staging buffer
        step = max(1, min(n_experts, (256 << 20) // per))
        stage = torch.empty(step * per, dtype=torch.uint8, device="cuda")
        for e0 in range(0, n_experts, step):
            n = min(step, n_experts - e0)
            buf = stage[:n * per]
            mq.synth_fill(buf, spec.seed, synth.stream_id(layer, proj, 0), e0 * per, _FIELDS[fmt][0], tab)
            if W.expert_stride == p0 and W.scale_expert_stride == p1:
                mq.pack_ggml_device(fmt, buf, rows, cols, n, W.data[e0 * p0:], W.scales[e0 * p1:])
            else:
                for j in range(n):
                    e = e0 + j
                    mq.pack_ggml_device(fmt, buf[j * per:(j + 1) * per], rows, cols, 1,
                                        W.data[e * W.expert_stride:], W.scales[e * W.scale_expert_stride:])
        torch.cuda.synchronize()
    else:
        for p, tensor, stride in ((0, W.data, W.expert_stride), (1, W.scales, W.scale_expert_stride)):
            nb = mq.plane_bytes(fmt, rows, cols, p)
            sid = synth.stream_id(layer, proj, p)
            if stride == nb:
                mq.synth_fill(tensor[:nb * n_experts], spec.seed, sid, 0, _FIELDS[fmt][p])
            else:
                for e in range(n_experts):
                    mq.synth_fill(tensor[e * stride:e * stride + nb], spec.seed, sid, e * nb, _FIELDS[fmt][p])
    if fmt == synth.FMT_NVFP4:
        W.scale2.copy_(torch.from_numpy(synth.scale2_values(spec.seed, layer, proj, n_experts)))
    if fmt == synth.FMT_IQ2_XXS:
        W.grid = torch.from_numpy(host_grid().reshape(-1)).cuda()
    return W


def build_layer(mq, spec: LayerSpec):
    g = fill_weight(mq, spec, 0, *spec.proj(0), spec.n_experts)
    u = fill_weight(mq, spec, 1, *spec.proj(1), spec.n_experts)
    d = fill_weight(mq, spec, 2, *spec.proj(2), spec.n_experts)
    return mq.Layer(spec.hidden, spec.inter, spec.n_experts, spec.top_k, g, u, d)


def build_linear(mq, seed: int, rows: int, cols: int, layer: int = 0):
    spec = LayerSpec(cols, rows, 1, 1, synth.FMT_FP8_B128, synth.FMT_FP8_B128, seed, layer)
    return fill_weight(mq, spec, synth.PROJ_LINEAR, synth.FMT_FP8_B128, rows, cols, 1)


def host_linear_planes(seed: int, rows: int, cols: int, layer: int = 0, fmt: int = synth.FMT_FP8_B128,
                       expert: int = 0):
    return synth.expert_source(seed, layer, synth.PROJ_LINEAR, fmt, rows, cols, expert)


def build_dense(mq, fmt: int, seed: int, rows: int, cols: int, n_copies: int = 1):
    """A dense FP8 weight with n_copies independent tensors (rotated through by the
    benchmark so that every launch reads HBM). MXFP8_TILED is filled as row-major
    MXFP8 and converted to the pre-stored order on the device."""
    src = synth.FMT_MXFP8 if fmt == mq.FMT_MXFP8_TILED else fmt
    spec = LayerSpec(cols, rows, n_copies, 1, src, src, seed, 0)
    W = fill_weight(mq, spec, synth.PROJ_LINEAR, src, rows, cols, n_copies)
    if fmt != mq.FMT_MXFP8_TILED:
        return W
    td, ts = mq.mxfp8_to_tiled(W.data, W.scales, rows, cols, n_copies)
    return mq.Weight(fmt, rows, cols, n_copies, td, ts, expert_stride=W.expert_stride,
                     scale_expert_stride=W.scale_expert_stride)


def routing(workload: Workload, T: int, step: int = 0):
    """(ids int32 [T, K], rw fp32 [T, K]) for a workload and token count."""
    s = workload.spec
    if workload.prefill:
        tok = synth.zipf_token_ids(s.seed, T)
        return synth.hash_routing(s.seed, tok, s.n_experts, s.top_k)
    if s.n_experts == 1:
        return np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32)
    return synth.uniform_routing(s.seed + 1000 * step + T, T, s.n_experts, s.top_k)


def activations(workload: Workload, T: int, layer: int = 0):
    return synth.activations_bf16(workload.spec.seed * 100 + layer + 7 * T, T, workload.spec.hidden)
