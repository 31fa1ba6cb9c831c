"""MI355X (gfx950) block-quantized routed-MoE kernels: Python binding.

A thin ctypes layer over ``libmoeq.so`` (C ABI in ``include/moeq.h``). PyTorch
provides device memory and the current HIP stream; every step of the path runs
in the library's HIP kernels. There is no CPU fallback: if the library is not
built, or no GPU is present, calls raise.

    import bit_quantized_moe_dequant_amd as mq
    W = mq.Weight.empty(mq.FMT_MXFP4, rows, cols, n_experts)   # device planes
    L = mq.Layer(hidden, inter, n_experts, top_k, gate, up, down)
    y = mq.expert_forward(L, x_bf16, ids, rw)
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoeq.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "moeq.h")

FMT_MXFP4, FMT_NVFP4, FMT_Q2_K, FMT_IQ2_XXS, FMT_FP8_B128 = 1, 2, 3, 4, 5
FMT_MXFP8, FMT_FP8_B32, FMT_MXFP8_TILED = 6, 7, 8
FMT_BY_NAME = {"mxfp4": 1, "nvfp4": 2, "q2_k": 3, "iq2_xxs": 4, "fp8_b128": 5, "mxfp8": 6, "fp8_b32": 7,
               "mxfp8_tiled": 8}

MOEQ_OK = 0
MOEQ_E_SCRATCH = -8
NOALLOC_SCRATCH_BYTES = 32 << 20
ABI_VERSION = 2
DEVERR_EXPERT_ID = 1


class MoeqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib().moeq_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{fn} failed: {msg} ({status})")


class MoeqWeight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("rows", ctypes.c_int), ("cols", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("data", ctypes.c_void_p), ("expert_stride", ctypes.c_size_t), ("scales", ctypes.c_void_p),
                ("scale_expert_stride", ctypes.c_size_t), ("scale2", ctypes.c_void_p), ("grid", ctypes.c_void_p)]


class MoeqLayer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("inter", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("gate", MoeqWeight), ("up", MoeqWeight), ("down", MoeqWeight)]


_LIB = None
_vp, _i, _sz, _u8p = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "moeq_abi_version": (_i, []),
    "moeq_status_string": (ctypes.c_char_p, [_i]),
    "moeq_plane_bytes": (_sz, [_i, _i, _i, _i]),
    "moeq_packed_bytes": (_sz, [_i, _i, _i]),
    "moeq_pack_ggml": (_i, [_i, _vp, _i, _i, _vp, _vp]),
    "moeq_pack_ggml_device": (_i, [_i, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "moeq_mxfp4_to_nvfp4": (_i, [_vp, _vp, _i, _i, _vp, _vp, _vp]),
    "moeq_dequant": (_i, [ctypes.POINTER(MoeqWeight), _i, _vp, _vp]),
    "moeq_workspace_bytes": (_sz, [ctypes.POINTER(MoeqLayer), _i]),
    "moeq_workspace_init": (_i, [_vp, _sz, _vp]),
    "moeq_expert_forward": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "moeq_expert_forward_noalloc": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "moeq_route": (_i, [ctypes.POINTER(MoeqLayer), _vp, _i, _vp, _sz, _vp]),
    "moeq_gate_up": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "moeq_down": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "moeq_gate_up_timed": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _i, _vp, _vp, _sz, _vp, _vp, _vp]),
    "moeq_prefill_gate_up": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moeq_prefill_down": (_i, [ctypes.POINTER(MoeqLayer), _vp, _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "moeq_linear": (_i, [ctypes.POINTER(MoeqWeight), _i, _vp, _i, _vp, _vp]),
    "moeq_quantize_mxfp8": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "moeq_quantize_mxfp8_f32": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "moeq_check_device_error": (_i, [_vp, _vp, ctypes.POINTER(ctypes.c_uint32), _i]),
    "moeq_mxfp8_to_tiled": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "moeq_mxfp4_to_nvfp4_device": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moeq_nvfp4_to_mxfp4_device": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "moeq_synth_fill": (_i, [_vp, _sz, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, _i, _vp, _vp]),
}


def library_path() -> str:
    return _LIB_PATH


def _lib():
    """Load libmoeq.so (fails loudly if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               f"`python -m bit_quantized_moe_dequant_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        if lib.moeq_abi_version() != ABI_VERSION:
            raise RuntimeError("libmoeq.so ABI version mismatch")
        _LIB = lib
    return _LIB


def header_functions(path: str = _HEADER):
    """Names of the functions declared in a header of this library."""
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moeq_[a-z0-9_]+)\s*\(", txt)))


def _check(fn, rc):
    if rc != MOEQ_OK:
        raise MoeqError(fn, rc)


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _stream_ptr():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must be on the GPU")


def _want(name, t, dtypes, shape):
    """Raise ValueError unless t is a contiguous tensor of one of `dtypes` with
    exactly `shape` (whether it is on the GPU is checked after all of them). The C ABI sees raw pointers only, so a wrong dtype (int64 ids
    read as pairs of int32), a short buffer or a strided view must be caught here,
    before anything is launched."""
    torch = _torch()
    if t is None:
        raise ValueError(f"{name}: missing")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _tokens(name, t, width):
    """Number of rows of a [T, width] tensor (before its full check)."""
    if t is None or not hasattr(t, "shape") or len(t.shape) != 2 or t.shape[1] != width:
        raise ValueError(f"{name}: expected shape (T, {width}), got {None if t is None else tuple(t.shape)}")
    return int(t.shape[0])


def _want_ws(layer, T, ws):
    torch = _torch()
    _want("ws", ws, (torch.uint8,), (ws.numel(),) if ws is not None and ws.dim() == 1 else (-1,))
    if ws.numel() < workspace_bytes(layer, T):
        raise ValueError(f"ws: {ws.numel()} bytes, need {workspace_bytes(layer, T)}")


def _routing_args(layer, T, ids, rw=None):
    torch = _torch()
    _want("ids", ids, (torch.int32,), (T, layer.top_k))
    if rw is not None:
        _want("rw", rw, (torch.float32,), (T, layer.top_k))


def plane_bytes(fmt: int, rows: int, cols: int, plane: int) -> int:
    return int(_lib().moeq_plane_bytes(fmt, rows, cols, plane))


def packed_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(_lib().moeq_packed_bytes(fmt, rows, cols))


def _round16(n: int) -> int:
    return (n + 15) // 16 * 16


class Weight:
    """Expert-major block-quantized tensor in the library's device layout."""

    def __init__(self, fmt, rows, cols, n_experts, data, scales, scale2=None, grid=None,
                 expert_stride=None, scale_expert_stride=None):
        self.fmt, self.rows, self.cols, self.n_experts = int(fmt), int(rows), int(cols), int(n_experts)
        self.data, self.scales, self.scale2, self.grid = data, scales, scale2, grid
        self.expert_stride = expert_stride if expert_stride is not None else _round16(plane_bytes(fmt, rows, cols, 0))
        self.scale_expert_stride = (scale_expert_stride if scale_expert_stride is not None
                                    else _round16(plane_bytes(fmt, rows, cols, 1)))

    @classmethod
    def empty(cls, fmt, rows, cols, n_experts, device="cuda"):
        torch = _torch()
        p0, p1 = plane_bytes(fmt, rows, cols, 0), plane_bytes(fmt, rows, cols, 1)
        if p0 == 0 or p1 == 0:
            raise ValueError(f"shape {rows}x{cols} not valid for format {fmt}")
        s0, s1 = _round16(p0), _round16(p1)
        data = torch.empty(s0 * n_experts, dtype=torch.uint8, device=device)
        scales = torch.empty(s1 * n_experts, dtype=torch.uint8, device=device)
        scale2 = torch.ones(n_experts, dtype=torch.float32, device=device) if fmt == FMT_NVFP4 else None
        return cls(fmt, rows, cols, n_experts, data, scales, scale2, None, s0, s1)

    def expert_planes(self, e):
        p0, p1 = plane_bytes(self.fmt, self.rows, self.cols, 0), plane_bytes(self.fmt, self.rows, self.cols, 1)
        return (self.data[e * self.expert_stride:e * self.expert_stride + p0],
                self.scales[e * self.scale_expert_stride:e * self.scale_expert_stride + p1])

    def struct(self) -> MoeqWeight:
        return MoeqWeight(self.fmt, self.rows, self.cols, self.n_experts, self.data.data_ptr(), self.expert_stride,
                          self.scales.data_ptr(), self.scale_expert_stride,
                          0 if self.scale2 is None else self.scale2.data_ptr(),
                          0 if self.grid is None else self.grid.data_ptr())

    def algorithmic_bytes(self) -> int:
        """Bytes of one expert tensor at the format's bits per weight."""
        return packed_bytes(self.fmt, self.rows, self.cols)


class Layer:
    def __init__(self, hidden, inter, n_experts, top_k, gate: Weight, up: Weight, down: Weight):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.gate, self.up, self.down = gate, up, down
        self._ws = {}

    def struct(self) -> MoeqLayer:
        return MoeqLayer(self.hidden, self.inter, self.n_experts, self.top_k, self.gate.struct(), self.up.struct(),
                         self.down.struct())

    def expert_bytes(self) -> int:
        return self.gate.algorithmic_bytes() + self.up.algorithmic_bytes() + self.down.algorithmic_bytes()

    def workspace(self, T: int):
        """A zero-initialised workspace for T tokens (cached per T)."""
        torch = _torch()
        n = workspace_bytes(self, T)
        ws = self._ws.get(T)
        if ws is None or ws.numel() < n:
            ws = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
            off = (-ws.data_ptr()) % 256
            ws = ws[off:off + n]
            self._ws[T] = ws
        return ws


def workspace_bytes(layer: Layer, T: int) -> int:
    L = layer.struct()
    n = int(_lib().moeq_workspace_bytes(ctypes.byref(L), T))
    if n == 0:
        raise MoeqError("moeq_workspace_bytes", -4)
    return n


# ---------------------------------------------------------------- entry points

def dequant(w: Weight, expert: int, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.float32, device="cuda")
    _want("out", out, (torch.float32,), (w.rows, w.cols))
    s = w.struct()
    _require_cuda(out)
    _check("moeq_dequant", _lib().moeq_dequant(ctypes.byref(s), expert, _ptr(out), _stream_ptr()))
    return out


def expert_forward(layer: Layer, x, ids, rw, y=None, ws=None):
    torch = _torch()
    T = _tokens("x", x, layer.hidden)
    _want("x", x, (torch.bfloat16,), (T, layer.hidden))
    _routing_args(layer, T, ids, rw)
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device="cuda")
    _want("y", y, (torch.float32,), (T, layer.hidden))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(x, ids, rw, y, ws)
    _check("moeq_expert_forward", _lib().moeq_expert_forward(ctypes.byref(L), _ptr(x), _ptr(ids), _ptr(rw), T,
                                                              _ptr(y), _ptr(ws), ws.numel(), _stream_ptr()))
    return y


def expert_forward_noalloc(layer: Layer, x, ids, rw, y=None, dev_err=None):
    """moeq_expert_forward_noalloc: the forward with the library's fixed device
    scratch instead of a workspace (nothing allocated by the library; y is
    allocated here only when not given). dev_err: optional int32/uint32 [1] device
    tensor that receives the device error bits by OR."""
    torch = _torch()
    T = _tokens("x", x, layer.hidden)
    _want("x", x, (torch.bfloat16,), (T, layer.hidden))
    _routing_args(layer, T, ids, rw)
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device="cuda")
    _want("y", y, (torch.float32,), (T, layer.hidden))
    if dev_err is not None:
        _want("dev_err", dev_err, (torch.int32, torch.uint32), (1,))
    L = layer.struct()
    _require_cuda(x, ids, rw, y, dev_err)
    _check("moeq_expert_forward_noalloc",
           _lib().moeq_expert_forward_noalloc(ctypes.byref(L), _ptr(x), _ptr(ids), _ptr(rw), T, _ptr(y),
                                              _ptr(dev_err), _stream_ptr()))
    return y


def route(layer: Layer, ids, ws=None):
    T = _tokens("ids", ids, layer.top_k)
    _routing_args(layer, T, ids)
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(ids, ws)
    _check("moeq_route", _lib().moeq_route(ctypes.byref(L), _ptr(ids), T, _ptr(ws), ws.numel(), _stream_ptr()))
    return ws


def gate_up(layer: Layer, x, ids, h=None, ws=None):
    torch = _torch()
    T = _tokens("x", x, layer.hidden)
    _want("x", x, (torch.bfloat16,), (T, layer.hidden))
    _routing_args(layer, T, ids)
    if h is None:
        h = torch.empty((T, layer.top_k, layer.inter), dtype=torch.float32, device="cuda")
    _want("h", h, (torch.float32,), (T, layer.top_k, layer.inter))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(x, ids, h, ws)
    _check("moeq_gate_up", _lib().moeq_gate_up(ctypes.byref(L), _ptr(x), _ptr(ids), T, _ptr(h), _ptr(ws), ws.numel(),
                                                _stream_ptr()))
    return h


def gate_up_timed(layer: Layer, x, ids, start, stop, h=None, ws=None):
    """gate_up with torch.cuda.Event objects (enable_timing=True, already recorded
    once) bracketing the kernel's own execution."""
    torch = _torch()
    T = _tokens("x", x, layer.hidden)
    _want("x", x, (torch.bfloat16,), (T, layer.hidden))
    _routing_args(layer, T, ids)
    if h is None:
        h = torch.empty((T, layer.top_k, layer.inter), dtype=torch.float32, device="cuda")
    _want("h", h, (torch.float32,), (T, layer.top_k, layer.inter))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(x, ids, h, ws)
    _check("moeq_gate_up_timed", _lib().moeq_gate_up_timed(ctypes.byref(L), _ptr(x), _ptr(ids), T, _ptr(h), _ptr(ws),
                                                            ws.numel(), _stream_ptr(),
                                                            ctypes.c_void_p(start.cuda_event),
                                                            ctypes.c_void_p(stop.cuda_event)))
    return h


def down(layer: Layer, h, ids, rw, y=None, ws=None):
    torch = _torch()
    T = _tokens("ids", ids, layer.top_k)
    _routing_args(layer, T, ids, rw)
    _want("h", h, (torch.float32,), (T, layer.top_k, layer.inter))
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device="cuda")
    _want("y", y, (torch.float32,), (T, layer.hidden))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(h, ids, rw, y, ws)
    _check("moeq_down", _lib().moeq_down(ctypes.byref(L), _ptr(h), _ptr(ids), _ptr(rw), T, _ptr(y), _ptr(ws),
                                          ws.numel(), _stream_ptr()))
    return y


def prefill_gate_up(layer: Layer, xq, xs, ids, hq=None, hs=None, h_f32=None, ws=None):
    torch = _torch()
    T = _tokens("xq", xq, layer.hidden)
    P = T * layer.top_k
    _want("xq", xq, (torch.uint8,), (T, layer.hidden))
    _want("xs", xs, (torch.uint8,), (T, layer.hidden // 32))
    _routing_args(layer, T, ids)
    if hq is None:
        hq = torch.empty((P, layer.inter), dtype=torch.uint8, device="cuda")
    if hs is None:
        hs = torch.empty((P, layer.inter // 32), dtype=torch.uint8, device="cuda")
    _want("hq", hq, (torch.uint8,), (P, layer.inter))
    _want("hs", hs, (torch.uint8,), (P, layer.inter // 32))
    if h_f32 is not None:
        _want("h_f32", h_f32, (torch.float32,), (P, layer.inter))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(xq, xs, ids, hq, hs, h_f32, ws)
    _check("moeq_prefill_gate_up", _lib().moeq_prefill_gate_up(ctypes.byref(L), _ptr(xq), _ptr(xs), _ptr(ids), T,
                                                                _ptr(h_f32), _ptr(hq), _ptr(hs), _ptr(ws), ws.numel(),
                                                                _stream_ptr()))
    return hq, hs


def prefill_down(layer: Layer, hq, hs, ids, rw, y=None, ws=None):
    torch = _torch()
    T = _tokens("ids", ids, layer.top_k)
    P = T * layer.top_k
    _routing_args(layer, T, ids, rw)
    _want("hq", hq, (torch.uint8,), (P, layer.inter))
    _want("hs", hs, (torch.uint8,), (P, layer.inter // 32))
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device="cuda")
    _want("y", y, (torch.float32,), (T, layer.hidden))
    if ws is None:
        ws = layer.workspace(T)
    _want_ws(layer, T, ws)
    L = layer.struct()
    _require_cuda(hq, hs, ids, rw, y, ws)
    _check("moeq_prefill_down", _lib().moeq_prefill_down(ctypes.byref(L), _ptr(hq), _ptr(hs), _ptr(ids), _ptr(rw), T,
                                                          _ptr(y), _ptr(ws), ws.numel(), _stream_ptr()))
    return y


def linear(w: Weight, expert: int, x, y=None):
    torch = _torch()
    T = _tokens("x", x, w.cols)
    _want("x", x, (torch.bfloat16,), (T, w.cols))
    if y is None:
        y = torch.empty((T, w.rows), dtype=torch.float32, device="cuda")
    _want("y", y, (torch.float32,), (T, w.rows))
    s = w.struct()
    _require_cuda(x, y)
    _check("moeq_linear", _lib().moeq_linear(ctypes.byref(s), expert, _ptr(x), T, _ptr(y), _stream_ptr()))
    return y


def quantize_mxfp8(x, q=None, e=None):
    """MXFP8 codes [T, K] and e8m0 scales [T, K/32] of a bf16 or fp32 [T, K] tensor."""
    torch = _torch()
    if x is None or len(x.shape) != 2:
        raise ValueError("x: expected a [T, K] tensor")
    T, K = x.shape
    _want("x", x, (torch.bfloat16, torch.float32), (T, K))
    if q is None:
        q = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    if e is None:
        e = torch.empty((T, K // 32), dtype=torch.uint8, device="cuda")
    _want("q", q, (torch.uint8,), (T, K))
    _want("e", e, (torch.uint8,), (T, K // 32))
    _require_cuda(x, q, e)
    if x.dtype == torch.float32:
        rc = _lib().moeq_quantize_mxfp8_f32(_ptr(x), T, K, _ptr(q), _ptr(e), _stream_ptr())
    else:
        rc = _lib().moeq_quantize_mxfp8(_ptr(x), T, K, _ptr(q), _ptr(e), _stream_ptr())
    _check("moeq_quantize_mxfp8", rc)
    return q, e


def check_device_error(ws, clear=True) -> int:
    v = ctypes.c_uint32(0)
    _check("moeq_check_device_error", _lib().moeq_check_device_error(_ptr(ws), _stream_ptr(), ctypes.byref(v),
                                                                      1 if clear else 0))
    return int(v.value)


# ---------------------------------------------------------------- host utilities

def pack_ggml(fmt: int, blocks: np.ndarray, rows: int, cols: int):
    """Contiguous ggml Q2_K / IQ2_XXS blocks -> (data plane, scale plane), host."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    d = np.zeros(plane_bytes(fmt, rows, cols, 0), np.uint8)
    s = np.zeros(plane_bytes(fmt, rows, cols, 1), np.uint8)
    _check("moeq_pack_ggml", _lib().moeq_pack_ggml(fmt, blocks.ctypes.data, rows, cols, d.ctypes.data, s.ctypes.data))
    return d, s


def pack_ggml_device(fmt: int, blocks, rows: int, cols: int, n: int, data, scales):
    _check("moeq_pack_ggml_device", _lib().moeq_pack_ggml_device(fmt, _ptr(blocks), rows, cols, n, _ptr(data),
                                                                  _ptr(scales), _stream_ptr()))


def mxfp4_to_nvfp4(nib: np.ndarray, e8m0: np.ndarray, rows: int, cols: int):
    """Host re-encode; returns (nibbles, e4m3 codes, scale_2) or raises MoeqError."""
    nib = np.ascontiguousarray(nib, dtype=np.uint8)
    e8 = np.ascontiguousarray(e8m0, dtype=np.uint8)
    n2 = np.zeros(rows * cols // 2, np.uint8)
    e4 = np.zeros(rows * cols // 16, np.uint8)
    s2 = ctypes.c_float(0)
    _check("moeq_mxfp4_to_nvfp4", _lib().moeq_mxfp4_to_nvfp4(nib.ctypes.data, e8.ctypes.data, rows, cols,
                                                              n2.ctypes.data, e4.ctypes.data, ctypes.byref(s2)))
    return n2, e4, np.float32(s2.value)


def mxfp8_to_tiled(data, scales, rows: int, cols: int, n: int = 1, tdata=None, tscales=None):
    """Row-major MXFP8 planes of n tensors (device uint8) -> the pre-stored operand
    order (MOEQ_FMT_MXFP8_TILED). Returns (tdata, tscales)."""
    torch = _torch()
    _want("data", data, (torch.uint8,), (n * rows * cols,))
    _want("scales", scales, (torch.uint8,), (n * rows * cols // 32,))
    if tdata is None:
        tdata = torch.empty_like(data)
    if tscales is None:
        tscales = torch.empty_like(scales)
    _want("tdata", tdata, (torch.uint8,), tuple(data.shape))
    _want("tscales", tscales, (torch.uint8,), tuple(scales.shape))
    _require_cuda(data, scales, tdata, tscales)
    _check("moeq_mxfp8_to_tiled", _lib().moeq_mxfp8_to_tiled(_ptr(data), _ptr(scales), rows, cols, n, _ptr(tdata),
                                                              _ptr(tscales), _stream_ptr()))
    return tdata, tscales


def mxfp4_to_nvfp4_device(nib, e8m0, rows: int, cols: int, n: int = 1, nib_out=None):
    """Device MXFP4 -> NVFP4 re-encode of n tensors. Returns (nibbles, e4m3 codes,
    scale_2 [n], status [n]); status 1 marks a tensor that cannot be carried
    exactly (its outputs are not written)."""
    torch = _torch()
    _want("nib", nib, (torch.uint8,), (n * rows * cols // 2,))
    _want("e8m0", e8m0, (torch.uint8,), (n * rows * cols // 32,))
    if nib_out is None:
        nib_out = torch.zeros_like(nib)
    e4 = torch.zeros(n * rows * cols // 16, dtype=torch.uint8, device=nib.device)
    s2 = torch.zeros(n, dtype=torch.float32, device=nib.device)
    st = torch.full((n,), 7, dtype=torch.int32, device=nib.device)
    _require_cuda(nib, e8m0, nib_out)
    _check("moeq_mxfp4_to_nvfp4_device", _lib().moeq_mxfp4_to_nvfp4_device(
        _ptr(nib), _ptr(e8m0), rows, cols, n, _ptr(nib_out), _ptr(e4), _ptr(s2), _ptr(st), _stream_ptr()))
    return nib_out, e4, s2, st


def nvfp4_to_mxfp4_device(nib, e4m3, scale2, rows: int, cols: int, n: int = 1, nib_out=None):
    """Device NVFP4 -> MXFP4 re-encode of n tensors. Returns (nibbles, e8m0 codes,
    status [n])."""
    torch = _torch()
    _want("nib", nib, (torch.uint8,), (n * rows * cols // 2,))
    _want("e4m3", e4m3, (torch.uint8,), (n * rows * cols // 16,))
    _want("scale2", scale2, (torch.float32,), (n,))
    if nib_out is None:
        nib_out = torch.zeros_like(nib)
    e8 = torch.zeros(n * rows * cols // 32, dtype=torch.uint8, device=nib.device)
    st = torch.full((n,), 7, dtype=torch.int32, device=nib.device)
    _require_cuda(nib, e4m3, scale2, nib_out)
    _check("moeq_nvfp4_to_mxfp4_device", _lib().moeq_nvfp4_to_mxfp4_device(
        _ptr(nib), _ptr(e4m3), _ptr(scale2), rows, cols, n, _ptr(nib_out), _ptr(e8), _ptr(st), _stream_ptr()))
    return nib_out, e8, st


def synth_fill(dst, seed: int, stream: int, byte_offset: int, field: int, d_table=None):
    _check("moeq_synth_fill", _lib().moeq_synth_fill(_ptr(dst), dst.numel(), seed, stream, byte_offset, field,
                                                      _ptr(d_table), _stream_ptr()))
