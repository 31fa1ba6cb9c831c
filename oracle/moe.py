"""Routed-MoE expert projection, dense block-quantized linear, and the W4A8
prefill chain, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The routed layer (DeepSeek-V4-Flash W4A16-FP8 card, "Architecture & precision",
base-model table: 256 routed experts per layer, top-6, hidden size 4096; REAP
K180 Mixed NVFP4 card, "Why this mix?": each expert is a gate and an up
projection followed by a down projection). For token t routed to experts
e_k with weights w_k, k = 0..top_k-1:

    g = G_e x_t,  u = U_e x_t,  h_k = silu(g) * u,  y_t = sum_k w_k (D_e h_k)

Readings where the pages are silent (listed in the design notes): SwiGLU is
silu(g) * u with silu(z) = z / (1 + e^-z), with no clamp and no extra factor; route
weights are applied after the down projection, as given (no routed scaling
factor); duplicate expert ids in one token are computed as given.

``weight(proj, e)`` supplies the exact decoded matrix of projection proj
(0 gate [I, H], 1 up [I, H], 2 down [H, I]) of expert e.
"""
from __future__ import annotations

from typing import Callable

import numpy as np

from .codecs import bf16_to_f64
from . import mxfp8

GATE, UP, DOWN = 0, 1, 2


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    return silu(g) * u


class CachedWeights:
    """Decode-on-demand cache around a ``(proj, e) -> float64 matrix`` function."""

    def __init__(self, fn: Callable[[int, int], np.ndarray]):
        self.fn = fn
        self.cache = {}

    def __call__(self, proj: int, e: int) -> np.ndarray:
        key = (proj, int(e))
        if key not in self.cache:
            self.cache[key] = self.fn(proj, int(e))
        return self.cache[key]


def moe_layer(x_bits: np.ndarray, ids: np.ndarray, rw: np.ndarray, weight) -> tuple:
    """x_bits: bf16 bit patterns [T, H]; ids int [T, K]; rw fp32 [T, K].
    Returns (y [T, H], h [T, K, I]) in float64."""
    X = bf16_to_f64(x_bits)
    return moe_layer_f64(X, ids, rw, weight)


def moe_layer_f64(X: np.ndarray, ids: np.ndarray, rw: np.ndarray, weight) -> tuple:
    T, K = ids.shape
    I = weight(GATE, ids[0, 0]).shape[0] if T else 0
    H = X.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    h = np.zeros((T, K, I), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            g = weight(GATE, e) @ X[t]
            u = weight(UP, e) @ X[t]
            h[t, k] = swiglu(g, u)
            y[t] += np.float64(rw[t, k]) * (weight(DOWN, e) @ h[t, k])
    return y, h


def linear(W: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """Dense linear y_t = W x_t, W the exact decoded [N, K] matrix."""
    return bf16_to_f64(x_bits) @ np.asarray(W, dtype=np.float64).T


# ----------------------------------------------------------------------------
# W4A8 prefill (DeepSeekv4 Flash for 1x Spark forum thread, second post:
# experts grouped by token, fp4 weights times E4M3 activations with a dynamic
# activation scale). Each stage is checked on its own, given identical inputs.

def prefill_h(xq: np.ndarray, xs: np.ndarray, ids: np.ndarray, weight) -> np.ndarray:
    """h [T, K, I] from MXFP8 activations (codes xq [T, H], e8m0 xs [T, H/32])."""
    Xh = mxfp8.dequantize(xq, xs)
    T, K = ids.shape
    I = weight(GATE, ids[0, 0]).shape[0]
    h = np.zeros((T, K, I), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            h[t, k] = swiglu(weight(GATE, e) @ Xh[t], weight(UP, e) @ Xh[t])
    return h


def prefill_y(hq: np.ndarray, hs: np.ndarray, ids: np.ndarray, rw: np.ndarray, weight) -> np.ndarray:
    """y [T, H] from MXFP8-quantised h (codes hq [T*K, I], e8m0 hs [T*K, I/32],
    row t*K + k belongs to token t, slot k)."""
    Hh = mxfp8.dequantize(hq, hs)
    T, K = ids.shape
    H = weight(DOWN, ids[0, 0]).shape[0]
    y = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            y[t] += np.float64(rw[t, k]) * (weight(DOWN, e) @ Hh[t * K + k])
    return y


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max_i |y_i - ref_i| / max(|ref_i|, rms(ref)): elementwise relative error
    floored at the reference's RMS, so outputs near zero do not dominate."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - ref) / den))
