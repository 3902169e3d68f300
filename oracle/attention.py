"""Oracle of attention, the second consumer type the pages name.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it.

The aicassindra.com page on GPU warp specialization names attention, next to
GEMM, as a kernel built on producer and consumer warps, and describes nothing
more of it. This module writes out scaled dot-product attention from its
definition, per batch and head, in fp64:
    S = scale * Q K^T,  P = softmax over keys of S (each query row),  O = P V.
With `causal`, query i sees key j only if j <= i + (Skv - Sq): the diagonal
meets the last query and the last key, so Sq == Skv gives j <= i. A query
row with no visible key has no softmax; its output is defined as zeros.
Operands are float32 arrays or uint16 arrays of bf16 bit patterns, widened
exactly to fp64; a matrix product of fp64 arrays is the only library step.
"""
from __future__ import annotations

import numpy as np


def widen(x) -> np.ndarray:
    """float32, or bf16 bit patterns (uint16), to float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    raise TypeError("operands are float32 or uint16 bf16 bit patterns, got %s" % x.dtype)


def visible(Sq: int, Skv: int, causal: bool) -> np.ndarray:
    """Boolean (Sq, Skv): may query i attend to key j."""
    if not causal:
        return np.ones((Sq, Skv), dtype=bool)
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    return j <= i + (Skv - Sq)


def attention(Q, K, V, scale: float, causal: bool = False) -> np.ndarray:
    """fp64 O (batch, heads, Sq, D) for Q (batch, heads, Sq, D), K and V (batch, heads, Skv, D)."""
    q, k, v = widen(Q), widen(K), widen(V)
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("Q must be (B, H, Sq, D) and K, V (B, H, Skv, D): got %s, %s, %s" % (q.shape, k.shape, v.shape))
    Bn, H, Sq, D = q.shape
    Skv = k.shape[2]
    vis = visible(Sq, Skv, causal)
    O = np.zeros((Bn, H, Sq, D), dtype=np.float64)
    if Sq == 0 or Skv == 0:
        return O
    rows = vis.any(axis=1)
    for b in range(Bn):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = np.where(vis, s, -np.inf)
            m = np.max(s[rows], axis=1, keepdims=True)
            p = np.exp(s[rows] - m)
            p /= np.sum(p, axis=1, keepdims=True)
            O[b, h, rows] = p @ v[b, h]
    return O


def attention_rows(Q, K, V, scale: float, causal: bool, b: int, h: int, rows) -> np.ndarray:
    """fp64 O[b, h, rows] only (the same definition, for sampled checks of large inputs)."""
    rows = np.asarray(rows, dtype=np.int64)
    q, k, v = widen(np.asarray(Q)[b, h, rows]), widen(np.asarray(K)[b, h]), widen(np.asarray(V)[b, h])
    Sq, Skv = np.asarray(Q).shape[2], k.shape[0]
    vis = visible(Sq, Skv, causal)[rows]
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    out = np.zeros((rows.size, k.shape[1]), dtype=np.float64)
    live = vis.any(axis=1)
    if np.any(live):
        m = np.max(s[live], axis=1, keepdims=True)
        p = np.exp(s[live] - m)
        p /= np.sum(p, axis=1, keepdims=True)
        out[live] = p @ v
    return out
