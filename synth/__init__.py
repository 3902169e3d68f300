"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws numbers. It holds none of the arithmetic of the GEMM,
the epilogue or the copy: both sides receive the arrays it returns and nothing
else. Every stream is counter-based (splitmix64 of Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014), so element i
of a tensor depends only on (seed, i) and can be regenerated piecewise.

Workload recipes (none of the source pages names a dataset; all inputs are
synthetic):
  * fp32 operands: i.i.d. uniform on [-1, 1), u = (x >> 40) * 2**-24,
    v = 2u - 1, which is exact in fp32;
  * bf16 operands: N(0, 1) * 0.1 by Box-Muller in fp64, rounded to fp32 and
    then to bf16, both round-to-nearest-even;
  * integer-valued operands for bit-exact parity: uniform on {lo..hi};
  * per-tensor seed = 1000 * workload_id + {A: 1, B: 2, bias: 3, src: 4};
  * mixture-of-experts routing (row counts per expert): each token takes its
    top_k experts by score = uniform noise + 0.3 * a per-expert popularity
    offset (both uniform on [-1, 1)), so experts get uneven loads, as with a
    learned router; see moe_group_rows.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "GOLDEN", "MUL1", "MUL2", "WORKLOADS", "TENSOR_IDS",
    "seed_for", "splitmix64", "uniform_pm1", "normal_bf16_bits",
    "small_int_f32", "small_int_bf16_bits", "f32_to_bf16_bits_rne",
    "bf16_bits_to_f32", "MOE", "moe_group_rows", "ATTENTION",
]

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
MUL1 = np.uint64(0xBF58476D1CE4E5B9)
MUL2 = np.uint64(0x94D049BB133111EB)

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _parallel_chunks(n: int, chunk: int, fn) -> None:
    """Run fn(lo, hi) over [0, n) in chunks on a thread pool (numpy drops the GIL)."""
    spans = [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]
    if len(spans) <= 1:
        for lo, hi in spans:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(lambda s: fn(*s), spans))


TENSOR_IDS = {"A": 1, "B": 2, "bias": 3, "src": 4}

# The five synthetic workloads: shapes and value recipes only.
WORKLOADS = {
    1: dict(kind="gemm", dtype="fp32", M=256, N=256, K=256, dist="uniform",
            tile=(64, 64, 16), stages=2,
            name="fp32 gemm+bias+relu 256x256x256, tile 64x64x16, 2-stage ring"),
    2: dict(kind="copy", dtype="fp32", bytes=1 << 30, dist="uniform",
            tile_bytes=64 * 1024, stages=2,
            name="LDS-staged copy of 1 GiB fp32, 64 KiB tiles, 2-stage ring"),
    3: dict(kind="gemm", dtype="fp32", M=4096, N=4096, K=4096, dist="uniform",
            stages=2, stage_sweep=(2, 3, 4),
            name="fp32 gemm+bias+relu 4096x4096x4096"),
    # 2 stages: a ring of 256x128x32 tiles (a 4-stage ring only holds k = 16)
    4: dict(kind="gemm", dtype="fp32", M=3000, N=5000, K=4100, dist="uniform",
            stages=2,
            name="fp32 gemm+bias+relu ragged 3000x5000x4100"),
    5: dict(kind="gemm", dtype="bf16", M=8192, N=8192, K=8192, dist="normal0.1",
            stages=4,
            name="bf16 gemm+bias+relu 8192x8192x8192, fp32 accumulate and output"),
}


# The expert layer of a mixture-of-experts model for the grouped GEMM: 8
# experts, 4096 tokens routed to their top 2, model width K = 4096, expert
# width N = 14336 (the shape of a widely used open 8-expert model; the pages
# name none), bf16 operands as workload 5, a 2-stage ring (its default tile
# is then 256x256x64; on MI355X the fastest depth for this layer: 802 TFLOP/s
# against 725 at S = 3 with 256x128x64 and 754 at S = 4 with 256x256x32, one
# box). Seeds use workload id 6.
MOE = dict(kind="grouped_gemm", dtype="bf16", experts=8, tokens=4096, top_k=2, K=4096, N=14336,
           dist="normal0.1", stages=2, id=6,
           name="bf16 grouped gemm+bias+relu, 8 experts, 4096 tokens top-2, K 4096, N 14336")


# Attention forward, the second consumer type: batch 4, 32 heads, 4096
# queries and keys, head dimension 128 (a common prefill shape; the pages name
# none), Q, K, V i.i.d. N(0, 1) rounded to bf16, scale 1 / sqrt(D), 3-stage
# ring; timed without and with the causal mask. Seeds use workload id 7.
ATTENTION = dict(kind="attention", dtype="bf16", batch=4, heads=32, S=4096, D=128, dist="normal1", stages=3, id=7,
                 name="bf16 attention forward, batch 4, 32 heads, 4096 queries and keys, head dim 128")


def moe_group_rows(seed: int, tokens: int, experts: int, top_k: int) -> np.ndarray:
    """Rows per expert (int64, length `experts`, summing to tokens * top_k):
    every token picks the top_k experts by its seeded score."""
    if not 1 <= top_k <= experts:
        raise ValueError("top_k must be in 1..experts")
    popularity = uniform_pm1(seed, experts).astype(np.float64)
    noise = uniform_pm1(seed + 1, tokens * experts).astype(np.float64).reshape(tokens, experts)
    score = noise + 0.3 * popularity
    top = np.argsort(-score, axis=1, kind="stable")[:, :top_k]
    return np.bincount(top.ravel(), minlength=experts).astype(np.int64)


def seed_for(workload_id: int, tensor: str) -> int:
    """Per-tensor seed: 1000 * workload id + a fixed tensor index."""
    return 1000 * int(workload_id) + TENSOR_IDS[tensor]


def _mix(z: np.ndarray) -> np.ndarray:
    # splitmix64 output function, in place on a uint64 array
    z ^= z >> np.uint64(30)
    z *= MUL1
    z ^= z >> np.uint64(27)
    z *= MUL2
    z ^= z >> np.uint64(31)
    return z


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of the splitmix64 sequence seeded with `seed`.

    Output i is mix(seed + (i + 1) * GOLDEN) modulo 2**64.
    """
    out = np.empty(int(n), dtype=np.uint64)
    s = np.uint64(int(seed) & 0xFFFFFFFFFFFFFFFF)

    def work(lo, hi):
        with np.errstate(over="ignore"):
            z = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
            z *= GOLDEN
            z += s
            out[lo:hi] = _mix(z)

    _parallel_chunks(int(n), _CHUNK, work)
    return out


def uniform_pm1(seed: int, n: int) -> np.ndarray:
    """fp32 i.i.d. uniform on [-1, 1): 2 * ((x >> 40) * 2**-24) - 1, exact."""
    out = np.empty(int(n), dtype=np.float32)

    def work(lo, hi):
        x = splitmix64(seed, hi - lo, start=lo)
        j = (x >> np.uint64(40)).astype(np.int64) - (1 << 23)  # in [-2^23, 2^23)
        out[lo:hi] = j.astype(np.float32) * np.float32(2.0 ** -23)

    _parallel_chunks(int(n), _CHUNK, work)
    return out


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits.

    NaN is kept quiet; the inputs drawn here are always finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (b >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed: int, n: int, scale: float = 0.1) -> np.ndarray:
    """N(0,1)*scale by Box-Muller on outputs (2i, 2i+1), rounded fp64->fp32->bf16."""
    out = np.empty(int(n), dtype=np.uint16)

    def work(lo, hi):
        x = splitmix64(seed, 2 * (hi - lo), start=2 * lo)
        u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
        u2 = (x[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)          # [0, 1)
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * scale
        out[lo:hi] = f32_to_bf16_bits_rne(z.astype(np.float32))

    _parallel_chunks(int(n), _CHUNK // 2, work)
    return out


def small_int_f32(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integer-valued fp32, uniform on {lo, ..., hi}: lo + ((x >> 32) mod (hi - lo + 1))."""
    out = np.empty(int(n), dtype=np.float32)
    span = np.uint64(hi - lo + 1)

    def work(a, b):
        x = splitmix64(seed, b - a, start=a)
        out[a:b] = ((x >> np.uint64(32)) % span).astype(np.int64).astype(np.float32) + np.float32(lo)

    _parallel_chunks(int(n), _CHUNK, work)
    return out


def small_int_bf16_bits(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integer-valued bf16 bits, uniform on {lo, ..., hi} (|values| <= 256 are exact)."""
    out = np.empty(int(n), dtype=np.uint16)

    def work(a, b):
        x = splitmix64(seed, b - a, start=a)
        v = ((x >> np.uint64(32)) % np.uint64(hi - lo + 1)).astype(np.int64).astype(np.float32) + np.float32(lo)
        out[a:b] = f32_to_bf16_bits_rne(v)

    _parallel_chunks(int(n), _CHUNK, work)
    return out
