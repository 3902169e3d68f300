"""CPU oracle: plain, slow, obviously correct references for the hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library never
loads it, and the two share no code: the only thing both sides use is the
seeded input module `synth`, which holds no arithmetic of the method.

Contents
  * gemm_bias_relu / gemm_bias_relu_rows / gemm_bias_relu_at: fp64 reference
    of C = relu(A @ B + bias) (oracle.c, compiled by oracle/build.py);
    the operator is the SGEMM-with-epilogue of the pwwt.cn article on
    intra-kernel pipelining, section 4.1.
  * copy / first_mismatch: the staged copy's reference (dst equals src), from
    the double-buffered load/store example of "Producer-Consumer Warp
    Specialization for TMA Operations".
  * ringsim: a simulator of the full/empty ring protocol (oracle/ringsim.py).
  * grouped_gemm_bias_relu / grouped_gemm_bias_relu_rows: the same operator
    once per expert of a mixture-of-experts layer (oracle/grouped.py).
  * attention.attention / attention.attention_rows: scaled dot-product
    attention in fp64, the second consumer type (oracle/attention.py).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def host_threads() -> int:
    """Threads the oracle uses by default: the cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _dtype_code(A: np.ndarray) -> int:
    if A.dtype == np.float32:
        return 0
    if A.dtype == np.uint16:
        return 1
    raise TypeError("oracle operands are float32 arrays or uint16 bf16 bit patterns, got %s" % A.dtype)


def _check(A, B, bias):
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    bias = np.ascontiguousarray(bias)
    code = _dtype_code(A)
    if B.dtype != A.dtype or bias.dtype != A.dtype:
        raise TypeError("A, B and bias must share one dtype")
    if A.ndim != 2 or B.ndim != 2 or bias.ndim != 1:
        raise ValueError("A must be MxK, B KxN, bias N")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or bias.shape[0] != N:
        raise ValueError("shape mismatch: A %s, B %s, bias %s" % (A.shape, B.shape, bias.shape))
    return A, B, bias, code, M, N, K


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleLib:
    """The compiled oracle (liboracle.so, or another build of oracle.c)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_gemm_bias_relu.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.c_int]
        lib.oracle_gemm_bias_relu.restype = ctypes.c_int
        lib.oracle_gemm_bias_relu_rows.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64,
                                                   _vp, ctypes.c_int]
        lib.oracle_gemm_bias_relu_rows.restype = ctypes.c_int
        lib.oracle_gemm_bias_relu_at.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                                 _i64, _vp, ctypes.c_int]
        lib.oracle_gemm_bias_relu_at.restype = ctypes.c_int
        lib.oracle_copy.argtypes = [_vp, _vp, ctypes.c_uint64, ctypes.c_int]
        lib.oracle_copy.restype = ctypes.c_int
        lib.oracle_first_mismatch.argtypes = [_vp, _vp, ctypes.c_uint64]
        lib.oracle_first_mismatch.restype = ctypes.c_int64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.path = path
        self._lib = lib

    def gemm_bias_relu(self, A, B, bias, threads: int | None = None) -> np.ndarray:
        """fp64 C = relu(A @ B + bias) with bias per column; A MxK, B KxN."""
        A, B, bias, code, M, N, K = _check(A, B, bias)
        C = np.empty((M, N), dtype=np.float64)
        rc = self._lib.oracle_gemm_bias_relu(code, M, N, K, _ptr(A), _ptr(B), _ptr(bias), _ptr(C),
                                             threads or host_threads())
        if rc != 0:
            raise RuntimeError("oracle_gemm_bias_relu returned %d" % rc)
        return C

    def gemm_bias_relu_rows(self, A, B, bias, rows, threads: int | None = None) -> np.ndarray:
        """Rows `rows` of the fp64 result, shape (len(rows), N)."""
        A, B, bias, code, M, N, K = _check(A, B, bias)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.shape[0], N), dtype=np.float64)
        rc = self._lib.oracle_gemm_bias_relu_rows(code, M, N, K, _ptr(A), _ptr(B), _ptr(bias), _ptr(rows),
                                                  rows.shape[0], _ptr(out), threads or host_threads())
        if rc != 0:
            raise RuntimeError("oracle_gemm_bias_relu_rows returned %d" % rc)
        return out

    def gemm_bias_relu_at(self, A, B, bias, ms, ns, threads: int | None = None) -> np.ndarray:
        """Elements C[ms[i], ns[i]] of the fp64 result, each as its own dot product."""
        A, B, bias, code, M, N, K = _check(A, B, bias)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        if ms.shape != ns.shape:
            raise ValueError("ms and ns must have the same length")
        out = np.empty(ms.shape[0], dtype=np.float64)
        rc = self._lib.oracle_gemm_bias_relu_at(code, M, N, K, _ptr(A), _ptr(B), _ptr(bias), _ptr(ms),
                                                _ptr(ns), ms.shape[0], _ptr(out), threads or host_threads())
        if rc != 0:
            raise RuntimeError("oracle_gemm_bias_relu_at returned %d" % rc)
        return out

    def copy(self, src: np.ndarray, threads: int | None = None) -> np.ndarray:
        """The staged copy's expected result: a byte-for-byte copy of src."""
        src = np.ascontiguousarray(src)
        flat = src.view(np.uint8).reshape(-1)
        dst = np.empty_like(flat)
        self._lib.oracle_copy(_ptr(flat), _ptr(dst), flat.nbytes, threads or host_threads())
        return dst.view(src.dtype).reshape(src.shape)

    def first_mismatch(self, a: np.ndarray, b: np.ndarray) -> int:
        """Index of the first differing byte, or -1 when a and b are byte-identical."""
        a = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
        b = np.ascontiguousarray(b).view(np.uint8).reshape(-1)
        if a.nbytes != b.nbytes:
            return min(a.nbytes, b.nbytes)
        return int(self._lib.oracle_first_mismatch(_ptr(a), _ptr(b), a.nbytes))

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())


_default = None


def library_path() -> str:
    return _LIB_PATH


def default() -> OracleLib:
    """The oracle built from oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _default = OracleLib(_LIB_PATH)
    return _default


def gemm_bias_relu(A, B, bias, threads: int | None = None) -> np.ndarray:
    return default().gemm_bias_relu(A, B, bias, threads)


def gemm_bias_relu_rows(A, B, bias, rows, threads: int | None = None) -> np.ndarray:
    return default().gemm_bias_relu_rows(A, B, bias, rows, threads)


def gemm_bias_relu_at(A, B, bias, ms, ns, threads: int | None = None) -> np.ndarray:
    return default().gemm_bias_relu_at(A, B, bias, ms, ns, threads)


def grouped_gemm_bias_relu(A, B, bias, group_rows, threads: int | None = None) -> np.ndarray:
    from . import grouped
    return grouped.grouped_gemm_bias_relu(A, B, bias, group_rows,
                                          lambda a, b, c: gemm_bias_relu(a, b, c, threads))


def grouped_gemm_bias_relu_rows(A, B, bias, group_rows, rows, threads: int | None = None) -> np.ndarray:
    from . import grouped
    return grouped.grouped_gemm_bias_relu_rows(A, B, bias, group_rows, rows,
                                               lambda a, b, c, r: gemm_bias_relu_rows(a, b, c, r, threads))


def copy(src: np.ndarray, threads: int | None = None) -> np.ndarray:
    return default().copy(src, threads)


def first_mismatch(a: np.ndarray, b: np.ndarray) -> int:
    return default().first_mismatch(a, b)


def compare(C_gpu: np.ndarray, C_ref: np.ndarray) -> dict:
    """max_abs and rel_fro of C_gpu against the fp64 reference, in fp64.

    rel_fro = ||C_gpu - C_ref||_F / ||C_ref||_F (0 reference norm: max_abs
    decides alone); any non-finite value in C_gpu is reported.
    """
    g = np.asarray(C_gpu, dtype=np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    finite = bool(np.all(np.isfinite(g)))
    d = g - r
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nr = float(np.sqrt(np.sum(r * r))) if r.size else 0.0
    rel = float(np.sqrt(np.sum(d * d)) / nr) if nr > 0 else 0.0
    return {"max_abs": max_abs, "rel_fro": rel, "finite": finite}


# Parity tolerances for floating point results (fp32 and bf16 operands).
TOL = {"fp32": (1e-3, 1e-5), "bf16": (2e-2, 5e-3)}


def within_tolerance(stats: dict, dtype: str) -> bool:
    max_abs, rel = TOL[dtype]
    return stats["finite"] and stats["max_abs"] <= max_abs and stats["rel_fro"] <= rel
