"""Oracle of the grouped (mixture-of-experts) GEMM + bias + ReLU.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it.

The pwwt.cn article on intra-kernel pipelining meets the load-barrier-compute
loop (section 1.1) while tuning the custom operators of a mixture-of-experts
model. Its operator (section 4.1, C = relu(A B + bias)) appears there once
per expert. The token rows routed to expert e are sorted by expert, with
group_rows[e] of them per expert. They are multiplied by that expert's weights
B[e], offset by its biases bias[e], and rectified. The pages say nothing more
about that layer; this module writes out exactly this reading, one expert's
row slice at a time through the fp64 GEMM oracle passed in as `gemm`.
"""
from __future__ import annotations

import numpy as np


def _shapes(A, B, bias, group_rows):
    rows = [int(r) for r in group_rows]
    if any(r < 0 for r in rows):
        raise ValueError("row counts must be >= 0")
    if A.ndim != 2 or B.ndim != 3 or bias.ndim != 2:
        raise ValueError("A must be rows x K, B experts x K x N, bias experts x N")
    G, K, N = B.shape
    if len(rows) != G or bias.shape != (G, N) or A.shape != (sum(rows), K):
        raise ValueError("shape mismatch: A %s, B %s, bias %s, rows %s" % (A.shape, B.shape, bias.shape, rows))
    return rows, G, K, N


def grouped_gemm_bias_relu(A, B, bias, group_rows, gemm) -> np.ndarray:
    """fp64 C with C[rows of e] = relu(A[rows of e] @ B[e] + bias[e]) for every expert e."""
    A, B, bias = np.asarray(A), np.asarray(B), np.asarray(bias)
    rows, G, K, N = _shapes(A, B, bias, group_rows)
    C = np.zeros((A.shape[0], N), dtype=np.float64)
    start = 0
    for e in range(G):
        stop = start + rows[e]
        if stop > start:
            C[start:stop] = gemm(A[start:stop], B[e], bias[e])
        start = stop
    return C


def grouped_gemm_bias_relu_rows(A, B, bias, group_rows, wanted, gemm_rows) -> np.ndarray:
    """Rows `wanted` of the grouped result, each from its own expert's GEMM
    (gemm_rows(A_slice, B_e, bias_e, local_rows) returns those rows)."""
    A, B, bias = np.asarray(A), np.asarray(B), np.asarray(bias)
    rows, G, K, N = _shapes(A, B, bias, group_rows)
    wanted = np.asarray(wanted, dtype=np.int64)
    out = np.empty((wanted.size, N), dtype=np.float64)
    start = 0
    for e in range(G):
        stop = start + rows[e]
        pick = np.nonzero((wanted >= start) & (wanted < stop))[0]
        if pick.size:
            out[pick] = gemm_rows(A[start:stop], B[e], bias[e], wanted[pick] - start)
        start = stop
    if np.any((wanted < 0) | (wanted >= start)):
        raise ValueError("row index out of range")
    return out
