"""Pins of the grouped (mixture-of-experts) oracle against what does not use it.

- brute force: integer inputs, a pure-Python triple loop per element whose row -> expert map is built by listing
  each expert's rows in turn (not by slicing);
- closed forms: zero weights give relu(bias of the row's expert); scaled identity weights give
  relu((e + 1) * A_row + bias_e);
- one expert is the plain GEMM oracle;
- permuting the experts (their row blocks, weights and biases) permutes the output blocks.
Every mutant below, a plausible mistake planted in a copy of oracle/grouped.py, fails one of them.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle
import synth

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "grouped.py")

ROW_PATTERNS = [[2, 0, 3, 1], [0, 4], [3, 0], [0, 0, 2], [1], [5, 2, 0, 0, 1, 3]]


def _ints(seed, shape, lo, hi):
    return synth.small_int_f32(seed, int(np.prod(shape)), lo, hi).reshape(shape)


def _brute(A, B, bias, rows):
    owner = []
    for e, n in enumerate(rows):
        owner.extend([e] * n)
    M, K = A.shape
    N = B.shape[2]
    C = np.zeros((M, N))
    for m in range(M):
        e = owner[m]
        for n in range(N):
            s = float(bias[e, n])
            for k in range(K):
                s += float(A[m, k]) * float(B[e, k, n])
            C[m, n] = s if s > 0 else 0.0
    return C


def _case(seed, rows, K=3, N=4):
    G = len(rows)
    A = _ints(seed, (sum(rows), K), -3, 3)
    B = _ints(seed + 1, (G, K, N), -3, 3)
    bias = _ints(seed + 2, (G, N), -8, 8)
    return A, B, bias


def run_pins(full, rows_fn):
    """Names of the pins that fail for the pair (full, rows_fn)."""
    failed = []
    for i, rows in enumerate(ROW_PATTERNS):
        A, B, bias = _case(100 + 7 * i, rows)
        ref = _brute(A, B, bias, rows)
        try:
            if not np.array_equal(full(A, B, bias, rows), ref):
                failed.append("brute_force_%d" % i)
            wanted = np.arange(sum(rows))[::-1]
            if wanted.size and not np.array_equal(rows_fn(A, B, bias, rows, wanted), ref[wanted]):
                failed.append("brute_force_rows_%d" % i)
        except (ValueError, IndexError):
            failed.append("brute_force_raises_%d" % i)
    # closed forms
    rows = [3, 0, 2, 4]
    G, K, N = len(rows), 5, 5
    A = synth.uniform_pm1(11, sum(rows) * K).reshape(sum(rows), K)
    bias = synth.uniform_pm1(12, G * N).reshape(G, N)
    owner = np.repeat(np.arange(G), rows)
    try:
        C0 = full(A, np.zeros((G, K, N), np.float32), bias, rows)
        if not np.array_equal(C0, np.maximum(bias[owner].astype(np.float64), 0.0)):
            failed.append("zero_weights")
        eye = np.stack([np.eye(K, dtype=np.float32) * (e + 1) for e in range(G)])
        want = np.maximum((owner[:, None] + 1) * A.astype(np.float64) + bias[owner].astype(np.float64), 0.0)
        if not np.allclose(full(A, eye, bias, rows), want, rtol=0, atol=1e-12):
            failed.append("scaled_identity")
    except (ValueError, IndexError):
        failed.append("closed_form_raises")
    # one expert
    A1, B1, b1 = _case(300, [6], K=7, N=3)
    if not np.array_equal(full(A1, B1, b1, [6]), oracle.gemm_bias_relu(A1, B1[0], b1[0])):
        failed.append("single_expert")
    # permutation of experts
    rows = [2, 5, 0, 3]
    G, K, N = len(rows), 6, 4
    A = synth.uniform_pm1(21, sum(rows) * K).reshape(sum(rows), K)
    B = synth.uniform_pm1(22, G * K * N).reshape(G, K, N)
    bias = synth.uniform_pm1(23, G * N).reshape(G, N)
    perm = [2, 0, 3, 1]
    starts = np.concatenate([[0], np.cumsum(rows)])
    blocks = [A[starts[e]:starts[e + 1]] for e in range(G)]
    try:
        C = full(A, B, bias, rows)
        Cp = full(np.concatenate([blocks[e] for e in perm]), B[perm], bias[perm], [rows[e] for e in perm])
        if not np.array_equal(Cp, np.concatenate([C[starts[e]:starts[e + 1]] for e in perm])):
            failed.append("permutation")
    except (ValueError, IndexError):
        failed.append("permutation_raises")
    return failed


def _reference_pair():
    return (lambda A, B, b, r: oracle.grouped_gemm_bias_relu(A, B, b, r, threads=2),
            lambda A, B, b, r, w: oracle.grouped_gemm_bias_relu_rows(A, B, b, r, w, threads=2))


def test_oracle_passes_every_pin():
    assert run_pins(*_reference_pair()) == []


MUTANTS = {
    "next_experts_weights": ("C[start:stop] = gemm(A[start:stop], B[e], bias[e])",
                             "C[start:stop] = gemm(A[start:stop], B[(e + 1) % G], bias[e])"),
    "first_experts_bias": ("C[start:stop] = gemm(A[start:stop], B[e], bias[e])",
                           "C[start:stop] = gemm(A[start:stop], B[e], bias[0])"),
    "offset_not_advanced": ("            C[start:stop] = gemm(A[start:stop], B[e], bias[e])\n        start = stop",
                            "            C[start:stop] = gemm(A[start:stop], B[e], bias[e])\n        start = 0"),
    "experts_reversed": ("    C = np.zeros((A.shape[0], N), dtype=np.float64)\n    start = 0\n    for e in range(G):",
                         "    C = np.zeros((A.shape[0], N), dtype=np.float64)\n    start = 0\n    for e in reversed(range(G)):"),
    "rows_from_the_top": ("C[start:stop] = gemm(A[start:stop], B[e], bias[e])",
                          "C[start:stop] = gemm(A[:stop - start], B[e], bias[e])"),
    "rows_fn_global_index": ("gemm_rows(A[start:stop], B[e], bias[e], wanted[pick] - start)",
                             "gemm_rows(A[start:stop], B[e], bias[e], np.minimum(wanted[pick], stop - start - 1))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site for %s no longer in grouped.py" % name
    path = tmp_path / ("grouped_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("grouped_mutant_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    full = lambda A, B, b, r: mod.grouped_gemm_bias_relu(A, B, b, r, lambda a, bb, c: oracle.gemm_bias_relu(a, bb, c, 2))
    rows_fn = lambda A, B, b, r, w: mod.grouped_gemm_bias_relu_rows(
        A, B, b, r, w, lambda a, bb, c, rr: oracle.gemm_bias_relu_rows(a, bb, c, rr, 2))
    assert run_pins(full, rows_fn), "mutant %s passed every pin" % name


def test_bf16_bits_per_expert():
    rows = [4, 0, 3]
    G, K, N = 3, 16, 8
    A = synth.normal_bf16_bits(31, sum(rows) * K).reshape(sum(rows), K)
    B = synth.normal_bf16_bits(32, G * K * N).reshape(G, K, N)
    bias = synth.normal_bf16_bits(33, G * N).reshape(G, N)
    C = oracle.grouped_gemm_bias_relu(A, B, bias, rows)
    assert np.array_equal(C[:4], oracle.gemm_bias_relu(A[:4], B[0], bias[0]))
    assert np.array_equal(C[4:], oracle.gemm_bias_relu(A[4:], B[2], bias[2]))


def test_argument_errors():
    A = np.zeros((3, 2), np.float32)
    B = np.zeros((2, 2, 4), np.float32)
    b = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bias_relu(A, B, b, [1, 1])  # rows do not add up to A's
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bias_relu(A, B, b, [4, -1])
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bias_relu(A, B[0], b, [1, 2])
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bias_relu_rows(A, B, b, [1, 2], [3])
