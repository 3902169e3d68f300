"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each pin takes a `compute(A, B, bias) -> fp64 C` callable, so the same pins
run against the full oracle, its row and element variants, and (in the
mutation tests) against deliberately broken builds of oracle.c. A pin raises
AssertionError when the oracle disagrees with what it is pinned to:

  * exact rational arithmetic (fractions.Fraction) on small seeded cases,
    with the fp64 error bound of a K-term sum;
  * closed forms: identity, zero and all-ones operands, K = 0;
  * integer-valued inputs, where the exact answer is an integer computed by
    Python integers or numpy int64 matmul;
  * the reflection identity relu(x) - relu(-x) = x;
  * a hand-derived worked example (tests/golden/gemm_worked_example.json);
  * the sign of zero after the ReLU and the ascending k order of the sum.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _relu_exact(x: Fraction) -> Fraction:
    return x if x > 0 else Fraction(0)


def exact_gemm_bias_relu(A, B, bias):
    """relu(A @ B + bias) in exact rationals (pure Python loops, small sizes)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    M, K = A.shape
    N = B.shape[1]
    out, mag = [], []
    for m in range(M):
        row, mrow = [], []
        for n in range(N):
            s = Fraction(0)
            a_abs = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[m, k])) * Fraction(float(B[k, n]))
                s += p
                a_abs += abs(p)
            s += Fraction(float(bias[n]))
            row.append(_relu_exact(s))
            mrow.append(a_abs + abs(Fraction(float(bias[n]))))
        out.append(row)
        mag.append(mrow)
    return out, mag


def _uniform(seed, shape):
    n = int(np.prod(shape)) if len(shape) else 1
    return synth.uniform_pm1(seed, n).reshape(shape)


def pin_fraction_bruteforce(compute, dtype: str = "fp32"):
    """Oracle within the fp64 summation bound of the exact rational result."""
    shapes = [(4, 4, 4)] * 5 + [(1, 1, 1), (3, 5, 7), (5, 3, 0), (2, 7, 3), (6, 2, 9)]
    for i, (M, N, K) in enumerate(shapes):
        seed = 9000 + 10 * i
        if dtype == "fp32":
            A = _uniform(seed + 1, (M, K))
            B = _uniform(seed + 2, (K, N))
            bias = _uniform(seed + 3, (N,))
            Af, Bf, bf = A, B, bias
        else:
            A = synth.normal_bf16_bits(seed + 1, M * K, 1.0).reshape(M, K)
            B = synth.normal_bf16_bits(seed + 2, K * N, 1.0).reshape(K, N)
            bias = synth.normal_bf16_bits(seed + 3, N, 1.0)
            Af, Bf, bf = (synth.bf16_bits_to_f32(x) for x in (A, B, bias))
        C = compute(A, B, bias)
        assert C.shape == (M, N), "shape %s for %s" % (C.shape, (M, N, K))
        exact, mag = exact_gemm_bias_relu(Af, Bf, bf)
        for m in range(M):
            for n in range(N):
                bound = float(mag[m][n]) * (K + 1) * 2.0 ** -52
                err = abs(Fraction(float(C[m, n])) - exact[m][n])
                assert err <= Fraction(bound), (
                    "case %d %s at (%d,%d): oracle %r exact %r err %g > bound %g"
                    % (i, (M, N, K), m, n, float(C[m, n]), float(exact[m][n]), float(err), bound))


def pin_closed_forms(compute):
    """Identity, zero, all-ones operands and K = 0 give exactly known results."""
    rng_seed = 777
    # A = I (M = K): C = relu(B + bias)
    K, N = 6, 5
    B = _uniform(rng_seed + 1, (K, N))
    bias = _uniform(rng_seed + 2, (N,))
    want = np.maximum(B.astype(np.float64) + bias.astype(np.float64), 0.0)
    got = compute(np.eye(K, dtype=np.float32), B, bias)
    assert np.array_equal(got, want), "A = I"
    # B = I (K = N): C = relu(A + bias)
    M, K = 4, 5
    A = _uniform(rng_seed + 3, (M, K))
    bias = _uniform(rng_seed + 4, (K,))
    want = np.maximum(A.astype(np.float64) + bias.astype(np.float64)[None, :], 0.0)
    got = compute(A, np.eye(K, dtype=np.float32), bias)
    assert np.array_equal(got, want), "B = I"
    # A = 0 or B = 0: every row is relu(bias)
    M, K, N = 3, 7, 4
    bias = _uniform(rng_seed + 5, (N,))
    want = np.tile(np.maximum(bias.astype(np.float64), 0.0), (M, 1))
    got = compute(np.zeros((M, K), np.float32), _uniform(rng_seed + 6, (K, N)), bias)
    assert np.array_equal(got, want), "A = 0"
    got = compute(_uniform(rng_seed + 7, (M, K)), np.zeros((K, N), np.float32), bias)
    assert np.array_equal(got, want), "B = 0"
    # K = 0
    got = compute(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), bias)
    assert np.array_equal(got, want), "K = 0"
    # A = B = 1: C = relu(K + bias)
    M, K, N = 2, 9, 3
    bias = np.array([-10.0, -9.0, 0.5], np.float32)
    want = np.tile(np.maximum(K + bias.astype(np.float64), 0.0), (M, 1))
    got = compute(np.ones((M, K), np.float32), np.ones((K, N), np.float32), bias)
    assert np.array_equal(got, want), "A = B = 1"


def pin_integer_exact(compute):
    """Integer-valued inputs: the result is an exact integer matrix."""
    # small: Python integers
    M, K, N = 5, 7, 6
    A = synth.small_int_f32(4001, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_f32(4002, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_f32(4003, N, -8, 8)
    Ai, Bi, bi = A.astype(int).tolist(), B.astype(int).tolist(), bias.astype(int).tolist()
    want = [[max(0, sum(Ai[m][k] * Bi[k][n] for k in range(K)) + bi[n]) for n in range(N)] for m in range(M)]
    got = compute(A, B, bias)
    assert np.array_equal(got, np.array(want, dtype=np.float64)), "integer brute force"
    # moderate: numpy int64 matmul (exact)
    M, K, N = 33, 129, 47
    A = synth.small_int_f32(4011, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_f32(4012, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_f32(4013, N, -8, 8)
    pre = A.astype(np.int64) @ B.astype(np.int64) + bias.astype(np.int64)[None, :]
    got = compute(A, B, bias)
    assert np.array_equal(got, np.maximum(pre, 0).astype(np.float64)), "integer matmul"


def pin_reflection(compute):
    """relu(x) - relu(-x) = x: C(A,B,b) - C(-A,B,-b) equals A@B + b exactly (integers)."""
    M, K, N = 9, 31, 11
    A = synth.small_int_f32(4021, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_f32(4022, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_f32(4023, N, -8, 8)
    pre = A.astype(np.int64) @ B.astype(np.int64) + bias.astype(np.int64)[None, :]
    d = compute(A, B, bias) - compute(-A, B, -bias)
    assert np.array_equal(d, pre.astype(np.float64)), "reflection identity"


def pin_worked_example(compute):
    """The hand-derived cases stored in tests/golden/gemm_worked_example.json."""
    with open(os.path.join(GOLDEN, "gemm_worked_example.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        bias = np.array([float(x) for x in case["bias"]], np.float32)
        N = bias.shape[0]
        K = case.get("K", None)
        if K == 0:
            M = len(case["A"])
            A = np.zeros((M, 0), np.float32)
            B = np.zeros((0, N), np.float32)
        else:
            A = np.array(case["A"], np.float32)
            B = np.array(case["B"], np.float32)
        got = compute(A, B, bias)
        want = np.array(case["C"], np.float64)
        assert np.array_equal(got, want), "worked example %s: got %s" % (case.get("note", ""), got)
        assert not np.any(np.signbit(got)), "ReLU output carries a sign bit"


def pin_relu_sign(compute):
    """Non-positive pre-activations give +0 (no -0), positives pass unchanged."""
    A = np.array([[-1.0], [0.0], [1.0], [-0.0]], np.float32)
    B = np.array([[1.0, -1.0, 0.0]], np.float32)
    bias = np.array([0.0, -0.0, -0.0], np.float32)
    got = compute(A, B, bias)
    want = np.array([[0, 1, 0], [0, 0, 0], [1, 0, 0], [0, 0, 0]], np.float64)
    assert np.array_equal(got, want)
    assert not np.any(np.signbit(got)), "-0 leaked through the ReLU"
    assert np.all(got >= 0)


def pin_k_order(compute):
    """The sum runs in ascending k (the oracle's documented order).

    Products 2^60, -2^60, 2^-30 summed in ascending k give 2^-30; the
    descending order loses the small term and gives 0.
    """
    A = np.array([[2.0 ** 30, -(2.0 ** 30), 1.0]], np.float32)
    B = np.array([[2.0 ** 30], [2.0 ** 30], [2.0 ** -30]], np.float32)
    bias = np.array([0.0], np.float32)
    got = compute(A, B, bias)
    assert got[0, 0] == 2.0 ** -30, "k order: got %r" % got[0, 0]


def pin_bf16_widening(compute_bf16):
    """bf16 bit patterns widen to the values the format defines."""
    # 0x3FC0 = 1.5, 0xC040 = -3.0, 0x4100 = 8.0, 0x3E80 = 0.25, 0x0001 = 2^-133
    A = np.array([[0x3FC0, 0x3E80]], np.uint16)
    B = np.array([[0xC040], [0x4100]], np.uint16)
    bias = np.array([0x4100], np.uint16)
    got = compute_bf16(A, B, bias)
    # 1.5 * -3 + 0.25 * 8 + 8 = 5.5
    assert got[0, 0] == 5.5, got
    A = np.array([[0x0001]], np.uint16)
    B = np.array([[0x3F80]], np.uint16)
    bias = np.array([0x0000], np.uint16)
    got = compute_bf16(A, B, bias)
    assert got[0, 0] == 2.0 ** -133, got
    # integers in bf16: exact
    M, K, N = 7, 40, 9
    A = synth.small_int_bf16_bits(4031, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_bf16_bits(4032, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_bf16_bits(4033, N, -8, 8)
    Ai = synth.bf16_bits_to_f32(A).astype(np.int64)
    Bi = synth.bf16_bits_to_f32(B).astype(np.int64)
    bi = synth.bf16_bits_to_f32(bias).astype(np.int64)
    want = np.maximum(Ai @ Bi + bi[None, :], 0).astype(np.float64)
    assert np.array_equal(compute_bf16(A, B, bias), want), "bf16 integer case"


FP32_PINS = [pin_fraction_bruteforce, pin_closed_forms, pin_integer_exact, pin_reflection,
             pin_worked_example, pin_relu_sign, pin_k_order]


def run_all(compute, compute_bf16=None):
    """Run every pin; returns the list of (pin name, error) that failed."""
    failures = []
    for pin in FP32_PINS:
        try:
            pin(compute)
        except AssertionError as e:  # noqa: PERF203
            failures.append((pin.__name__, str(e)[:200]))
    if compute_bf16 is not None:
        for pin in (pin_bf16_widening, lambda c: pin_fraction_bruteforce(c, "bf16")):
            try:
                pin(compute_bf16)
            except AssertionError as e:
                failures.append((getattr(pin, "__name__", "bf16"), str(e)[:200]))
    return failures
