"""The CPU oracle against its pins (exact rationals, closed forms, integers...)."""
import numpy as np
import pytest

import oracle
import synth
from oracle_pins import (FP32_PINS, pin_bf16_widening, pin_fraction_bruteforce,
                         exact_gemm_bias_relu)


def _full(lib):
    return lambda A, B, b: lib.gemm_bias_relu(A, B, b, threads=2)


def _rows(lib):
    def f(A, B, b):
        M = np.asarray(A).shape[0]
        return lib.gemm_bias_relu_rows(A, B, b, np.arange(M)[::-1], threads=2)[::-1]
    return f


def _at(lib):
    def f(A, B, b):
        M, N = np.asarray(A).shape[0], np.asarray(B).shape[1]
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return lib.gemm_bias_relu_at(A, B, b, mm.ravel(), nn.ravel(), threads=2).reshape(M, N)
    return f


@pytest.mark.parametrize("variant", [_full, _rows, _at], ids=["full", "rows", "at"])
@pytest.mark.parametrize("pin", FP32_PINS, ids=lambda p: p.__name__)
def test_fp32_pin(oracle_lib, variant, pin):
    pin(variant(oracle_lib))


@pytest.mark.parametrize("variant", [_full, _rows, _at], ids=["full", "rows", "at"])
def test_bf16_pins(oracle_lib, variant):
    pin_bf16_widening(variant(oracle_lib))
    pin_fraction_bruteforce(variant(oracle_lib), "bf16")


def test_blocking_spans_several_blocks(oracle_lib):
    """Sizes beyond the oracle's row/column blocks still match exact integers."""
    M, K, N = 37, 70, 1100  # 3 row blocks, 3 column blocks
    A = synth.small_int_f32(4101, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_f32(4102, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_f32(4103, N, -8, 8)
    pre = A.astype(np.int64) @ B.astype(np.int64) + bias.astype(np.int64)[None, :]
    assert np.array_equal(oracle_lib.gemm_bias_relu(A, B, bias), np.maximum(pre, 0).astype(np.float64))


def test_thread_count_does_not_change_result(oracle_lib):
    M, K, N = 40, 300, 600
    A = synth.uniform_pm1(4201, M * K).reshape(M, K)
    B = synth.uniform_pm1(4202, K * N).reshape(K, N)
    bias = synth.uniform_pm1(4203, N)
    c1 = oracle_lib.gemm_bias_relu(A, B, bias, threads=1)
    c4 = oracle_lib.gemm_bias_relu(A, B, bias, threads=4)
    assert np.array_equal(c1, c4)


def test_uniform_case_against_fractions_wide(oracle_lib):
    """A few elements of a non-square product with K = 257 against exact sums."""
    M, K, N = 3, 257, 5
    A = synth.uniform_pm1(4301, M * K).reshape(M, K)
    B = synth.uniform_pm1(4302, K * N).reshape(K, N)
    bias = synth.uniform_pm1(4303, N)
    C = oracle_lib.gemm_bias_relu(A, B, bias)
    exact, mag = exact_gemm_bias_relu(A, B, bias)
    for m in range(M):
        for n in range(N):
            assert abs(C[m, n] - float(exact[m][n])) <= float(mag[m][n]) * (K + 1) * 2.0 ** -52


def test_compare_metrics():
    ref = np.array([[1.0, 2.0], [0.0, 4.0]])
    s = oracle.compare(ref + np.array([[1e-4, 0.0], [0.0, -2e-4]]), ref)
    assert s["max_abs"] == pytest.approx(2e-4)
    assert s["rel_fro"] == pytest.approx(np.sqrt(1e-8 + 4e-8) / np.sqrt(21.0))
    assert oracle.within_tolerance(s, "fp32") is False  # rel_fro 4.9e-5 > 1e-5
    assert oracle.within_tolerance(oracle.compare(ref, ref), "fp32")
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert not oracle.within_tolerance(oracle.compare(bad, ref), "bf16")


def test_argument_errors(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.gemm_bias_relu(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32),
                                  np.zeros(2, np.float32))
    with pytest.raises(TypeError):
        oracle_lib.gemm_bias_relu(np.zeros((2, 3)), np.zeros((3, 2)), np.zeros(2))
    with pytest.raises(RuntimeError):
        oracle_lib.gemm_bias_relu_at(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32),
                                     np.zeros(2, np.float32), [2], [0])
