"""The pins are strong enough: each plausible mistake planted in the oracle fails one.

Every mutant is a textual patch of oracle/oracle.c, compiled on the CPU into a
temporary library; the real oracle is never modified.
"""
import os
import subprocess

import pytest

from oracle import OracleLib
from oracle_pins import run_all

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTANTS = {
    "drop_bias": ("relu64(C[i * N + j] + bias[j])", "relu64(C[i * N + j])"),
    "bias_per_row": ("relu64(C[i * N + j] + bias[j])", "relu64(C[i * N + j] + bias[i % N])"),
    "relu_flipped": ("if (s > 0.0) return s;", "if (s < 0.0) return s;"),
    "relu_passes_negatives": ("return 0.0;           /* +0", "return s;           /* +0"),
    "relu_minus_zero": ("return 0.0;           /* +0", "return -0.0;           /* +0"),
    "skip_first_k": ("for (int64_t k = 0; k < K; ++k) {\n                const double *brow",
                     "for (int64_t k = 1; k < K; ++k) {\n                const double *brow"),
    "k_descending": ("for (int64_t k = 0; k < K; ++k) {\n                const double *brow",
                     "for (int64_t k = K - 1; k >= 0; --k) {\n                const double *brow"),
    "a_transposed": ("double a = A[i * K + k];", "double a = A[k * M + i];"),
    "b_transposed": ("crow[j] += a * brow[j];", "crow[j] += a * B[j * K + k];"),
    "fp32_accumulator": ("crow[j] += a * brow[j];", "crow[j] = (float)(crow[j] + a * brow[j]);"),
    "sign_of_product": ("crow[j] += a * brow[j];", "crow[j] += a * (j % 7 == 3 ? -brow[j] : brow[j]);"),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, "mutation site for %s no longer in oracle.c" % name
    mutated = source.replace(old, new, 1)
    c_path = tmp_path / ("oracle_%s.c" % name)
    so_path = tmp_path / ("liboracle_%s.so" % name)
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so_path),
                    str(c_path)], check=True)
    lib = OracleLib(str(so_path))
    failures = run_all(lambda A, B, b: lib.gemm_bias_relu(A, B, b, threads=2),
                       lambda A, B, b: lib.gemm_bias_relu(A, B, b, threads=2))
    assert failures, "mutant %s passed every pin" % name


def test_unmutated_source_passes(source, tmp_path):
    so_path = tmp_path / "liboracle_clean.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so_path), SRC],
                   check=True)
    lib = OracleLib(str(so_path))
    assert run_all(lambda A, B, b: lib.gemm_bias_relu(A, B, b, threads=2),
                   lambda A, B, b: lib.gemm_bias_relu(A, B, b, threads=2)) == []
