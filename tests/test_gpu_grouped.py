"""Grouped (mixture-of-experts) GEMM + bias + ReLU on the GPU against the fp64 oracle.

Operands sit inside NaN-filled buffers and C inside a sentinel-filled one, so a
read past an expert's rows or blocks, or a write past C, shows up.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows
from test_gpu_gemm_fp32 import run_gemm as run_f32

pytestmark = pytest.mark.gpu

SLACK = 4096
C_GUARD = 4096
C_SENTINEL = -12345.0
NAN_BF16 = 0x7FC0


def _padded(x):
    import torch
    if x.dtype == np.float32:
        flat = np.ascontiguousarray(x).reshape(-1)
        buf = torch.full((flat.size + 2 * SLACK,), float("nan"), dtype=torch.float32, device="cuda")
    else:
        flat = np.ascontiguousarray(x).reshape(-1).view(np.int16)
        buf = torch.full((flat.size + 2 * SLACK,), NAN_BF16, dtype=torch.int16, device="cuda")
    buf[SLACK:SLACK + flat.size] = torch.from_numpy(flat).cuda()
    return buf[SLACK:SLACK + flat.size].view(*x.shape)


def _plain(x):
    import torch
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x if x.dtype == np.float32 else x.view(np.int16)).cuda()


def run_grouped(gpu, A, B, bias, rows, stages=4, config=None, guards=True):
    import torch
    M, N = A.shape[0], B.shape[2]
    if guards:
        dA, dB, db = _padded(A), _padded(B), _padded(bias)
        cbuf = torch.full((M * N + 2 * C_GUARD,), C_SENTINEL, dtype=torch.float32, device="cuda")
        dC = cbuf[C_GUARD:C_GUARD + M * N].view(M, N)
    else:
        dA, dB, db = _plain(A), _plain(B), _plain(bias)
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("grouped %s rows=%s N=%d K=%d stages=%d config=%s" % (A.dtype, list(rows)[:12], N, A.shape[1], stages, config))
    gpu.grouped_gemm_bias_relu_ex(dA, dB, db, rows, dC, stages=stages, config=config)
    gpu.check_device_status()
    if guards:
        c = cbuf.cpu().numpy()
        assert np.all(c[:C_GUARD] == C_SENTINEL) and np.all(c[C_GUARD + M * N:] == C_SENTINEL), "C guard written"
        return c[C_GUARD:C_GUARD + M * N].reshape(M, N)
    return dC.cpu().numpy()


def int_f32(seed, rows, N, K):
    G, M = len(rows), sum(rows)
    return (synth.small_int_f32(seed + 1, M * K, -3, 3).reshape(M, K),
            synth.small_int_f32(seed + 2, G * K * N, -3, 3).reshape(G, K, N),
            synth.small_int_f32(seed + 3, G * N, -8, 8).reshape(G, N))


def int_bf16(seed, rows, N, K):
    G, M = len(rows), sum(rows)
    return (synth.small_int_bf16_bits(seed + 1, M * K, -3, 3).reshape(M, K),
            synth.small_int_bf16_bits(seed + 2, G * K * N, -3, 3).reshape(G, K, N),
            synth.small_int_bf16_bits(seed + 3, G * N, -8, 8).reshape(G, N))


def uniform_f32(seed, rows, N, K):
    G, M = len(rows), sum(rows)
    return (synth.uniform_pm1(seed + 1, M * K).reshape(M, K), synth.uniform_pm1(seed + 2, G * K * N).reshape(G, K, N),
            synth.uniform_pm1(seed + 3, G * N).reshape(G, N))


def normal_bf16(seed, rows, N, K):
    G, M = len(rows), sum(rows)
    return (synth.normal_bf16_bits(seed + 1, M * K).reshape(M, K),
            synth.normal_bf16_bits(seed + 2, G * K * N).reshape(G, K, N),
            synth.normal_bf16_bits(seed + 3, G * N).reshape(G, N))


# empty experts first, inside and last; single rows; several tiles; ragged tails
ROWS = [[0, 1, 37, 300, 0, 513, 64, 0], [257], [0, 0, 5], [128, 128, 128], [1, 1, 1, 1, 1, 1, 1, 700]]

F32_CONFIGS = [None, dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4),
               dict(BM=128, BN=128, BK=16), dict(BM=64, BN=64, BK=16), dict(flags=4),
               dict(flags=1)]


def _cid(c):
    return "default" if c is None else "_".join("%s%s" % (k, v) for k, v in c.items())


@pytest.mark.parametrize("config", F32_CONFIGS, ids=_cid)
@pytest.mark.parametrize("ri", range(len(ROWS)))
def test_fp32_integer_bit_exact(gpu, ri, config):
    rows = ROWS[ri]
    A, B, bias = int_f32(700 + ri, rows, 520, 212)
    C = run_grouped(gpu, A, B, bias, rows, stages=3, config=config)
    assert np.array_equal(C.astype(np.float64), oracle.grouped_gemm_bias_relu(A, B, bias, rows))


@pytest.mark.parametrize("ri", range(len(ROWS)))
def test_bf16_integer_bit_exact(gpu, ri):
    rows = ROWS[ri]
    A, B, bias = int_bf16(800 + ri, rows, 264, 200)
    C = run_grouped(gpu, A, B, bias, rows, stages=4)
    assert np.array_equal(C.astype(np.float64), oracle.grouped_gemm_bias_relu(A, B, bias, rows))


def test_fp32_unaligned_k_register_producer(gpu):
    rows = [0, 90, 200, 1]
    A, B, bias = int_f32(900, rows, 130, 211)  # K = 211: rows not 16-byte aligned
    C = run_grouped(gpu, A, B, bias, rows, stages=2)
    assert np.array_equal(C.astype(np.float64), oracle.grouped_gemm_bias_relu(A, B, bias, rows))


def test_fp32_uniform_within_tolerance(gpu):
    rows = [300, 0, 129, 700]
    A, B, bias = uniform_f32(910, rows, 384, 1000)
    C = run_grouped(gpu, A, B, bias, rows, stages=2)
    s = oracle.compare(C, oracle.grouped_gemm_bias_relu(A, B, bias, rows))
    assert oracle.within_tolerance(s, "fp32"), s


def test_bf16_normal_within_tolerance(gpu):
    rows = [100, 0, 257, 31]
    A, B, bias = normal_bf16(920, rows, 264, 520)
    C = run_grouped(gpu, A, B, bias, rows, stages=4)
    s = oracle.compare(C, oracle.grouped_gemm_bias_relu(A, B, bias, rows))
    assert oracle.within_tolerance(s, "bf16"), s


def test_each_expert_equals_the_plain_gemm_bit_for_bit(gpu):
    """One launch over all experts against one plain launch per expert, same configuration."""
    rows = [300, 0, 129, 700, 64]
    A, B, bias = uniform_f32(930, rows, 384, 1000)
    cfg = dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4)
    C = run_grouped(gpu, A, B, bias, rows, stages=2, config=cfg, guards=False)
    start = 0
    for e, n in enumerate(rows):
        if n:
            Ce = run_f32(gpu, A[start:start + n], B[e], bias[e], stages=2, config=dict(cfg, flags=32),  # NO_STREAM_K
                         guards=False)
            assert np.array_equal(C[start:start + n].view(np.uint32), Ce.view(np.uint32)), "expert %d" % e
        start += n


def test_most_experts(gpu):
    G = gpu.WSG_MAX_GROUPS
    counts = synth.small_int_f32(940, G, 0, 40).astype(np.int64)
    rows = [int(r) for r in counts]
    A, B, bias = int_f32(941, rows, 136, 64)
    C = run_grouped(gpu, A, B, bias, rows, stages=2)
    assert np.array_equal(C.astype(np.float64), oracle.grouped_gemm_bias_relu(A, B, bias, rows))


def test_no_rows_or_columns_is_a_no_op(gpu):
    import torch
    A = torch.zeros((0, 16), device="cuda")
    B = torch.zeros((3, 16, 8), device="cuda")
    b = torch.zeros((3, 8), device="cuda")
    C = torch.full((0, 8), 1.0, device="cuda")
    gpu.grouped_gemm_bias_relu_ex(A, B, b, [0, 0, 0], C)
    A = torch.ones((5, 16), device="cuda")
    B0 = torch.zeros((2, 16, 0), device="cuda")
    C0 = torch.empty((5, 0), device="cuda")
    gpu.grouped_gemm_bias_relu_ex(A, B0, torch.zeros((2, 0), device="cuda"), [2, 3], C0)
    gpu.check_device_status()


def test_errors(gpu):
    import ctypes
    import torch
    A = torch.zeros((4, 16), device="cuda")
    B = torch.zeros((2, 16, 8), device="cuda")
    b = torch.zeros((2, 8), device="cuda")
    C = torch.zeros((4, 8), device="cuda")
    lib = gpu.lib

    def call(groups, rows, Bp=B.data_ptr(), Cp=C.data_ptr()):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        return lib.grouped_gemm_bias_relu_ex(gpu.WSG_FP32, groups, arr, 8, 16, A.data_ptr(), Bp, b.data_ptr(), Cp,
                                             2, None)
    assert call(0, []) == gpu.WSG_EINVAL
    assert call(gpu.WSG_MAX_GROUPS + 1, [0] * (gpu.WSG_MAX_GROUPS + 1)) == gpu.WSG_EUNSUPPORTED
    assert call(2, [5, -1]) == gpu.WSG_EINVAL
    assert lib.grouped_gemm_bias_relu_ex(gpu.WSG_FP32, 2, None, 8, 16, A.data_ptr(), B.data_ptr(), b.data_ptr(),
                                         C.data_ptr(), 2, None) == gpu.WSG_EINVAL
    big = torch.zeros(2 * 16 * 8 + 64, device="cuda")
    # C inside the second expert's block of B
    assert call(2, [2, 2], Bp=big.data_ptr(), Cp=big.data_ptr() + 4 * 16 * 8 + 64) == gpu.WSG_EINVAL
    assert call(2, [2, 2]) == gpu.WSG_OK
    with pytest.raises(ValueError):
        gpu.grouped_gemm_bias_relu_ex(A, B, b, [1, 2])  # rows do not add up to A's
    gpu.check_device_status()


def test_full_size_moe_layer_sampled(gpu):
    """The benchmark's expert layer (8 experts, 4096 tokens top-2, K 4096, N 14336, bf16),
    in the launch configuration the benchmark times, against the oracle on sampled rows
    of every expert."""
    w = synth.MOE
    rows = [int(r) for r in synth.moe_group_rows(synth.seed_for(w["id"], "A") + 50, w["tokens"], w["experts"],
                                                    w["top_k"])]
    G, K, N, M = w["experts"], w["K"], w["N"], sum(rows)
    A = synth.normal_bf16_bits(synth.seed_for(w["id"], "A"), M * K).reshape(M, K)
    B = synth.normal_bf16_bits(synth.seed_for(w["id"], "B"), G * K * N).reshape(G, K, N)
    bias = synth.normal_bf16_bits(synth.seed_for(w["id"], "bias"), G * N).reshape(G, N)
    C = run_grouped(gpu, A, B, bias, rows, stages=w["stages"], guards=False)
    # three rows of every tile row of every expert (each expert's tiles start at its first row)
    BM = gpu.resolve_config(gpu.WSG_BF16, M, N, K, w["stages"])["BM"]
    starts = np.concatenate([[0], np.cumsum(rows)])
    want = np.concatenate([starts[e] + stratified_rows(rows[e], BM, e) for e in range(G) if rows[e]])
    s = oracle.compare(C[want], oracle.grouped_gemm_bias_relu_rows(A, B, bias, rows, want))
    assert oracle.within_tolerance(s, "bf16"), s
    assert np.all(C >= 0) and np.all(np.isfinite(C))
