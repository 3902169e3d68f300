"""The homogeneous baseline GEMM (no producer waves; every wave loads, a
workgroup barrier, every wave computes) against the fp64 oracle, and against
the wave-specialized kernel with the same tile and consumer fragments."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_gemm_bf16 import int_case as int_bf16
from test_gpu_gemm_bf16 import normal_case
from test_gpu_gemm_bf16 import run_gemm as run_bf16
from conftest import stratified_rows
from test_gpu_gemm_fp32 import uniform_case
from test_gpu_gemm_fp32 import int_case as int_f32
from test_gpu_gemm_fp32 import run_gemm as run_f32

pytestmark = pytest.mark.gpu

HOMOGENEOUS = 4  # WSG_FLAG_HOMOGENEOUS

F32_TILES = [dict(BM=256, BN=128, BK=32, consumer_waves=4), dict(BM=256, BN=128, BK=16, consumer_waves=4),
             dict(BM=256, BN=128, BK=32, consumer_waves=8), dict(BM=256, BN=128, BK=16, consumer_waves=8),
             dict(BM=128, BN=128, BK=32, consumer_waves=4), dict(BM=64, BN=64, BK=16, consumer_waves=4)]
BF16_TILES = [dict(BM=256, BN=128, BK=64, consumer_waves=4), dict(BM=256, BN=128, BK=64, consumer_waves=8),
              dict(BM=256, BN=128, BK=32, consumer_waves=4), dict(BM=128, BN=128, BK=32, consumer_waves=4),
              dict(BM=64, BN=64, BK=32, consumer_waves=4), dict(BM=256, BN=128, BK=48, consumer_waves=4),
              dict(BM=256, BN=256, BK=32, consumer_waves=8)]


def _h(cfg):
    return dict(cfg, flags=HOMOGENEOUS)


def _lds(cfg, stages, esz):
    return 256 + stages * (cfg["BM"] * cfg["BK"] + cfg["BK"] * cfg["BN"]) * esz


def _id(c):
    return "%dx%dx%d_w%d" % (c["BM"], c["BN"], c["BK"], c["consumer_waves"])


@pytest.mark.parametrize("config", F32_TILES, ids=_id)
@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_fp32_tiles_and_stages_integer_bit_exact(gpu, config, stages):
    # several tiles both ways, ragged M and N, 14 k-tiles of 16 (the last one 4 wide)
    M, N, K = 300, 520, 16 * 13 + 4
    A, B, bias = int_f32(2000 + stages, M, N, K)
    if _lds(config, stages, 4) > 163840:
        with pytest.raises(gpu.WsgError) as e:
            run_f32(gpu, A, B, bias, stages=stages, config=_h(config))
        assert e.value.code == gpu.WSG_EUNSUPPORTED
        return
    C = run_f32(gpu, A, B, bias, stages=stages, config=_h(config))
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


@pytest.mark.parametrize("config", BF16_TILES, ids=_id)
@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_bf16_tiles_and_stages_integer_bit_exact(gpu, config, stages):
    M, N, K = 300, 520, 32 * 6 + 8
    A, B, bias = int_bf16(3000 + stages, M, N, K)
    if _lds(config, stages, 2) > 163840:
        with pytest.raises(gpu.WsgError) as e:
            run_bf16(gpu, A, B, bias, stages=stages, config=_h(config))
        assert e.value.code == gpu.WSG_EUNSUPPORTED
        return
    C = run_bf16(gpu, A, B, bias, stages=stages, config=_h(config))
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


# aligned shapes (K and N multiples of 4 fp32 / 8 bf16 elements): tiny, empty K, one
# partial tile, a single k-tile, many k-tiles
F32_SHAPES = [(1, 4, 4), (5, 8, 0), (3, 4, 12), (65, 64, 20), (129, 260, 36), (300, 200, 100), (64, 64, 16),
              (257, 132, 4), (33, 700, 64)]
BF16_SHAPES = [(1, 8, 8), (5, 8, 0), (3, 8, 16), (65, 64, 24), (129, 264, 40), (300, 200, 104), (64, 64, 32),
               (257, 136, 8)]


@pytest.mark.parametrize("M,N,K", F32_SHAPES)
def test_fp32_shapes_uniform(gpu, M, N, K):
    A, B, bias = uniform_case(5 * M + 7 * N + K, M, N, K)
    C = run_f32(gpu, A, B, bias, stages=2, config=dict(flags=HOMOGENEOUS))
    s = oracle.compare(C, oracle.gemm_bias_relu(A, B, bias))
    assert oracle.within_tolerance(s, "fp32"), s


@pytest.mark.parametrize("M,N,K", BF16_SHAPES)
def test_bf16_shapes_normal(gpu, M, N, K):
    A, B, bias = normal_case(3 * M + 11 * N + K, M, N, K)
    C = run_bf16(gpu, A, B, bias, stages=2, config=dict(flags=HOMOGENEOUS))
    s = oracle.compare(C, oracle.gemm_bias_relu(A, B, bias))
    assert oracle.within_tolerance(s, "bf16"), s


def test_same_bits_as_the_specialized_kernel(gpu):
    """Same tile, consumer fragments and MFMA order: the roles change when a
    tile is loaded, not the arithmetic, so the outputs agree bit for bit."""
    M, N, K = 512, 384, 1000
    A, B, bias = uniform_case(99, M, N, K)
    for waves in (4, 8):
        spec = dict(BM=256, BN=128, BK=32, producer_waves=2, consumer_waves=waves)
        C_spec = run_f32(gpu, A, B, bias, stages=3, config=spec, guards=False)
        for stages in (1, 2, 3):
            C_h = run_f32(gpu, A, B, bias, stages=stages,
                          config=_h(dict(BM=256, BN=128, BK=32, consumer_waves=waves)), guards=False)
            assert np.array_equal(C_h.view(np.uint32), C_spec.view(np.uint32))
    Ab, Bb, bb = normal_case(98, M, N, 1024)
    Cb_spec = run_bf16(gpu, Ab, Bb, bb, stages=2, config=dict(BM=256, BN=128, BK=64, producer_waves=1,
                                                                consumer_waves=4, group_k=32), guards=False)
    Cb_h = run_bf16(gpu, Ab, Bb, bb, stages=2, config=_h(dict(BM=256, BN=128, BK=64, consumer_waves=4)),
                    guards=False)
    assert np.array_equal(Cb_h.view(np.uint32), Cb_spec.view(np.uint32))
    # 256 x 256 tiles: the single-fragment consumer walk of the specialized kernel (three waves per SIMD)
    # and the homogeneous kernel's group-at-a-time MFMAs accumulate every block in the same k order
    for bk, stages in ((32, 4), (32, 2)):
        Cw_spec = run_bf16(gpu, Ab, Bb, bb, stages=stages, config=dict(BM=256, BN=256, BK=bk, producer_waves=4,
                                                                       consumer_waves=8), guards=False)
        Cw_h = run_bf16(gpu, Ab, Bb, bb, stages=stages, config=_h(dict(BM=256, BN=256, BK=bk, consumer_waves=8)),
                        guards=False)
        assert np.array_equal(Cw_h.view(np.uint32), Cw_spec.view(np.uint32)), (bk, stages)


def test_full_size_fp32_sampled(gpu):
    """4096^3 fp32, the homogeneous kernel in the configuration the benchmark times."""
    w = synth.WORKLOADS[3]
    M, N, K = w["M"], w["N"], w["K"]
    A = synth.uniform_pm1(synth.seed_for(3, "A"), M * K).reshape(M, K)
    B = synth.uniform_pm1(synth.seed_for(3, "B"), K * N).reshape(K, N)
    bias = synth.uniform_pm1(synth.seed_for(3, "bias"), N)
    C = run_f32(gpu, A, B, bias, stages=2, config=dict(flags=HOMOGENEOUS), guards=False)
    rows = stratified_rows(M, 256, 33)
    s = oracle.compare(C[rows], oracle.gemm_bias_relu_rows(A, B, bias, rows))
    assert oracle.within_tolerance(s, "fp32"), s
    assert np.all(C >= 0) and np.all(np.isfinite(C))


def test_ragged_full_size_integer_bit_exact(gpu):
    M, N, K = 3000, 5000, 4100
    A, B, bias = int_f32(4545, M, N, K)
    C = run_f32(gpu, A, B, bias, stages=2, config=dict(flags=HOMOGENEOUS), guards=False)
    rows = stratified_rows(M, 256, 7)
    assert np.array_equal(C[rows].astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))
    cols = np.arange(N - 8, N)
    ms = np.repeat(np.arange(M - 56, M), cols.size)
    ns = np.tile(cols, 56)
    assert np.array_equal(C[ms, ns].astype(np.float64), oracle.gemm_bias_relu_at(A, B, bias, ms, ns))


def test_resolve_and_errors(gpu):
    import torch
    r = gpu.resolve_config(gpu.WSG_FP32, 4096, 4096, 4096, 2, dict(flags=HOMOGENEOUS))
    assert r["producer_waves"] == 0 and r["flags"] & HOMOGENEOUS and (r["BM"], r["BN"]) == (256, 128)
    r = gpu.resolve_config(gpu.WSG_BF16, 8192, 8192, 8192, 2, dict(flags=HOMOGENEOUS))
    assert r["producer_waves"] == 0 and r["flags"] & HOMOGENEOUS
    # the plain entry points never pick the homogeneous kernel
    assert gpu.resolve_config(gpu.WSG_FP32, 4096, 4096, 4096, 2)["producer_waves"] > 0
    A = torch.zeros((64, 64), device="cuda")
    b = torch.zeros(64, device="cuda")
    with pytest.raises(gpu.WsgError) as e:  # roles asked of the kernel without roles
        gpu.gemm_bias_relu_ex(A, A, b, config=dict(flags=HOMOGENEOUS, producer_waves=1))
    assert e.value.code == gpu.WSG_EINVAL
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu_ex(A, A, b, config=dict(flags=HOMOGENEOUS | gpu.WSG_FLAG_GENERAL_PRODUCER))
    assert e.value.code == gpu.WSG_EINVAL
    A7 = torch.zeros((64, 7), device="cuda")  # K = 7: rows not 16-byte aligned
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu_ex(A7, torch.zeros((7, 64), device="cuda"), b, config=dict(flags=HOMOGENEOUS))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
