"""bf16 GEMM + bias + ReLU (fp32 accumulate and output) on the GPU against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows

pytestmark = pytest.mark.gpu

SLACK = 4096
NAN_BF16 = 0x7FC0
C_GUARD = 4096
C_SENTINEL = -12345.0


def _padded(bits):
    """A device view of bf16 bit patterns inside a buffer whose slack is NaN."""
    import torch
    flat = np.ascontiguousarray(bits).reshape(-1).view(np.int16)
    buf = torch.full((flat.size + 2 * SLACK,), NAN_BF16, dtype=torch.int16, device="cuda")
    buf[SLACK:SLACK + flat.size] = torch.from_numpy(flat).cuda()
    return buf[SLACK:SLACK + flat.size].view(*bits.shape)


def run_gemm(gpu, A, B, bias, stages=4, config=None, guards=True):
    import torch
    M, K = A.shape
    N = B.shape[1]
    if guards:
        dA, dB, db = _padded(A), _padded(B), _padded(bias)
        cbuf = torch.full((M * N + 2 * C_GUARD,), C_SENTINEL, dtype=torch.float32, device="cuda")
        dC = cbuf[C_GUARD:C_GUARD + M * N].view(M, N)
    else:
        dA, dB, db = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda() for x in (A, B, bias))
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("gemm bf16 M=%d N=%d K=%d stages=%d config=%s" % (M, N, K, stages, config))
    if config is None:
        gpu.gemm_bias_relu_bf16(dA, dB, db, dC, stages=stages)
    else:
        gpu.gemm_bias_relu_ex(dA, dB, db, dC, stages=stages, config=config)
    gpu.check_device_status()
    if guards:
        c = cbuf.cpu().numpy()
        assert np.all(c[:C_GUARD] == C_SENTINEL) and np.all(c[C_GUARD + M * N:] == C_SENTINEL), "C guard written"
        return c[C_GUARD:C_GUARD + M * N].reshape(M, N)
    return dC.cpu().numpy()


def int_case(seed, M, N, K):
    return (synth.small_int_bf16_bits(seed + 1, M * K, -3, 3).reshape(M, K),
            synth.small_int_bf16_bits(seed + 2, K * N, -3, 3).reshape(K, N),
            synth.small_int_bf16_bits(seed + 3, N, -8, 8))


def normal_case(seed, M, N, K):
    return (synth.normal_bf16_bits(seed + 1, M * K).reshape(M, K),
            synth.normal_bf16_bits(seed + 2, K * N).reshape(K, N),
            synth.normal_bf16_bits(seed + 3, N))


def assert_close(C, ref):
    s = oracle.compare(C, ref)
    assert oracle.within_tolerance(s, "bf16"), s
    return s


SHAPES = [(1, 1, 1), (1, 300, 1), (300, 1, 7), (5, 7, 0), (3, 5, 7), (65, 64, 17), (129, 257, 33),
          (300, 200, 104), (200, 136, 264), (64, 64, 32), (256, 128, 32), (257, 129, 8), (33, 700, 64),
          (300, 520, 12)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes_integer_bit_exact_with_nan_guards(gpu, M, N, K):
    A, B, bias = int_case(M * 7 + N * 3 + K, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=3)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes_normal(gpu, M, N, K):
    A, B, bias = normal_case(M + 11 * N + 13 * K, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=2)
    assert_close(C, oracle.gemm_bias_relu(A, B, bias))


VARIANTS = [
    dict(BM=256, BN=128, BK=64, producer_waves=2, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=64, producer_waves=1, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=32, producer_waves=1, consumer_waves=4, group_k=32),
    dict(BM=128, BN=128, BK=64, producer_waves=1, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=32, producer_waves=1, consumer_waves=4),
    dict(BM=128, BN=128, BK=32, producer_waves=1, consumer_waves=4),
    dict(BM=256, BN=128, BK=64, producer_waves=2, consumer_waves=4),
    dict(BM=64, BN=64, BK=32, producer_waves=1, consumer_waves=4),
    dict(BM=64, BN=64, BK=32, producer_waves=2, consumer_waves=4),
    dict(BM=64, BN=64, BK=32, producer_waves=4, consumer_waves=4),
    dict(BM=256, BN=128, BK=32, producer_waves=1, consumer_waves=4, flags=1),
    dict(BM=128, BN=128, BK=32, producer_waves=1, consumer_waves=4, flags=1),
    dict(BM=64, BN=64, BK=32, producer_waves=1, consumer_waves=4, flags=1),
    dict(BM=256, BN=128, BK=64, producer_waves=2, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=32, producer_waves=1, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=64, producer_waves=2, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=64, producer_waves=4, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=64, producer_waves=4, consumer_waves=4, group_k=16),
    dict(BM=256, BN=128, BK=32, producer_waves=2, consumer_waves=4, group_k=32),
    dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4, group_k=16),
    # 48-deep k tiles: rows of 6 chunks, rotation swizzle; K = 296 leaves an 8-deep last tile
    dict(BM=256, BN=128, BK=48, producer_waves=4, consumer_waves=4, group_k=16),
    dict(BM=256, BN=128, BK=48, producer_waves=2, consumer_waves=4, group_k=16),
    # 256x256 tiles: 4 producers + 8 consumers (three waves per SIMD), single-fragment consumer walk
    dict(BM=256, BN=256, BK=32, producer_waves=4, consumer_waves=8),
    dict(BM=256, BN=256, BK=64, producer_waves=4, consumer_waves=8),
]


@pytest.mark.parametrize("config", VARIANTS, ids=lambda c: "x".join(str(v) for v in c.values()))
@pytest.mark.parametrize("stages", [1, 2, 3, 4, 6])
def test_variants_and_stages_integer_bit_exact(gpu, config, stages):
    M, N, K = 300, 520, 32 * 9 + 8
    A, B, bias = int_case(2000 + stages, M, N, K)
    lds = 256 + stages * (config["BM"] * config["BK"] + config["BK"] * config["BN"]) * 2
    if lds > 163840:
        with pytest.raises(gpu.WsgError) as e:
            run_gemm(gpu, A, B, bias, stages=stages, config=config)
        assert e.value.code == gpu.WSG_EUNSUPPORTED
        return
    C = run_gemm(gpu, A, B, bias, stages=stages, config=config)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


@pytest.mark.parametrize("K", [0, 16, 32 * 7, 32 * 8, 32 * 9 + 8])
def test_four_slot_ring_even_and_odd_tile_counts(gpu, K):
    """At S = 4 the 256 x 256 x 32 producers fill two slots per step when the k
    tile count is even and one slot per step when it is odd (here 0, 1, 7, 8
    and 10 tiles, the last one 8 deep); both give the oracle's integers
    exactly."""
    M, N = 300, 520
    A, B, bias = int_case(2100 + K, M, N, K)
    config = dict(BM=256, BN=256, BK=32, producer_waves=4, consumer_waves=8)
    C = run_gemm(gpu, A, B, bias, stages=4, config=config)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


def test_power_of_two_scaling_and_determinism(gpu):
    M, N, K = 384, 256, 520
    A, B, bias = normal_case(99, M, N, K)
    two = lambda x: synth.f32_to_bf16_bits_rne(2 * synth.bf16_bits_to_f32(x))  # noqa: E731  exact
    C1 = run_gemm(gpu, A, B, bias, guards=False)
    C1b = run_gemm(gpu, A, B, bias, guards=False)
    C2 = run_gemm(gpu, two(A), B, two(bias), guards=False)
    assert np.array_equal(C1.view(np.uint32), C1b.view(np.uint32)), "not deterministic"
    assert np.array_equal(C2, 2 * C1)


def test_full_size_workload_sampled(gpu):
    """8192^3 bf16, N(0,1)*0.1, 4-stage ring, default launch configuration: three rows of every
    tile row (every workgroup's output tile) against the oracle, and the reflection C(A, B, b) -
    C(-A, B, -b) (negating bf16 values flips their sign bit, exactly) against the oracle's
    pre-activation."""
    w = synth.WORKLOADS[5]
    M, N, K = w["M"], w["N"], w["K"]
    A = synth.normal_bf16_bits(synth.seed_for(5, "A"), M * K).reshape(M, K)
    B = synth.normal_bf16_bits(synth.seed_for(5, "B"), K * N).reshape(K, N)
    bias = synth.normal_bf16_bits(synth.seed_for(5, "bias"), N)
    C = run_gemm(gpu, A, B, bias, stages=w["stages"], guards=False)
    BM = gpu.resolve_config(gpu.WSG_BF16, M, N, K, w["stages"])["BM"]
    rows = stratified_rows(M, BM, 5)
    ref = oracle.gemm_bias_relu_rows(A, B, bias, rows)
    assert_close(C[rows], ref)
    assert np.all(C >= 0) and np.all(np.isfinite(C))
    assert 0.4 < float(np.mean(C == 0)) < 0.6
    neg = lambda x: x ^ np.uint16(0x8000)  # noqa: E731
    Cn = run_gemm(gpu, neg(A), B, neg(bias), stages=w["stages"], guards=False)
    assert not np.any((C > 0) & (Cn > 0)), "a pre-activation and its negation both positive"
    x_gpu = C[rows].astype(np.float64) - Cn[rows].astype(np.float64)
    x_ref = ref - oracle.gemm_bias_relu_rows(neg(A), B, neg(bias), rows)
    s = oracle.compare(x_gpu, x_ref)
    assert oracle.within_tolerance(s, "bf16"), s


def test_argument_errors(gpu):
    import torch
    A = torch.zeros((64, 64), dtype=torch.int16, device="cuda")
    b = torch.zeros(64, dtype=torch.int16, device="cuda")
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu_ex(A, A, b, config=dict(BM=96, BN=64, BK=32))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    rc = gpu.lib.gemm_bias_relu_bf16(4, 4, 4, A.data_ptr() + 1, A.data_ptr(), b.data_ptr(),
                                     torch.zeros(16, device="cuda").data_ptr(), 2)
    assert rc == gpu.WSG_EINVAL
