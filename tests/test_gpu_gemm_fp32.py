"""fp32 GEMM + bias + ReLU on the GPU against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows

pytestmark = pytest.mark.gpu

NAN_SLACK = 4096  # elements of NaN around each input view
C_GUARD = 4096
C_SENTINEL = -12345.0


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _nan_padded(x):
    """A device view of x inside a larger buffer whose slack is NaN."""
    import torch
    flat = np.ascontiguousarray(x).reshape(-1)
    buf = torch.full((flat.size + 2 * NAN_SLACK,), float("nan"), dtype=torch.float32, device="cuda")
    buf[NAN_SLACK:NAN_SLACK + flat.size] = torch.from_numpy(flat).cuda()
    return buf[NAN_SLACK:NAN_SLACK + flat.size].view(*x.shape)


def run_gemm(gpu, A, B, bias, stages=4, config=None, guards=True):
    import torch
    M, K = A.shape
    N = B.shape[1]
    if guards:
        dA, dB, db = _nan_padded(A), _nan_padded(B), _nan_padded(bias)
        cbuf = torch.full((M * N + 2 * C_GUARD,), C_SENTINEL, dtype=torch.float32, device="cuda")
        dC = cbuf[C_GUARD:C_GUARD + M * N].view(M, N)
    else:
        dA, dB, db = _dev(A), _dev(B), _dev(bias)
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("gemm fp32 M=%d N=%d K=%d stages=%d config=%s" % (M, N, K, stages, config))
    if config is None:
        gpu.gemm_bias_relu(dA, dB, db, dC, stages=stages)
    else:
        gpu.gemm_bias_relu_ex(dA, dB, db, dC, stages=stages, config=config)
    gpu.check_device_status()
    if guards:
        c = cbuf.cpu().numpy()
        assert np.all(c[:C_GUARD] == C_SENTINEL) and np.all(c[C_GUARD + M * N:] == C_SENTINEL), "C guard written"
        return c[C_GUARD:C_GUARD + M * N].reshape(M, N)
    return dC.cpu().numpy()


def uniform_case(seed, M, N, K):
    return (synth.uniform_pm1(seed + 1, M * K).reshape(M, K), synth.uniform_pm1(seed + 2, K * N).reshape(K, N),
            synth.uniform_pm1(seed + 3, N))


def int_case(seed, M, N, K):
    return (synth.small_int_f32(seed + 1, M * K, -3, 3).reshape(M, K),
            synth.small_int_f32(seed + 2, K * N, -3, 3).reshape(K, N),
            synth.small_int_f32(seed + 3, N, -8, 8))


def assert_close(C, ref):
    s = oracle.compare(C, ref)
    assert oracle.within_tolerance(s, "fp32"), s
    return s


# ---------------------------------------------------------------- workloads

def test_workload_256_tile64_two_stages(gpu):
    """256^3, tile 64x64x16, 2-stage ring, uniform[-1,1)."""
    A, B, bias = uniform_case(synth.seed_for(1, "A") - 1, 256, 256, 256)
    C = run_gemm(gpu, A, B, bias, stages=2, config=dict(BM=64, BN=64, BK=16))
    assert_close(C, oracle.gemm_bias_relu(A, B, bias))


def test_workload_256_integer_bit_exact(gpu):
    A, B, bias = int_case(50, 256, 256, 256)
    C = run_gemm(gpu, A, B, bias, stages=2, config=dict(BM=64, BN=64, BK=16))
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


# ---------------------------------------------------------------- shapes

SHAPES = [(1, 1, 1), (1, 300, 1), (300, 1, 7), (5, 7, 0), (3, 5, 7), (65, 64, 17), (129, 257, 33),
          (300, 200, 100), (200, 136, 260), (64, 64, 16), (128, 128, 16), (257, 129, 4), (33, 700, 64)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes_integer_bit_exact_with_nan_guards(gpu, M, N, K):
    A, B, bias = int_case(M * 7 + N * 3 + K, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=3)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes_uniform(gpu, M, N, K):
    A, B, bias = uniform_case(M + 11 * N + 13 * K, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=2)
    assert_close(C, oracle.gemm_bias_relu(A, B, bias))


def test_empty_problems(gpu):
    import torch
    for M, N, K in [(0, 5, 5), (5, 0, 5), (0, 0, 0)]:
        A = torch.zeros((M, K), device="cuda")
        B = torch.zeros((K, N), device="cuda")
        bias = torch.zeros((N,), device="cuda")
        C = gpu.gemm_bias_relu(A, B, bias)
        assert tuple(C.shape) == (M, N)


# ---------------------------------------------------------------- configurations

VARIANTS = [
    dict(BM=128, BN=128, BK=16, producer_waves=1, consumer_waves=4),
    dict(BM=128, BN=128, BK=16, producer_waves=2, consumer_waves=4),
    dict(BM=256, BN=128, BK=16, producer_waves=2, consumer_waves=8),
    dict(BM=128, BN=256, BK=16, producer_waves=2, consumer_waves=8),
    dict(BM=128, BN=128, BK=32, producer_waves=2, consumer_waves=4),
    dict(BM=64, BN=64, BK=16, producer_waves=1, consumer_waves=4),
    dict(BM=64, BN=64, BK=16, producer_waves=2, consumer_waves=4),
    dict(BM=64, BN=64, BK=16, producer_waves=4, consumer_waves=4),
    dict(BM=128, BN=128, BK=16, producer_waves=1, consumer_waves=4, flags=1),
    dict(BM=64, BN=64, BK=16, producer_waves=1, consumer_waves=4, flags=1),
    dict(BM=256, BN=128, BK=32, producer_waves=2, consumer_waves=4),
    dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4),
    dict(BM=256, BN=128, BK=16, producer_waves=4, consumer_waves=4),
    dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=8),
]


@pytest.mark.parametrize("config", VARIANTS, ids=lambda c: "x".join(str(v) for v in c.values()))
@pytest.mark.parametrize("stages", [1, 2, 3, 4, 6])
def test_variants_and_stages_integer_bit_exact(gpu, config, stages):
    # several tiles in both directions, a ragged edge, and enough k-tiles to lap the ring
    M, N, K = 300, 520, 16 * 13 + 4
    A, B, bias = int_case(1000 + stages, M, N, K)
    lds = 256 + stages * (config["BM"] * config["BK"] + config["BK"] * config["BN"]) * 4
    if lds > 163840:
        # a ring that does not fit in LDS is refused, not launched
        with pytest.raises(gpu.WsgError) as e:
            run_gemm(gpu, A, B, bias, stages=stages, config=config)
        assert e.value.code == gpu.WSG_EUNSUPPORTED
        return
    C = run_gemm(gpu, A, B, bias, stages=stages, config=config)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


def test_power_of_two_scaling_and_determinism(gpu):
    M, N, K = 384, 256, 520
    A, B, bias = uniform_case(77, M, N, K)
    C1 = run_gemm(gpu, A, B, bias, guards=False)
    C1b = run_gemm(gpu, A, B, bias, guards=False)
    C2 = run_gemm(gpu, 2 * A, B, 2 * bias, guards=False)
    assert np.array_equal(C1.view(np.uint32), C1b.view(np.uint32)), "not deterministic"
    assert np.array_equal(C2, 2 * C1), "2A, 2b must give exactly 2C"


def test_argument_errors(gpu):
    import torch
    A = torch.zeros((64, 64), device="cuda")
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu(A, A, torch.zeros(64, device="cuda"), stages=0)
    assert e.value.code == gpu.WSG_EINVAL
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu(A, A, torch.zeros(64, device="cuda"), stages=30)  # 30 x 16 KiB > LDS
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu_ex(A, A, torch.zeros(64, device="cuda"), config=dict(BM=96, BN=64, BK=16))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    buf = torch.zeros(64 * 64 * 2, device="cuda")
    with pytest.raises(gpu.WsgError) as e:  # C overlaps A
        gpu.gemm_bias_relu(buf[:4096].view(64, 64), A, torch.zeros(64, device="cuda"),
                           buf[2048:6144].view(64, 64))
    assert e.value.code == gpu.WSG_EINVAL


# ---------------------------------------------------------------- full sizes (sampled)

def _tile_rows(gpu, M, N, K, stages, dtype=None):
    """BM of the launch configuration the library picks for this problem."""
    return gpu.resolve_config(gpu.WSG_FP32 if dtype is None else dtype, M, N, K, stages)["BM"]


@pytest.mark.parametrize("wid", [3, 4])
def test_full_size_workload_sampled(gpu, wid):
    """4096^3 and the ragged 3000x5000x4100 in the default launch configuration: three rows of
    every tile row (every workgroup's output tile) against the oracle, and the reflection
    C(A, B, b) - C(-A, B, -b), which gives back the GPU's own pre-activation (ReLU(x) - ReLU(-x)
    = x, and negating A and b negates every product and sum exactly), against the oracle's."""
    w = synth.WORKLOADS[wid]
    M, N, K = w["M"], w["N"], w["K"]
    A = synth.uniform_pm1(synth.seed_for(wid, "A"), M * K).reshape(M, K)
    B = synth.uniform_pm1(synth.seed_for(wid, "B"), K * N).reshape(K, N)
    bias = synth.uniform_pm1(synth.seed_for(wid, "bias"), N)
    C = run_gemm(gpu, A, B, bias, stages=w["stages"], guards=False)
    rows = stratified_rows(M, _tile_rows(gpu, M, N, K, w["stages"]), wid)
    ref = oracle.gemm_bias_relu_rows(A, B, bias, rows)
    assert_close(C[rows], ref)
    # properties over the whole output
    assert np.all(C >= 0) and np.all(np.isfinite(C))
    frac_zero = float(np.mean(C == 0))
    assert 0.4 < frac_zero < 0.6, frac_zero  # symmetric pre-activations: about half clamp to 0
    # the negative half: reflected inputs
    Cn = run_gemm(gpu, -A, B, -bias, stages=w["stages"], guards=False)
    assert not np.any((C > 0) & (Cn > 0)), "a pre-activation and its negation both positive"
    x_gpu = C[rows].astype(np.float64) - Cn[rows].astype(np.float64)
    x_ref = ref - oracle.gemm_bias_relu_rows(-A, B, -bias, rows)
    s = oracle.compare(x_gpu, x_ref)
    assert oracle.within_tolerance(s, "fp32"), s


@pytest.mark.parametrize("stages", [2, 4])  # 256x128x32 and 256x128x16 tiles
def test_ragged_full_size_integer_bit_exact(gpu, stages):
    M, N, K = 3000, 5000, 4100
    A, B, bias = int_case(4444, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=stages, guards=False)
    rows = stratified_rows(M, _tile_rows(gpu, M, N, K, stages), 5 + stages)
    assert np.array_equal(C[rows].astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))
    # last tile row and column (56 rows, 8 columns past the last full tile)
    cols = np.arange(N - 8, N)
    ms = np.repeat(np.arange(M - 56, M), cols.size)
    ns = np.tile(cols, 56)
    got = C[ms, ns].astype(np.float64)
    assert np.array_equal(got, oracle.gemm_bias_relu_at(A, B, bias, ms, ns))
