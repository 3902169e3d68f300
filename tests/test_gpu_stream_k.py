"""Stream-K tail of the fp32 GEMM against the fp64 oracle.

A stream-K launch splits the K loop of some tiles between workgroups and sums
the pieces in a fixed order, so with small-integer inputs (every partial sum
exact in fp32) it must match the oracle bit for bit, and with random inputs it
must be deterministic and within the fp32 tolerance."""
import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows
from test_gpu_gemm_fp32 import int_case, run_gemm, uniform_case

pytestmark = pytest.mark.gpu

STREAM_K, NO_STREAM_K = 16, 32  # WSG_FLAG_STREAM_K, WSG_FLAG_NO_STREAM_K

TILES = [dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4),
         dict(BM=256, BN=128, BK=16, producer_waves=2, consumer_waves=8),
         dict(BM=128, BN=128, BK=32, producer_waves=2, consumer_waves=4),
         dict(BM=64, BN=64, BK=16, producer_waves=1, consumer_waves=4),
         dict(BM=128, BN=256, BK=16, producer_waves=2, consumer_waves=8)]


def _id(c):
    return "%dx%dx%d_p%d_c%d" % (c["BM"], c["BN"], c["BK"], c["producer_waves"], c["consumer_waves"])


def _uses_sk(gpu, M, N, K, stages, config):
    return bool(gpu.resolve_config(gpu.WSG_FP32, M, N, K, stages, config)["flags"] & STREAM_K)


# fewer tiles than workgroups (every tile split, some shares a single k step or
# none), one tile, one k step, ragged M, N and K
SHAPES = [(300, 520, 212), (1, 4, 4), (64, 64, 16), (257, 132, 36), (2000, 1000, 1000), (33, 700, 1604)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forced_integer_bit_exact(gpu, M, N, K):
    A, B, bias = int_case(6100 + M, M, N, K)
    config = dict(flags=STREAM_K)
    assert _uses_sk(gpu, M, N, K, 2, config)
    C = run_gemm(gpu, A, B, bias, stages=2, config=config)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


@pytest.mark.parametrize("config", TILES, ids=_id)
@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_forced_tiles_and_stages_integer_bit_exact(gpu, config, stages):
    M, N, K = 700, 900, 16 * 41 + 4
    A, B, bias = int_case(6200 + stages, M, N, K)
    cfg = dict(config, flags=STREAM_K)
    lds = 256 + stages * (config["BM"] + config["BN"]) * config["BK"] * 4
    if lds > 163840:
        with pytest.raises(gpu.WsgError) as e:
            run_gemm(gpu, A, B, bias, stages=stages, config=cfg)
        assert e.value.code == gpu.WSG_EUNSUPPORTED
        return
    assert _uses_sk(gpu, M, N, K, stages, cfg)
    C = run_gemm(gpu, A, B, bias, stages=stages, config=cfg)
    assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


def test_forced_uniform_within_tolerance_and_deterministic(gpu):
    M, N, K = 1000, 1200, 3000
    A, B, bias = uniform_case(6300, M, N, K)
    ref = oracle.gemm_bias_relu(A, B, bias)
    runs = [run_gemm(gpu, A, B, bias, stages=2, config=dict(flags=STREAM_K)) for _ in range(3)]
    for C in runs[1:]:
        assert np.array_equal(C.view(np.uint32), runs[0].view(np.uint32))
    s = oracle.compare(runs[0], ref)
    assert oracle.within_tolerance(s, "fp32"), s
    plain = run_gemm(gpu, A, B, bias, stages=2, config=dict(flags=NO_STREAM_K))
    assert oracle.within_tolerance(oracle.compare(plain, ref), "fp32")


def test_decision(gpu):
    # 3000 x 5000 with 256 x 128 tiles: 480 tiles, a ragged second round
    assert _uses_sk(gpu, 3000, 5000, 4100, 2, None)
    assert not _uses_sk(gpu, 3000, 5000, 4100, 2, dict(flags=NO_STREAM_K))
    # 512 tiles: whole rounds, no tail to spread
    assert not _uses_sk(gpu, 4096, 4096, 4096, 2, None)
    # fewer tiles than one round: the default launch is one wave of tiles
    assert not _uses_sk(gpu, 300, 520, 212, 2, None)
    # no stream-K kernel: the register-staged producer, the homogeneous baseline, bf16
    assert not _uses_sk(gpu, 300, 522, 212, 2, dict(flags=STREAM_K))
    assert not _uses_sk(gpu, 300, 520, 212, 2, dict(flags=STREAM_K | 4))
    assert not gpu.resolve_config(gpu.WSG_BF16, 3000, 5000, 4096, 2, dict(flags=STREAM_K))["flags"] & STREAM_K
    # K == 0: nothing to split; C = relu(bias)
    assert not _uses_sk(gpu, 300, 520, 0, 2, dict(flags=STREAM_K))
    # fewer 256 x 128 tiles than CUs but a deep K: the big tile, split along K
    r = gpu.resolve_config(gpu.WSG_FP32, 1024, 1024, 16384, 2)
    assert (r["BM"], r["BN"]) == (256, 128) and r["flags"] & STREAM_K
    # ... unless stream-K is turned off, or K is too short to give every CU 16 k steps
    r = gpu.resolve_config(gpu.WSG_FP32, 1024, 1024, 16384, 2, dict(flags=NO_STREAM_K))
    assert (r["BM"], r["BN"]) == (64, 64) and not r["flags"] & STREAM_K
    r = gpu.resolve_config(gpu.WSG_FP32, 1024, 1024, 1024, 2)
    assert (r["BM"], r["BN"]) == (64, 64) and not r["flags"] & STREAM_K
    # ... or when 256 tiles of 128 x 128 fill the chip and K is not very deep
    r = gpu.resolve_config(gpu.WSG_FP32, 2048, 2048, 1024, 2)
    assert (r["BM"], r["BN"]) == (128, 128) and not r["flags"] & STREAM_K
    r = gpu.resolve_config(gpu.WSG_FP32, 2048, 2048, 8192, 2)
    assert (r["BM"], r["BN"]) == (256, 128) and r["flags"] & STREAM_K
    # small tiles chosen explicitly with fewer tiles than workers: not split by default
    assert not _uses_sk(gpu, 1024, 1024, 16384, 2, dict(BM=128, BN=128, BK=32))


def test_workspace_reuse_and_growth(gpu):
    """Launches on one stream share a workspace that grows when needed; the
    counters start at zero on every launch."""
    small = dict(BM=64, BN=64, BK=16, producer_waves=1, consumer_waves=4, flags=STREAM_K)
    cases = [(500, 300, 404, small), (1500, 1300, 900, dict(flags=STREAM_K)), (500, 300, 404, small),
             (300, 520, 212, dict(flags=STREAM_K))]
    for i, (M, N, K, config) in enumerate(cases):
        A, B, bias = int_case(6400 + i, M, N, K)
        C = run_gemm(gpu, A, B, bias, stages=2, config=config)
        assert np.array_equal(C.astype(np.float64), oracle.gemm_bias_relu(A, B, bias)), (M, N, K)


def test_two_streams(gpu):
    """Stream-K launches on two streams at once use separate workspaces."""
    import torch
    shapes = [(700, 900, 660), (900, 700, 1204)]
    cases = [int_case(6500 + i, M, N, K) for i, (M, N, K) in enumerate(shapes)]
    refs = [oracle.gemm_bias_relu(*c) for c in cases]
    dev = [[torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in c] for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    say("stream-K on two streams")
    for i in range(10):
        j = i % 2
        with torch.cuda.stream(streams[j]):
            outs.append((j, gpu.gemm_bias_relu_ex(*dev[j], stages=2, config=dict(flags=STREAM_K))))
    torch.cuda.synchronize()
    gpu.check_device_status()
    for j, o in outs:
        assert np.array_equal(o.cpu().numpy().astype(np.float64), refs[j])


def test_full_size_ragged_default(gpu):
    """The 3000 x 5000 x 4100 workload as the benchmark launches it (stream-K
    tail by default): integer inputs exact on stratified rows and the last
    columns, uniform inputs deterministic and within tolerance."""
    w = synth.WORKLOADS[4]
    M, N, K = w["M"], w["N"], w["K"]
    assert _uses_sk(gpu, M, N, K, w["stages"], None)
    A, B, bias = int_case(6600, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=w["stages"], guards=False)
    rows = stratified_rows(M, 256, 11)
    assert np.array_equal(C[rows].astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))
    cols = np.arange(N - 8, N)
    ms = np.repeat(np.arange(M - 40, M), cols.size)
    ns = np.tile(cols, 40)
    assert np.array_equal(C[ms, ns].astype(np.float64), oracle.gemm_bias_relu_at(A, B, bias, ms, ns))

    A = synth.uniform_pm1(synth.seed_for(4, "A"), M * K).reshape(M, K)
    B = synth.uniform_pm1(synth.seed_for(4, "B"), K * N).reshape(K, N)
    bias = synth.uniform_pm1(synth.seed_for(4, "bias"), N)
    C1 = run_gemm(gpu, A, B, bias, stages=w["stages"], guards=False)
    C2 = run_gemm(gpu, A, B, bias, stages=w["stages"], guards=False)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    s = oracle.compare(C1[rows], oracle.gemm_bias_relu_rows(A, B, bias, rows))
    assert oracle.within_tolerance(s, "fp32"), s


def test_deep_k_default(gpu):
    """1024 x 1024 x 16384 by default: 32 tiles of 256 x 128 whose 512 k steps each are shared by every
    CU; integer inputs exact on rows of every tile row, and repeatable."""
    M, N, K = 1024, 1024, 16384
    A, B, bias = int_case(6700, M, N, K)
    C = run_gemm(gpu, A, B, bias, stages=2)
    rows = stratified_rows(M, 256, 5)
    assert np.array_equal(C[rows].astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))
    C2 = run_gemm(gpu, A, B, bias, stages=2, guards=False)
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32))
