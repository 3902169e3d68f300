"""gemm_bias_relu_ex_noalloc (the entry point for callers that cannot allocate
device memory) against gemm_bias_relu_ex: the same kernels, so the same bits,
on consecutive calls that reuse the per-device scratch array, the second
smaller than the first."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from conftest import say
from test_gpu_gemm_fp32 import int_case

pytestmark = pytest.mark.gpu

STREAM_K, NO_STREAM_K = 16, 32  # WSG_FLAG_STREAM_K, WSG_FLAG_NO_STREAM_K


def _both(gpu, dtype, A, B, bias, stages, config):
    """One call of each entry point through the C ABI on the same device
    operands; returns (noalloc C, ex C) as numpy arrays."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    C_na = torch.full((M, N), -7.0, dtype=torch.float32, device="cuda")
    C_ex = torch.full((M, N), -9.0, dtype=torch.float32, device="cuda")
    cfg = gpu.Config(**config) if config else None
    ptr = ctypes.byref(cfg) if cfg is not None else None
    say("noalloc dtype=%d M=%d N=%d K=%d stages=%d config=%s" % (dtype, M, N, K, stages, config))
    rc = gpu.lib.gemm_bias_relu_ex_noalloc(dtype, M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(),
                                           C_na.data_ptr(), stages, ptr)
    assert rc == gpu.WSG_OK, gpu.last_error()
    torch.cuda.synchronize()
    gpu.check_device_status()
    rc = gpu.lib.gemm_bias_relu_ex(dtype, M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C_ex.data_ptr(),
                                   stages, ptr)
    assert rc == gpu.WSG_OK, gpu.last_error()
    torch.cuda.synchronize()
    gpu.check_device_status()
    return C_na.cpu().numpy(), C_ex.cpu().numpy()


def _dev(*xs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in xs]


def test_two_calls_second_smaller(gpu):
    # 1: the ragged 3000 x 5000 x 4100 fp32 workload, stream-K tail by default
    M, N, K = 3000, 5000, 4100
    assert gpu.resolve_config(gpu.WSG_FP32, M, N, K, 2)["flags"] & STREAM_K
    A = synth.uniform_pm1(synth.seed_for(4, "A"), M * K).reshape(M, K)
    B = synth.uniform_pm1(synth.seed_for(4, "B"), K * N).reshape(K, N)
    bias = synth.uniform_pm1(synth.seed_for(4, "bias"), N)
    na, ex = _both(gpu, gpu.WSG_FP32, *_dev(A, B, bias), 2, None)
    assert np.array_equal(na.view(np.uint32), ex.view(np.uint32))
    rows = np.array([0, 1, 255, 256, 1500, 2047, 2999])
    s = oracle.compare(na[rows], oracle.gemm_bias_relu_rows(A, B, bias, rows))
    assert oracle.within_tolerance(s, "fp32"), s

    # 2: smaller, forced stream-K with small tiles (more workgroups, other slots)
    M, N, K = 700, 900, 660
    A, B, bias = int_case(7100, M, N, K)
    config = dict(BM=64, BN=64, BK=16, producer_waves=1, consumer_waves=4, flags=STREAM_K)
    na, ex = _both(gpu, gpu.WSG_FP32, *_dev(A, B, bias), 2, config)
    assert np.array_equal(na.view(np.uint32), ex.view(np.uint32))
    assert np.array_equal(na.astype(np.float64), oracle.gemm_bias_relu(A, B, bias))


def test_every_stream_k_tile_fits_and_matches(gpu):
    """Each fp32 tile shape with a stream-K kernel, forced, then a launch with
    no stream-K tail and a bf16 launch (neither uses the scratch array)."""
    M, N, K = 600, 700, 16 * 31 + 4
    A, B, bias = int_case(7200, M, N, K)
    dA, dB, db = _dev(A, B, bias)
    ref = oracle.gemm_bias_relu(A, B, bias)
    tiles = [(256, 128, 32, 4, 4), (256, 128, 16, 4, 4), (256, 128, 32, 2, 4), (256, 128, 16, 2, 4),
             (128, 128, 32, 2, 4), (128, 128, 16, 1, 4), (128, 128, 16, 2, 4), (64, 64, 16, 1, 4),
             (256, 128, 32, 1, 4), (256, 128, 32, 2, 8), (256, 128, 16, 2, 8), (256, 128, 32, 1, 8),
             (256, 128, 16, 1, 8), (256, 128, 32, 4, 8), (128, 256, 16, 2, 8)]
    for BM, BN, BK, P, C in tiles:
        config = dict(BM=BM, BN=BN, BK=BK, producer_waves=P, consumer_waves=C, flags=STREAM_K)
        assert gpu.resolve_config(gpu.WSG_FP32, M, N, K, 2, config)["flags"] & STREAM_K
        na, ex = _both(gpu, gpu.WSG_FP32, dA, dB, db, 2, config)
        assert np.array_equal(na.view(np.uint32), ex.view(np.uint32)), config
        assert np.array_equal(na.astype(np.float64), ref), config
    na, ex = _both(gpu, gpu.WSG_FP32, dA, dB, db, 3, dict(flags=NO_STREAM_K))
    assert np.array_equal(na.astype(np.float64), ref) and np.array_equal(na, ex)

    from test_gpu_gemm_bf16 import int_case as int_bf16
    Ab, Bb, bb = int_bf16(7300, 300, 520, 200)
    dAb, dBb, dbb = _dev(*(np.ascontiguousarray(x).view(np.int16) for x in (Ab, Bb, bb)))
    na, ex = _both(gpu, gpu.WSG_BF16, dAb, dBb, dbb, 4, None)
    assert np.array_equal(na.astype(np.float64), oracle.gemm_bias_relu(Ab, Bb, bb)) and np.array_equal(na, ex)


def test_binding_requires_output(gpu):
    import torch
    A = torch.zeros((8, 8), device="cuda")
    b = torch.zeros((8,), device="cuda")
    with pytest.raises(ValueError):
        gpu.gemm_bias_relu_ex_noalloc(A, A, b, None)
    C = torch.full((8, 8), -1.0, device="cuda")
    gpu.gemm_bias_relu_ex_noalloc(A, A, b, C)
    assert torch.equal(C, torch.zeros_like(C))


def test_graph_capture_replays(gpu):
    """The caller this entry point is for: a HIP graph that captures it (counter clearing and the
    stream-K launch included) is replayed three times, with the program's own eager work and
    synchronizations between replays; every replay equals the eager result."""
    import torch
    M, N, K = 3000, 5000, 4100  # a stream-K tail by default
    assert gpu.resolve_config(gpu.WSG_FP32, M, N, K, 2)["flags"] & STREAM_K
    A = synth.uniform_pm1(synth.seed_for(4, "A"), M * K).reshape(M, K)
    B = synth.uniform_pm1(synth.seed_for(4, "B"), K * N).reshape(K, N)
    bias = synth.uniform_pm1(synth.seed_for(4, "bias"), N)
    dA, dB, db = _dev(A, B, bias)
    C_eager = torch.empty((M, N), dtype=torch.float32, device="cuda")
    gpu.gemm_bias_relu_ex_noalloc(dA, dB, db, C_eager, stages=2)  # also does the one-time set-up
    torch.cuda.synchronize()
    gpu.check_device_status()
    C = torch.empty_like(C_eager)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    say("capture gemm_bias_relu_ex_noalloc M=%d N=%d K=%d" % (M, N, K))
    with torch.cuda.graph(graph, stream=side):
        gpu.gemm_bias_relu_ex_noalloc(dA, dB, db, C, stages=2)
    Ai, Bi, bi = int_case(7400, 700, 900, 660)
    dAi, dBi, dbi = _dev(Ai, Bi, bi)
    Ci = torch.empty((700, 900), dtype=torch.float32, device="cuda")
    for i in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gpu.check_device_status()
        assert torch.equal(C, C_eager), "replay %d" % i
        # eager work on the same scratch array between replays
        gpu.gemm_bias_relu_ex_noalloc(dAi, dBi, dbi, Ci, stages=2, config=dict(flags=STREAM_K))
        torch.cuda.synchronize()
        assert np.array_equal(Ci.cpu().numpy().astype(np.float64), oracle.gemm_bias_relu(Ai, Bi, bi))
