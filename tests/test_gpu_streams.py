"""GEMMs and staged copies launched on two streams at once: each launch is
independent (its ring lives in its workgroups' LDS), so concurrent launches
must give the same results as serial ones, and the shared device status word
must stay clear."""
import numpy as np
import pytest

import oracle
from test_gpu_gemm_bf16 import int_case as int_bf16
from test_gpu_gemm_fp32 import int_case as int_f32

pytestmark = pytest.mark.gpu


def test_concurrent_gemms_and_copies(gpu):
    import torch
    M, N, K = 640, 768, 520
    A, B, bias = int_f32(71, M, N, K)
    Ab, Bb, bb = int_bf16(72, M, N, 520)
    ref = oracle.gemm_bias_relu(A, B, bias)
    refb = oracle.gemm_bias_relu(Ab, Bb, bb)
    dA, dB, db = (torch.from_numpy(x).cuda() for x in (A, B, bias))
    dAb, dBb, dbb = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda() for x in (Ab, Bb, bb))
    src = torch.randint(-2**31, 2**31 - 1, ((1 << 24) // 4,), dtype=torch.int32, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, outsb, copies = [], [], []
    torch.cuda.synchronize()
    for i in range(12):
        with torch.cuda.stream(streams[i % 2]):
            outs.append(gpu.gemm_bias_relu(dA, dB, db, stages=2 + i % 3))
            outsb.append(gpu.gemm_bias_relu_bf16(dAb, dBb, dbb, stages=2 + i % 2))
            copies.append(gpu.staged_copy(src, stages=2))
    torch.cuda.synchronize()
    gpu.check_device_status()
    for o in outs:
        assert np.array_equal(o.cpu().numpy().astype(np.float64), ref)
    for o in outsb:
        assert np.array_equal(o.cpu().numpy().astype(np.float64), refb)
    for c in copies:
        assert torch.equal(c, src)
