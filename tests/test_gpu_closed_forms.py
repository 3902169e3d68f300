"""Closed forms and the reflection identity of C = relu(A @ B + bias) on the GPU.

The operator is the SGEMM with a bias + ReLU epilogue of the pwwt.cn article on
intra-kernel pipelining (section 4.1). Its closed forms hold exactly:
  A = I (M = K)      -> C = relu(B + bias)
  B = I (K = N)      -> C = relu(A + bias)
  A = 0 or B = 0     -> C = relu(bias) on every row
  A = B = all ones   -> C = relu(K + bias)
In each, the K-sum is exact in fp32 (one nonzero term, or an integer below
2^24), so the only rounding is the one fp32 addition of the bias: the GPU
must return the fp32 rounding of the fp64 oracle, bit for bit.

Reflection: relu(x) - relu(-x) = x, and negating A and bias negates every
product and partial sum exactly (round-to-nearest-even is symmetric), so
C(A, B, b) - C(-A, B, -b) is the GPU's own pre-activation, and at most one of
the two outputs is nonzero at each element. The pre-activation is then
compared with the oracle's within the fp32 / bf16 tolerance, which checks the
half of the result that the ReLU hides.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import say

pytestmark = pytest.mark.gpu

BF16_ONE = np.uint16(0x3F80)


def _dev(x):
    import torch
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x if x.dtype == np.float32 else x.view(np.int16)).cuda()


def _run(gpu, A, B, bias, stages, config):
    import torch
    M, N = A.shape[0], B.shape[1]
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("closed form %s M=%d N=%d K=%d stages=%d config=%s" % (A.dtype, M, N, A.shape[1], stages, config))
    if config is None and A.dtype == np.float32:
        gpu.gemm_bias_relu(_dev(A), _dev(B), _dev(bias), C, stages=stages)
    elif config is None:
        gpu.gemm_bias_relu_bf16(_dev(A), _dev(B), _dev(bias), C, stages=stages)
    else:
        gpu.gemm_bias_relu_ex(_dev(A), _dev(B), _dev(bias), C, stages=stages, config=config)
    gpu.check_device_status()
    return C.cpu().numpy()


def _values(dtype, seed, n):
    if dtype == "fp32":
        return synth.uniform_pm1(seed, n)
    return synth.normal_bf16_bits(seed, n)


def _eye(dtype, n):
    if dtype == "fp32":
        return np.eye(n, dtype=np.float32)
    e = np.zeros((n, n), dtype=np.uint16)
    e[np.arange(n), np.arange(n)] = BF16_ONE
    return e


def _fill(dtype, shape, one):
    if dtype == "fp32":
        return np.full(shape, 1.0 if one else 0.0, dtype=np.float32)
    return np.full(shape, BF16_ONE if one else 0, dtype=np.uint16)


def _neg(x):
    return -x if x.dtype == np.float32 else x ^ np.uint16(0x8000)


def _widen(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x


# (dtype, size, stages, config): the 256^3 workload in its 64x64x16 two-stage configuration, the
# default launch at 256^3, and ragged squares on the LDS-DMA producer (K a multiple of 16 bytes)
# and on the register-staged producer (K not)
CASES = [
    ("fp32", 256, 2, dict(BM=64, BN=64, BK=16)),
    ("fp32", 256, 2, None),
    ("fp32", 300, 3, None),
    ("fp32", 301, 2, None),
    ("bf16", 256, 4, None),
    ("bf16", 296, 4, None),
    ("bf16", 300, 2, None),
]


def _cid(c):
    return "%s_%d_s%d_%s" % (c[0], c[1], c[2], "cfg" if c[3] else "default")


@pytest.mark.parametrize("case", CASES, ids=_cid)
def test_closed_forms_bit_exact(gpu, case):
    dtype, n, stages, config = case
    X = _values(dtype, 9100 + n, n * n).reshape(n, n)
    bias = _values(dtype, 9200 + n, n)
    forms = {
        "A=I": (_eye(dtype, n), X, relu_f32(_widen(X) + _widen(bias)[None, :])),
        "B=I": (X, _eye(dtype, n), relu_f32(_widen(X) + _widen(bias)[None, :])),
        "A=0": (_fill(dtype, (n, n), False), X, np.broadcast_to(relu_f32(_widen(bias)), (n, n))),
        "B=0": (X, _fill(dtype, (n, n), False), np.broadcast_to(relu_f32(_widen(bias)), (n, n))),
        "ones": (_fill(dtype, (n, n), True), _fill(dtype, (n, n), True),
                 np.broadcast_to(relu_f32(np.float32(n) + _widen(bias)), (n, n))),
    }
    for name, (A, B, closed) in forms.items():
        C = _run(gpu, A, B, bias, stages, config)
        ref32 = oracle.gemm_bias_relu(A, B, bias).astype(np.float32)
        assert np.array_equal(C.view(np.uint32), ref32.view(np.uint32)), name
        assert np.array_equal(C.view(np.uint32), np.ascontiguousarray(closed).view(np.uint32)), name


def relu_f32(x):
    """max(x, +0) in fp32 (one fp32 rounding of x, then the ReLU; -0 -> +0)."""
    x = np.asarray(x, dtype=np.float32)
    return np.where(x > 0, x, np.float32(0.0)).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=_cid)
def test_reflection_recovers_the_pre_activation(gpu, case):
    dtype, n, stages, config = case
    # several tiles, ragged in every dimension; rows of a multiple of 16 bytes keep the LDS-DMA
    # producer, odd sizes take the register-staged one (as the closed-form case of this size does)
    dma = n % 8 == 0 or (dtype == "fp32" and n % 4 == 0)
    M, N, K = (n, n + 40, n + 8) if dma else (n, n + 37, n + 11)
    A = _values(dtype, 9300 + n, M * K).reshape(M, K)
    B = _values(dtype, 9400 + n, K * N).reshape(K, N)
    bias = _values(dtype, 9500 + n, N)
    Cp = _run(gpu, A, B, bias, stages, config)
    Cn = _run(gpu, _neg(A), B, _neg(bias), stages, config)
    assert np.all(Cp >= 0) and np.all(Cn >= 0)
    assert not np.any((Cp > 0) & (Cn > 0)), "a pre-activation and its negation both positive"
    x_gpu = Cp.astype(np.float64) - Cn.astype(np.float64)
    x_ref = oracle.gemm_bias_relu(A, B, bias) - oracle.gemm_bias_relu(_neg(A), B, _neg(bias))
    s = oracle.compare(x_gpu, x_ref)
    assert oracle.within_tolerance(s, dtype), s
    # C is zero exactly where the oracle's pre-activation is clearly negative, positive where clearly positive
    tol = oracle.TOL[dtype][0]
    assert np.all(Cp[x_ref < -tol] == 0) and np.all(Cp[x_ref > tol] > 0)
