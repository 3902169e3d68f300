"""Size limits on the GPU: operands past 2^31 and 2^32 bytes, and the deepest rings.

The LDS-DMA producers and the buffer-store epilogues address a tile's rows
with 32-bit offsets under a buffer resource whose range is capped at 2^31 - 1
bytes; the planner switches to kernels with 64-bit addressing where a tile's
rows would span more. Each GEMM case sits on one side of such a threshold,
with integer inputs whose sums stay below 2^24, so the result must match the
oracle bit for bit on rows of every tile row. The copy moves more than 4 GiB,
so its byte offsets pass 2^31 and 2^32; attention and the grouped GEMM take
operands past 2^31 bytes, whose per-head and per-expert bases are 64-bit. The
ring cases run the deepest ring that fits in LDS and check that one slot more
is refused.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows
from oracle import attention as att

pytestmark = pytest.mark.gpu

GENERAL_PRODUCER, STREAM_K = 1, 16  # WSG_FLAG_GENERAL_PRODUCER, WSG_FLAG_STREAM_K
LDS_BYTES, FLAG_BYTES = 163840, 256  # LDS a workgroup may use on gfx950; the ring's flag words


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _fp32_ones_case(seed, M, N, K):
    # entries in {-1, 0, 1}: every partial sum of a row is an integer of at most K < 2^24 in magnitude
    return (synth.small_int_f32(seed + 1, M * K, -1, 1).reshape(M, K),
            synth.small_int_f32(seed + 2, K * N, -1, 1).reshape(K, N),
            synth.small_int_f32(seed + 3, N, -8, 8))


def _run_fp32_rows(gpu, A, B, bias, rows):
    import torch
    M, K = A.shape
    N = B.shape[1]
    dA, dB, db = (torch.from_numpy(x).cuda() for x in (A, B, bias))
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    say("gemm fp32 M=%d N=%d K=%d default launch" % (M, N, K))
    gpu.gemm_bias_relu(dA, dB, db, dC)
    gpu.check_device_status()
    assert not bool(torch.isnan(dC).any()), "an output element was not written"
    out = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
    del dA, dB, db, dC
    _free()
    return out


def test_fp32_a_rows_just_below_31_bits(gpu):
    """256 rows of A span 2^31 - 8192 bytes: the LDS-DMA producer with its
    largest offsets, and the deep K split by stream-K over every CU."""
    M, N, K = 260, 24, (1 << 21) - 4
    cfg = gpu.resolve_config(gpu.WSG_FP32, M, N, K)
    assert (cfg["BM"], cfg["BN"]) == (256, 128) and not cfg["flags"] & GENERAL_PRODUCER
    assert cfg["flags"] & STREAM_K
    A, B, bias = _fp32_ones_case(7100, M, N, K)
    rows = np.unique(np.concatenate([stratified_rows(M, 256, 3), [128, 254, 257, 258]]))
    got = _run_fp32_rows(gpu, A, B, bias, rows)
    assert np.array_equal(got.astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))


def test_fp32_a_rows_past_31_bits(gpu):
    """256 rows of A span more than 2^31 bytes: the register-staged producer
    (64-bit element offsets), one workgroup per tile."""
    M, N, K = 257, 24, (1 << 21) + 4
    cfg = gpu.resolve_config(gpu.WSG_FP32, M, N, K)
    assert cfg["flags"] & GENERAL_PRODUCER and not cfg["flags"] & STREAM_K
    A, B, bias = _fp32_ones_case(7200, M, N, K)
    rows = np.unique(np.concatenate([stratified_rows(M, cfg["BM"], 5), [129, 255]]))
    got = _run_fp32_rows(gpu, A, B, bias, rows)
    assert np.array_equal(got.astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))


@pytest.mark.parametrize("N,lean", [((1 << 21) - 8, True), ((1 << 21) + 8, False)])
def test_bf16_c_rows_around_31_bits(gpu, N, lean):
    """256 rows of C just below 2^31 bytes keep the 12-wave 256 x 256 kernels,
    whose epilogue stores through a buffer resource at the tile's origin; past
    it the planner takes a 256 x 128 kernel with 64-bit store addresses."""
    import torch
    M, K = 300, 64
    cfg = gpu.resolve_config(gpu.WSG_BF16, M, N, K)
    if lean:
        assert (cfg["BM"], cfg["BN"]) == (256, 256) and cfg["producer_waves"] + cfg["consumer_waves"] == 12
    else:
        assert (cfg["BM"], cfg["BN"]) == (256, 128) and cfg["producer_waves"] + cfg["consumer_waves"] <= 8
    A = synth.small_int_bf16_bits(7301, M * K, -3, 3).reshape(M, K)
    B = synth.small_int_bf16_bits(7302 + N % 7, K * N, -3, 3).reshape(K, N)
    bias = synth.small_int_bf16_bits(7303, N, -8, 8)
    dA, dB, db = (torch.from_numpy(x.view(np.int16)).cuda() for x in (A, B, bias))
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    say("gemm bf16 M=%d N=%d K=%d default launch" % (M, N, K))
    gpu.gemm_bias_relu_bf16(dA, dB, db, dC)
    gpu.check_device_status()
    assert not bool(torch.isnan(dC).any()), "an output element was not written"
    rows = np.unique(np.concatenate([stratified_rows(M, 256, 1), [131, 256, 299]]))
    got = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
    del dA, dB, db, dC
    _free()
    assert np.array_equal(got.astype(np.float64), oracle.gemm_bias_relu_rows(A, B, bias, rows))


def test_copy_past_4_gib(gpu):
    """(2^32 + 3 * 64 Ki + 7) bytes, staged and unstaged: the whole buffer
    equal to the source, windows at 0, 2^31, 2^32 and the tail against the
    oracle, guard bands intact."""
    import torch
    n = (1 << 32) + 3 * 65536 + 7
    guard = 4096
    src_np = synth.splitmix64(7400, (n + 7) // 8).view(np.uint8)[:n]
    src = torch.from_numpy(src_np).cuda()
    buf = torch.empty((n + 2 * guard,), dtype=torch.uint8, device="cuda")
    dst = buf[guard:guard + n]
    windows = [(0, 1 << 20), ((1 << 31) - (1 << 19), (1 << 31) + (1 << 19)),
               ((1 << 32) - (1 << 19), (1 << 32) + (1 << 19)), (n - (1 << 20), n)]
    for name, config in (("staged", None), ("unstaged", dict(flags=8))):  # WSG_FLAG_DIRECT_COPY
        buf.fill_(0xA5)
        say("%s copy bytes=%d" % (name, n))
        if config is None:
            gpu.staged_copy(src, dst, stages=2)
        else:
            gpu.staged_copy_ex(src, dst, stages=2, config=config)
        gpu.check_device_status()
        assert bool(torch.equal(dst, src)), name
        assert bool((buf[:guard] == 0xA5).all()) and bool((buf[guard + n:] == 0xA5).all()), "guard band written"
        for a, b in windows:
            got = dst[a:b].cpu().numpy()
            assert oracle.first_mismatch(got, oracle.copy(src_np[a:b])) == -1, (name, a)
    del src, buf, dst
    _free()


def _copy_bits(seed, n):
    return synth.splitmix64(seed, (n + 7) // 8).view(np.uint8)[:n].copy()


def test_copy_deepest_ring(gpu):
    """32 slots of 4 KiB (the flag area's limit) over several laps; a 33rd slot is refused."""
    import torch
    config = dict(copy_tile_bytes=4096, producer_waves=1, consumer_waves=1)
    n = 256 * 70 * 4096 + 4321
    src_np = _copy_bits(7500, n)
    src = torch.from_numpy(src_np).cuda()
    dst = torch.zeros_like(src)
    say("staged copy bytes=%d stages=32" % n)
    gpu.staged_copy_ex(src, dst, stages=32, config=config)
    gpu.check_device_status()
    assert oracle.first_mismatch(dst.cpu().numpy(), oracle.copy(src_np)) == -1
    with pytest.raises(gpu.WsgError) as e:
        gpu.staged_copy_ex(src, dst, stages=33, config=config)
    assert e.value.code == gpu.WSG_EUNSUPPORTED


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_gemm_deepest_ring(gpu, dtype):
    """64 x 64 tiles (8 KiB slots): the deepest ring that fits in LDS, over
    several laps, bit-exact; one slot more is refused."""
    import torch
    M, N, K = 300, 200, 16 * 50 + 8
    config = dict(BM=64, BN=64, BK=16 if dtype == "fp32" else 32, producer_waves=1, consumer_waves=4)
    es = 4 if dtype == "fp32" else 2
    slot = (config["BM"] + config["BN"]) * config["BK"] * es
    deepest = (LDS_BYTES - FLAG_BYTES) // slot
    assert deepest == 19
    if dtype == "fp32":
        A = synth.small_int_f32(7601, M * K, -3, 3).reshape(M, K)
        B = synth.small_int_f32(7602, K * N, -3, 3).reshape(K, N)
        bias = synth.small_int_f32(7603, N, -8, 8)
        dev = [torch.from_numpy(x).cuda() for x in (A, B, bias)]
    else:
        A = synth.small_int_bf16_bits(7611, M * K, -3, 3).reshape(M, K)
        B = synth.small_int_bf16_bits(7612, K * N, -3, 3).reshape(K, N)
        bias = synth.small_int_bf16_bits(7613, N, -8, 8)
        dev = [torch.from_numpy(x.view(np.int16)).cuda() for x in (A, B, bias)]
    say("gemm %s M=%d N=%d K=%d stages=%d config=%s" % (dtype, M, N, K, deepest, config))
    C = gpu.gemm_bias_relu_ex(*dev, stages=deepest, config=config)
    gpu.check_device_status()
    assert np.array_equal(C.cpu().numpy().astype(np.float64), oracle.gemm_bias_relu(A, B, bias))
    with pytest.raises(gpu.WsgError) as e:
        gpu.gemm_bias_relu_ex(*dev, stages=deepest + 1, config=config)
    assert e.value.code == gpu.WSG_EUNSUPPORTED


def _pooled(pool, count):
    """Blocks 0 .. count - 1 where block i is pool[i mod len(pool)], built on the GPU."""
    import torch
    d = torch.from_numpy(np.ascontiguousarray(pool).view(np.int16)).cuda()
    return d.index_select(0, torch.arange(count, device="cuda") % d.shape[0])


def test_attention_past_2_gib(gpu):
    """2 x 4100 heads of 1024 queries and keys, head dimension 128: Q, K and V
    pass 2^31 bytes at head 8192, O (fp32) at head 4096 and 2^32 bytes at
    head 8192. Head i of Q, K and V repeats seeded pools of 61, 59 and 53
    heads; none of those periods divides 4096 or 8192, so a head read from
    or written to a wrapped offset would not match the oracle."""
    import torch
    Bn, H, S, D = 2, 4100, 1024, 128
    heads = Bn * H
    pools = [synth.normal_bf16_bits(7700 + i, p * S * D, scale=1.0).reshape(p, S, D)
             for i, p in enumerate((61, 59, 53))]
    dQ, dK, dV = (_pooled(p, heads).view(Bn, H, S, D) for p in pools)
    dO = torch.empty((Bn, H, S, D), dtype=torch.float32, device="cuda")
    flat_heads = [0, 4095, 4096, 4100, 8191, 8192, heads - 1]
    rows = np.array([0, 223, 224, 611, S - 1])
    scale = 1.0 / math.sqrt(D)
    for causal in (False, True):
        dO.fill_(float("nan"))
        say("attention %s causal=%s default launch" % ((Bn, H, S, D), causal))
        gpu.attention_fwd(dQ, dK, dV, dO, causal=causal)
        gpu.check_device_status()
        assert not bool(torch.isnan(dO).any()), "an output element was not written"
        got, ref = [], []
        for f in flat_heads:
            got.append(dO[f // H, f % H, torch.from_numpy(rows).cuda()].cpu().numpy())
            q, k, v = (p[f % p.shape[0]][None, None] for p in pools)
            ref.append(att.attention_rows(q, k, v, scale, causal, 0, 0, rows))
        s = oracle.compare(np.concatenate(got), np.concatenate(ref))
        assert oracle.within_tolerance(s, "bf16"), (causal, s)
    del dQ, dK, dV, dO
    _free()


def test_grouped_weights_past_2_gib(gpu):
    """16 experts of 8192 x 8200 bf16 weights (2.0 GiB in all; the last
    expert's block crosses 2^31 bytes), uneven row counts with an empty
    expert, integer inputs: rows of every expert bit-exact."""
    import torch
    E, K, N = 16, 8192, 8200
    group_rows = [37, 0, 300, 5, 256, 1, 90, 257, 12, 64, 3, 128, 40, 7, 200, 33]
    M = sum(group_rows)
    A = synth.small_int_bf16_bits(7801, M * K, -2, 2).reshape(M, K)
    B = synth.small_int_bf16_bits(7802, E * K * N, -2, 2).reshape(E, K, N)
    bias = synth.small_int_bf16_bits(7803, E * N, -8, 8).reshape(E, N)
    dA, dB, db = (torch.from_numpy(x.view(np.int16)).cuda() for x in (A, B, bias))
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    say("grouped gemm bf16 experts=%d K=%d N=%d rows=%d default launch" % (E, K, N, M))
    gpu.grouped_gemm_bias_relu_ex(dA, dB, db, group_rows, dC)
    gpu.check_device_status()
    assert not bool(torch.isnan(dC).any()), "an output element was not written"
    starts = np.cumsum([0] + group_rows[:-1])
    rows = np.unique(np.concatenate([[s, s + r // 2, s + r - 1] for s, r in zip(starts, group_rows) if r > 0]))
    got = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
    del dA, dB, db, dC
    _free()
    want = oracle.grouped_gemm_bias_relu_rows(A, B, bias, group_rows, rows)
    assert np.array_equal(got.astype(np.float64), want)
