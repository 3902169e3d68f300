"""The ring handshake's wait counters: exact counts, and the pages' steady state."""
import numpy as np
import pytest

import synth
from conftest import say

pytestmark = pytest.mark.gpu


def test_gemm_wait_counts_match_protocol(gpu):
    import torch
    M, N, K = 512, 512, 1024
    cfg = dict(BM=256, BN=128, BK=32, producer_waves=2, consumer_waves=8)
    A = torch.from_numpy(synth.uniform_pm1(1, M * K).reshape(M, K)).cuda()
    B = torch.from_numpy(synth.uniform_pm1(2, K * N).reshape(K, N)).cuda()
    b = torch.from_numpy(synth.uniform_pm1(3, N)).cuda()
    gpu.read_wait_stats()  # clear
    gpu.set_wait_stats(True)
    try:
        say("gemm wait stats %dx%dx%d %s" % (M, N, K, cfg))
        gpu.gemm_bias_relu_ex(A, B, b, stages=2, config=cfg)
        st = gpu.read_wait_stats()
    finally:
        gpu.set_wait_stats(False)
    wgs, T = (M // 256) * (N // 128), K // 32
    assert st["gemm_consumer_full"]["waits"] == wgs * 8 * T
    assert st["gemm_producer_empty"]["waits"] == wgs * 2 * T
    for k in ("gemm_consumer_full", "gemm_producer_empty"):
        assert st[k]["blocked"] <= st[k]["waits"]
        assert (st[k]["polls"] == 0) == (st[k]["blocked"] == 0)
    assert st["copy_consumer_full"]["waits"] == 0
    # with statistics off nothing is counted
    gpu.gemm_bias_relu_ex(A, B, b, stages=2, config=cfg)
    assert gpu.read_wait_stats()["gemm_consumer_full"]["waits"] == 0


@pytest.mark.parametrize("M,N,K,flags", [(700, 900, 660, 16), (1024, 1024, 16384, 0)])
def test_stream_k_wait_counts_match_protocol(gpu, M, N, K, flags):
    """A stream-K launch (forced, or by default for a deep K) walks every k tile of every output tile
    through the ring exactly once, whatever the split: one full wait per consumer wave and one empty
    wait per producer wave for each of them, as the one-workgroup-per-tile launch."""
    import torch
    cfg = dict(BM=256, BN=128, BK=32, producer_waves=4, consumer_waves=4, flags=flags)
    assert gpu.resolve_config(gpu.WSG_FP32, M, N, K, 2, cfg)["flags"] & 16  # WSG_FLAG_STREAM_K
    A = torch.from_numpy(synth.uniform_pm1(4, M * K).reshape(M, K)).cuda()
    B = torch.from_numpy(synth.uniform_pm1(5, K * N).reshape(K, N)).cuda()
    b = torch.from_numpy(synth.uniform_pm1(6, N)).cuda()
    gpu.read_wait_stats()  # clear
    gpu.set_wait_stats(True)
    try:
        say("stream-K wait stats %dx%dx%d %s" % (M, N, K, cfg))
        gpu.gemm_bias_relu_ex(A, B, b, stages=2, config=cfg)
        st = gpu.read_wait_stats()
    finally:
        gpu.set_wait_stats(False)
    steps = -(-M // 256) * -(-N // 128) * -(-K // 32)
    assert st["gemm_consumer_full"]["waits"] == 4 * steps
    assert st["gemm_producer_empty"]["waits"] == 4 * steps
    for k in ("gemm_consumer_full", "gemm_producer_empty"):
        assert st[k]["blocked"] <= st[k]["waits"]


def test_copy_wait_counts_match_protocol(gpu):
    import torch
    tile = 16384
    ntiles = 256 * 5 + 3
    src = torch.from_numpy(synth.splitmix64(9, ntiles * tile // 8).view(np.uint8)).cuda()
    gpu.read_wait_stats()
    gpu.set_wait_stats(True)
    try:
        say("copy wait stats %d tiles" % ntiles)
        dst = gpu.staged_copy_ex(src, stages=8, config=dict(copy_tile_bytes=tile, producer_waves=2,
                                                            consumer_waves=2, flags=2))
        st = gpu.read_wait_stats()
    finally:
        gpu.set_wait_stats(False)
    assert torch.equal(dst, src)
    assert st["copy_consumer_full"]["waits"] == ntiles * 2
    assert st["copy_producer_empty"]["waits"] == ntiles * 2


@pytest.mark.parametrize("D,consumers", [(64, 4), (128, 7)])
def test_attention_wait_counts_match_protocol(gpu, D, consumers):
    """Attention consumers wait once per key tile (64 keys) each; the binding reports their counters."""
    import torch
    Bn, H, Sq, Skv = 1, 2, 300, 200
    dev = lambda seed, s: torch.from_numpy(synth.normal_bf16_bits(seed, int(np.prod(s)), scale=1.0)  # noqa: E731
                                           .reshape(s).view(np.int16)).cuda()
    q, k, v = dev(31, (Bn, H, Sq, D)), dev(32, (Bn, H, Skv, D)), dev(33, (Bn, H, Skv, D))
    gpu.read_wait_stats()
    gpu.set_wait_stats(True)
    try:
        say("attention wait stats D=%d consumers=%d" % (D, consumers))
        gpu.attention_fwd(q, k, v, stages=2, config=dict(producer_waves=1, consumer_waves=consumers))
        st = gpu.read_wait_stats()
    finally:
        gpu.set_wait_stats(False)
    q_tiles = -(-Sq // (32 * consumers))
    key_tiles = -(-Skv // 64)
    a = st["attention_consumer_full"]
    assert a["waits"] == Bn * H * q_tiles * consumers * key_tiles, a
    assert a["blocked"] <= a["waits"]
    assert st["gemm_consumer_full"]["waits"] == 0 and st["copy_consumer_full"]["waits"] == 0
