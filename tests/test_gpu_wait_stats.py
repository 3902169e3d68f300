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
