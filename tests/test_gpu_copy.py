"""Staged copy on the GPU against the oracle: bit-exact, guard bands intact."""
import numpy as np
import pytest

import oracle
import synth
from conftest import say

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5


def _run_copy(gpu, src_np, stages, config=None):
    import torch
    n = src_np.nbytes
    src = torch.from_numpy(src_np.view(np.uint8).reshape(-1).copy()).cuda()
    # dst sits between two guard bands of sentinel bytes
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    dst = buf[GUARD:GUARD + n]
    say("staged_copy bytes=%d stages=%d config=%s" % (n, stages, config))
    if config is None:
        gpu.staged_copy(src, dst, stages=stages)
    else:
        gpu.staged_copy_ex(src, dst, stages=stages, config=config)
    gpu.check_device_status()
    out = buf.cpu().numpy()
    want = oracle.copy(src_np.view(np.uint8).reshape(-1))
    assert oracle.first_mismatch(out[GUARD:GUARD + n], want) == -1
    assert np.all(out[:GUARD] == SENTINEL) and np.all(out[GUARD + n:] == SENTINEL), "guard band written"


def _bytes(seed, n):
    return synth.splitmix64(seed, (n + 7) // 8).view(np.uint8)[:n].copy()


@pytest.mark.parametrize("n", [1, 3, 15, 16, 17, 1000, 4095, 65535, 65536, 65537, 131072 + 5, 3 * 65536 - 7])
@pytest.mark.parametrize("stages", [1, 2])
def test_copy_sizes(gpu, n, stages):
    _run_copy(gpu, _bytes(100 + n, n), stages)


@pytest.mark.parametrize("config,stages", [
    (dict(copy_tile_bytes=65536, producer_waves=2, consumer_waves=2), 2),
    (dict(copy_tile_bytes=65536, producer_waves=8, consumer_waves=8), 2),
    (dict(copy_tile_bytes=65536, producer_waves=4, consumer_waves=8), 2),
    (dict(copy_tile_bytes=32768, producer_waves=4, consumer_waves=4), 4),
    (dict(copy_tile_bytes=32768, producer_waves=2, consumer_waves=2), 3),
    (dict(copy_tile_bytes=16384, producer_waves=2, consumer_waves=2), 8),
    (dict(copy_tile_bytes=16384, producer_waves=1, consumer_waves=1), 5),
    (dict(copy_tile_bytes=4096, producer_waves=1, consumer_waves=1), 16),
    (dict(copy_tile_bytes=16384, producer_waves=1, consumer_waves=1, flags=2), 8),
    (dict(copy_tile_bytes=8192, producer_waves=1, consumer_waves=1, flags=2), 16),
    (dict(copy_tile_bytes=65536, producer_waves=4, consumer_waves=4, flags=2), 2),
    (dict(copy_tile_bytes=32768, producer_waves=2, consumer_waves=2, flags=2), 4),
])
def test_copy_configs_multi_lap(gpu, config, stages):
    # enough tiles that every workgroup laps its ring several times, plus a ragged tail
    n = 256 * 6 * config["copy_tile_bytes"] + 12345
    _run_copy(gpu, _bytes(7 + stages, n), stages, config)


@pytest.mark.parametrize("workgroups", [1, 3, 100, 192, 100000])
def test_copy_explicit_grid(gpu, workgroups):
    # any grid size: one workgroup copying everything, grids that do not divide
    # the tile count, and more workgroups than tiles (capped at the tile count)
    n = 700 * 65536 + 777
    _run_copy(gpu, _bytes(900 + workgroups, n), 2,
              dict(copy_tile_bytes=65536, producer_waves=8, consumer_waves=8, flags=2, copy_workgroups=workgroups))


def test_copy_special_float_bits(gpu):
    bits = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x7FBFFFFF],
                    np.uint32)
    src = np.tile(bits, 50_000)
    _run_copy(gpu, src, 2)


def test_copy_one_gib_uniform(gpu):
    """The 1 GiB fp32 workload with 64 KiB tiles and a 2-stage ring, bit-exact."""
    import torch
    n = 1 << 28
    src_np = synth.uniform_pm1(synth.seed_for(2, "src"), n)
    src = torch.from_numpy(src_np).cuda()
    dst = torch.empty_like(src)
    say("staged_copy 1 GiB stages=2")
    gpu.staged_copy(src, dst, stages=2)
    gpu.check_device_status()
    want = oracle.copy(src_np)
    assert oracle.first_mismatch(dst.cpu().numpy(), want) == -1


def test_copy_argument_errors(gpu):
    import torch
    x = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    assert gpu.lib.staged_copy(x.data_ptr(), x.data_ptr() + 4096, 8192, 2) == gpu.WSG_EINVAL  # overlap
    with pytest.raises(gpu.WsgError) as e:  # 3 x 64 KiB exceeds LDS
        gpu.staged_copy_ex(x[:65536], x[65536:131072], stages=3, config=dict(copy_tile_bytes=65536))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    with pytest.raises(gpu.WsgError) as e:  # 20 x 8 KiB exceeds LDS even at the smallest default slot
        gpu.staged_copy(x[:65536], x[65536:131072], stages=20)
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    with pytest.raises(gpu.WsgError) as e:
        gpu.staged_copy_ex(x[:1024], x[2048:3072], stages=2, config=dict(copy_tile_bytes=12345))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    rc = gpu.lib.staged_copy(x.data_ptr() + 8, x.data_ptr() + 65536, 64, 2)
    assert rc == gpu.WSG_EINVAL
    with pytest.raises(gpu.WsgError) as e:
        gpu.staged_copy_ex(x[:1024], x[2048:3072], stages=2, config=dict(copy_workgroups=-1))
    assert e.value.code == gpu.WSG_EINVAL


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4095, 65537, 256 * 256 * 16 * 4 + 7, 3 * 1048576 + 9])
@pytest.mark.parametrize("flags", [8, 8 | 2])  # WSG_FLAG_DIRECT_COPY, with and without streaming
def test_direct_copy_baseline_sizes(gpu, n, flags):
    """The unstaged baseline: same arguments, same bytes, guard bands intact, every tail size."""
    _run_copy(gpu, _bytes(300 + n, n), 2, config=dict(flags=flags))


@pytest.mark.parametrize("workgroups", [1, 7, 256, 1024])
def test_direct_copy_grid_sizes(gpu, workgroups):
    """Grid-stride loop: any grid covers every chunk exactly once (remainder loop included)."""
    n = 256 * 256 * 16 * 3 + 4096 * 16 + 5
    _run_copy(gpu, _bytes(400 + workgroups, n), 2, config=dict(flags=8 | 2, copy_workgroups=workgroups))
