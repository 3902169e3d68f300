"""Attention forward on the GPU against the fp64 oracle (bf16 tolerance: P is
rounded to bf16 for the P V products, everything else is fp32).

Inputs sit inside NaN-filled buffers and O inside a sentinel-filled one, so a
read past a head's rows (NaN would reach O) or a write past O shows up.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import say, stratified_rows
from oracle import attention as att

pytestmark = pytest.mark.gpu

SLACK = 4096
GUARD = 4096
SENTINEL = -12345.0
NAN_BF16 = 0x7FC0


def _padded(bits):
    import torch
    flat = np.ascontiguousarray(bits).reshape(-1).view(np.int16)
    buf = torch.full((flat.size + 2 * SLACK,), NAN_BF16, dtype=torch.int16, device="cuda")
    buf[SLACK:SLACK + flat.size] = torch.from_numpy(flat).cuda()
    return buf[SLACK:SLACK + flat.size].view(*bits.shape)


def run_attention(gpu, Q, K, V, causal, stages=2, config=None, scale=None, guards=True):
    import torch
    Bn, H, Sq, D = Q.shape
    n = Bn * H * Sq * D
    if guards:
        dQ, dK, dV = _padded(Q), _padded(K), _padded(V)
        obuf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.float32, device="cuda")
        dO = obuf[GUARD:GUARD + n].view(Bn, H, Sq, D)
    else:
        dQ, dK, dV = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda() for x in (Q, K, V))
        dO = torch.empty((Bn, H, Sq, D), dtype=torch.float32, device="cuda")
    say("attention %s Skv=%d causal=%s stages=%d config=%s" % ((Bn, H, Sq, D), K.shape[2], causal, stages, config))
    gpu.attention_fwd(dQ, dK, dV, dO, scale=scale, causal=causal, stages=stages, config=config)
    gpu.check_device_status()
    if guards:
        o = obuf.cpu().numpy()
        assert np.all(o[:GUARD] == SENTINEL) and np.all(o[GUARD + n:] == SENTINEL), "O guard written"
        return o[GUARD:GUARD + n].reshape(Bn, H, Sq, D)
    return dO.cpu().numpy()


def case(seed, Bn, H, Sq, Skv, D):
    return (synth.normal_bf16_bits(seed + 1, Bn * H * Sq * D, scale=1.0).reshape(Bn, H, Sq, D),
            synth.normal_bf16_bits(seed + 2, Bn * H * Skv * D, scale=1.0).reshape(Bn, H, Skv, D),
            synth.normal_bf16_bits(seed + 3, Bn * H * Skv * D, scale=1.0).reshape(Bn, H, Skv, D))


def check(O, ref):
    s = oracle.compare(O, ref)
    assert oracle.within_tolerance(s, "bf16"), s
    return s


# one tile; several query and key tiles with ragged tails; a single query; more queries than keys;
# fewer queries than keys; head dimension 64
SHAPES = [(1, 1, 128, 128, 128), (2, 3, 200, 333, 128), (1, 2, 1, 64, 128), (1, 1, 300, 70, 128),
          (1, 1, 65, 500, 128), (2, 2, 257, 129, 64), (1, 1, 128, 1, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(gpu, shape, causal):
    Bn, H, Sq, Skv, D = shape
    Q, K, V = case(sum(shape) * 7 + causal, Bn, H, Sq, Skv, D)
    O = run_attention(gpu, Q, K, V, causal)
    check(O, att.attention(Q, K, V, 1.0 / math.sqrt(D), causal))


@pytest.mark.parametrize("stages", [1, 2, 3, 4])
@pytest.mark.parametrize("producers", [1, 2, 4])
def test_ring_depths_and_producers(gpu, stages, producers):
    Q, K, V = case(100 * stages + producers, 1, 2, 130, 600, 128)
    O = run_attention(gpu, Q, K, V, True, stages=stages, config=dict(producer_waves=producers))
    check(O, att.attention(Q, K, V, 1.0 / math.sqrt(128), True))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [s for s in SHAPES if s[4] == 128], ids=lambda s: "x".join(map(str, s)))
def test_seven_consumers(gpu, shape, causal):
    """224 queries per workgroup (7 consumer waves, one of which arrives twice on the empty flags)."""
    Bn, H, Sq, Skv, D = shape
    Q, K, V = case(sum(shape) * 11 + causal, Bn, H, Sq, Skv, D)
    cfg = dict(producer_waves=1, consumer_waves=7)
    O = run_attention(gpu, Q, K, V, causal, stages=3, config=cfg)
    check(O, att.attention(Q, K, V, 1.0 / math.sqrt(D), causal))


def test_seven_consumers_same_bits_as_four(gpu):
    """Each query's arithmetic does not depend on how queries are grouped into workgroups."""
    Q, K, V = case(800, 2, 2, 500, 700, 128)
    for causal in (False, True):
        four = run_attention(gpu, Q, K, V, causal, stages=3, config=dict(producer_waves=1, consumer_waves=4),
                             guards=False)
        for stages in (1, 2, 3, 4):
            seven = run_attention(gpu, Q, K, V, causal, stages=stages,
                                  config=dict(producer_waves=1, consumer_waves=7), guards=False)
            assert np.array_equal(seven.view(np.uint32), four.view(np.uint32))


def test_scale_and_large_scores(gpu):
    """Scores far from 1: the running max keeps the exponentials in range."""
    Q, K, V = case(500, 1, 1, 96, 300, 64)
    for scale in (0.01, 1.0, 4.0):
        O = run_attention(gpu, Q, K, V, False, scale=scale)
        check(O, att.attention(Q, K, V, scale, False))


def test_no_visible_key_gives_zeros(gpu):
    Q, K, V = case(600, 1, 1, 200, 40, 128)
    O = run_attention(gpu, Q, K, V, True)  # queries 0..159 see no key
    assert np.array_equal(O[0, 0, :160], np.zeros((160, 128), np.float32))
    check(O, att.attention(Q, K, V, 1.0 / math.sqrt(128), True))
    Q, K, V = case(601, 1, 1, 50, 0, 128)
    O = run_attention(gpu, Q, K, V, False)
    assert np.array_equal(O, np.zeros_like(O))


def test_same_result_across_ring_depths(gpu):
    """The arithmetic does not depend on the ring: every depth and producer count gives the same bits."""
    Q, K, V = case(700, 1, 2, 256, 512, 128)
    base = run_attention(gpu, Q, K, V, True, stages=2, guards=False)
    for stages, prod in ((1, 1), (3, 2), (4, 4)):
        O = run_attention(gpu, Q, K, V, True, stages=stages, config=dict(producer_waves=prod), guards=False)
        assert np.array_equal(O.view(np.uint32), base.view(np.uint32))


def test_errors(gpu):
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(q[..., :96].contiguous(), q[..., :96].contiguous(), q[..., :96].contiguous())
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(q, q, q, stages=5)  # 5 slots of 32 KiB do not fit
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(q, q, q, scale=float("nan"))
    assert e.value.code == gpu.WSG_EINVAL
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(q, q, q, config=dict(producer_waves=3))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    for cfg in (dict(producer_waves=2, consumer_waves=7), dict(consumer_waves=5)):
        with pytest.raises(gpu.WsgError) as e:
            gpu.attention_fwd(q, q, q, config=cfg)
        assert e.value.code == gpu.WSG_EUNSUPPORTED
    q64 = q[..., :64].contiguous()
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(q64, q64, q64, config=dict(consumer_waves=7))
    assert e.value.code == gpu.WSG_EUNSUPPORTED
    buf = torch.zeros(64 * 128 + 8, dtype=torch.int16, device="cuda")
    mis = buf[1:1 + 64 * 128].view(1, 1, 64, 128)  # 2-byte offset
    with pytest.raises(gpu.WsgError) as e:
        gpu.attention_fwd(mis, q, q)
    assert e.value.code == gpu.WSG_EINVAL
    gpu.check_device_status()


@pytest.mark.parametrize("consumers", [7, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_full_size_sampled(gpu, causal, consumers):
    """The benchmark's shape (batch 4, 32 heads, 4096 x 4096, D 128) in the launch configuration the
    benchmark times (one producer, seven consumers) and with four consumers, against the oracle on
    sampled rows of sampled heads."""
    w = synth.ATTENTION
    Bn, H, S, D = w["batch"], w["heads"], w["S"], w["D"]
    n = Bn * H * S * D
    Q = synth.normal_bf16_bits(synth.seed_for(w["id"], "A"), n, scale=1.0).reshape(Bn, H, S, D)
    K = synth.normal_bf16_bits(synth.seed_for(w["id"], "B"), n, scale=1.0).reshape(Bn, H, S, D)
    V = synth.normal_bf16_bits(synth.seed_for(w["id"], "src"), n, scale=1.0).reshape(Bn, H, S, D)
    O = run_attention(gpu, Q, K, V, causal, stages=w["stages"], guards=False,
                      config=dict(producer_waves=1, consumer_waves=consumers))
    # every head, three rows of every query tile (each workgroup owns one query tile of one head)
    for b in range(Bn):
        for h in range(H):
            rows = stratified_rows(S, 32 * consumers, b * H + h)
            check(O[b, h, rows], att.attention_rows(Q, K, V, 1.0 / math.sqrt(D), causal, b, h, rows))
    assert np.all(np.isfinite(O))
