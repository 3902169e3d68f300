"""The seeded input generators (shared by the oracle and the GPU path)."""
import numpy as np

import synth


def test_splitmix64_reference_vector():
    # Widely published reference outputs of splitmix64 seeded with 1234567.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert synth.splitmix64(1234567, 5).tolist() == want


def test_splitmix64_offset_and_chunks_agree():
    full = synth.splitmix64(42, 10_000)
    assert np.array_equal(synth.splitmix64(42, 100, start=5000), full[5000:5100])


def test_uniform_range_exactness_and_determinism():
    x = synth.uniform_pm1(3001, 1 << 20)
    assert x.dtype == np.float32
    assert x.min() >= -1.0 and x.max() < 1.0
    # every value is a multiple of 2^-23, i.e. exact in fp32
    assert np.all((x.astype(np.float64) * 2.0 ** 23) % 1 == 0)
    assert abs(float(x.mean())) < 5e-3
    assert np.array_equal(x, synth.uniform_pm1(3001, 1 << 20))
    # element i does not depend on the requested length
    assert np.array_equal(synth.uniform_pm1(3001, 1000), x[:1000])


def test_bf16_rounding_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, -0.0], np.float32)
    bits = synth.f32_to_bf16_bits_rne(f)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6 (0x3F82)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x0000, 0x8000]
    assert np.array_equal(synth.bf16_bits_to_f32(bits)[[0, 4]], np.array([1.0, -2.5], np.float32))


def test_normal_bf16_moments():
    x = synth.bf16_bits_to_f32(synth.normal_bf16_bits(5001, 1 << 18)).astype(np.float64)
    assert abs(x.mean()) < 2e-3
    assert abs(x.std() - 0.1) < 2e-3


def test_small_ints_cover_range():
    x = synth.small_int_f32(11, 10_000, -3, 3)
    assert set(np.unique(x).tolist()) == {-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0}


def test_seeds_distinct_per_tensor():
    seeds = {synth.seed_for(w, t) for w in synth.WORKLOADS for t in synth.TENSOR_IDS}
    assert len(seeds) == len(synth.WORKLOADS) * len(synth.TENSOR_IDS)


def test_moe_group_rows():
    rows = synth.moe_group_rows(600, 4096, 8, 2)
    assert rows.dtype == np.int64 and rows.shape == (8,)
    assert rows.sum() == 4096 * 2 and rows.max() <= 4096 and rows.min() >= 0
    assert rows.max() > 1.5 * rows.min()  # uneven loads
    assert np.array_equal(rows, synth.moe_group_rows(600, 4096, 8, 2))
    assert not np.array_equal(rows, synth.moe_group_rows(601, 4096, 8, 2))
    assert synth.moe_group_rows(1, 10, 4, 4).tolist() == [10, 10, 10, 10]
