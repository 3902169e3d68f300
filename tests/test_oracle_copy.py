"""The staged copy's oracle: the destination is the source, byte for byte."""
import numpy as np

import synth


def test_copy_is_identity_on_bytes(oracle_lib):
    for n in [0, 1, 3, 15, 16, 65535, 65536, 65537, 5 << 20]:
        src = (synth.splitmix64(5000 + n, (n + 7) // 8).view(np.uint8)[:n]).copy()
        dst = oracle_lib.copy(src, threads=4)
        assert dst.nbytes == n
        assert np.array_equal(dst, src)
        assert oracle_lib.first_mismatch(dst, src) == -1


def test_copy_keeps_special_float_bit_patterns(oracle_lib):
    bits = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x7F800000, 0x00000001], np.uint32)
    f = bits.view(np.float32)
    out = oracle_lib.copy(f)
    assert np.array_equal(out.view(np.uint32), bits)


def test_first_mismatch_finds_planted_difference(oracle_lib):
    a = synth.splitmix64(77, 1 << 16).view(np.uint8)
    b = a.copy()
    b[123457] ^= 0x10
    assert oracle_lib.first_mismatch(a, b) == 123457
    assert oracle_lib.first_mismatch(a, a[:-1]) == a.nbytes - 1
