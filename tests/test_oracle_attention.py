"""Pins of the attention oracle against what does not use it, and mutants it must catch.

- brute force: a pure-Python loop per query with math.exp, its own max and its own sums;
- closed forms: Q = 0 gives the mean of the visible V rows (causal: of V[0 .. i + Skv - Sq]); V all ones
  gives ones; a key that one query selects by a large margin returns that key's V row;
- invariance: permuting the keys together with their values leaves non-causal O unchanged;
- range: scores far beyond exp's range (about 800) still give finite, correct outputs.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

import synth
from oracle import attention as att

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")


def _bf16(seed, shape, scale=1.0):
    return synth.normal_bf16_bits(seed, int(np.prod(shape)), scale=scale).reshape(shape)


def _brute(Q, K, V, scale, causal):
    q, k, v = att.widen(Q), att.widen(K), att.widen(V)
    Bn, H, Sq, D = q.shape
    Skv = k.shape[2]
    O = np.zeros((Bn, H, Sq, D))
    for b in range(Bn):
        for h in range(H):
            for i in range(Sq):
                keys = [j for j in range(Skv) if not causal or j <= i + (Skv - Sq)]
                if not keys:
                    continue
                s = [scale * sum(float(q[b, h, i, d]) * float(k[b, h, j, d]) for d in range(D)) for j in keys]
                top = max(s)
                w = [math.exp(x - top) for x in s]
                tot = sum(w)
                for d in range(D):
                    O[b, h, i, d] = sum(wj * float(v[b, h, j, d]) for wj, j in zip(w, keys)) / tot
    return O


CASES = [(1, 1, 5, 5, 4, False), (1, 2, 3, 7, 4, True), (2, 1, 6, 4, 8, True), (1, 1, 4, 4, 8, True),
         (1, 1, 1, 9, 4, False)]


def run_pins(fn, rows_fn):
    failed = []
    for n, (Bn, H, Sq, Skv, D, causal) in enumerate(CASES):
        Q, K, V = _bf16(10 + n, (Bn, H, Sq, D)), _bf16(20 + n, (Bn, H, Skv, D)), _bf16(30 + n, (Bn, H, Skv, D))
        ref = _brute(Q, K, V, 0.5, causal)
        try:
            if not np.allclose(fn(Q, K, V, 0.5, causal), ref, rtol=1e-12, atol=1e-13):
                failed.append("brute_force_%d" % n)
            rows = np.arange(Sq)[::-1]
            if not np.allclose(rows_fn(Q, K, V, 0.5, causal, Bn - 1, H - 1, rows), ref[Bn - 1, H - 1, rows],
                               rtol=1e-12, atol=1e-13):
                failed.append("brute_force_rows_%d" % n)
        except (ValueError, IndexError, FloatingPointError):
            failed.append("brute_force_raises_%d" % n)
    # Q = 0: every visible key weighs the same
    Bn, H, Sq, Skv, D = 1, 1, 6, 9, 4
    Q0 = np.zeros((Bn, H, Sq, D), np.uint16)
    K, V = _bf16(40, (Bn, H, Skv, D)), _bf16(41, (Bn, H, Skv, D))
    v = att.widen(V)[0, 0]
    for causal in (False, True):
        want = np.stack([v[:min(Skv, i + Skv - Sq + 1) if causal else Skv].mean(axis=0) for i in range(Sq)])
        if not np.allclose(fn(Q0, K, V, 0.7, causal)[0, 0], want, rtol=1e-12, atol=1e-14):
            failed.append("uniform_%s" % causal)
    # V = 1: the weights sum to one
    ones = np.full((Bn, H, Skv, D), 0x3F80, np.uint16)  # bf16 1.0
    Q = _bf16(42, (Bn, H, Sq, D))
    if not np.allclose(fn(Q, K, ones, 0.9, True), 1.0, rtol=0, atol=1e-14):
        failed.append("weights_sum_to_one")
    # a large margin selects one key: query i -> key (3 i) mod Skv
    D = 8
    Kh = np.zeros((1, 1, Skv, D), np.float32)
    Qh = np.zeros((1, 1, Sq, D), np.float32)
    for j in range(Skv):
        Kh[0, 0, j, j % D] = 1.0 if j < D else -1.0
    for i in range(Sq):
        Qh[0, 0, i, (3 * i) % Skv % D] = 60.0
    Vh = synth.uniform_pm1(43, Skv * D).reshape(1, 1, Skv, D)
    got = fn(Qh, Kh, Vh, 1.0, False)[0, 0]
    want = np.stack([Vh[0, 0, (3 * i) % Skv % D] for i in range(Sq)]).astype(np.float64)
    if not np.allclose(got, want, rtol=0, atol=1e-20):  # the other keys weigh exp(-60) ~ 1e-26 or less
        failed.append("selected_key")
    # permuting keys with their values
    Q, K, V = _bf16(44, (1, 2, 5, 4)), _bf16(45, (1, 2, 7, 4)), _bf16(46, (1, 2, 7, 4))
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    a = fn(Q, K, V, 0.4, False)
    b = fn(Q, K[:, :, perm], V[:, :, perm], 0.4, False)
    if not np.allclose(a, b, rtol=1e-12, atol=1e-14) or np.allclose(a, fn(Q, K, V[:, :, perm], 0.4, False)):
        failed.append("key_permutation")
    # scores near 800: exp of the raw score overflows
    Kb = np.zeros((1, 1, 3, 4), np.float32)
    Kb[0, 0, :, 0] = [800.0, 799.0, 790.0]
    Qb = np.zeros((1, 1, 1, 4), np.float32)
    Qb[0, 0, 0, 0] = 1.0
    Vb = np.zeros((1, 1, 3, 4), np.float32)
    Vb[0, 0, :, 1] = [1.0, 2.0, 3.0]
    with np.errstate(over="ignore", invalid="ignore"):
        try:
            o = fn(Qb, Kb, Vb, 1.0, False)[0, 0, 0, 1]
        except (FloatingPointError, OverflowError):
            o = float("nan")
    w = np.exp(np.array([0.0, -1.0, -10.0]))
    if not (np.isfinite(o) and abs(o - float((w * [1, 2, 3]).sum() / w.sum())) < 1e-12):
        failed.append("large_scores")
    return failed


def test_oracle_passes_every_pin():
    assert run_pins(att.attention, att.attention_rows) == []


MUTANTS = {
    "no_scale": ("s = scale * (q[b, h] @ k[b, h].T)", "s = q[b, h] @ k[b, h].T"),
    "keys_transposed_product": ("s = scale * (q[b, h] @ k[b, h].T)", "s = scale * (q[b, h] @ q[b, h].T)[:, :k.shape[2]] if q.shape[2] >= k.shape[2] else scale * (q[b, h] @ k[b, h].T)"),
    "causal_strict": ("return j <= i + (Skv - Sq)", "return j < i + (Skv - Sq)"),
    "causal_top_left": ("return j <= i + (Skv - Sq)", "return j <= i"),
    "no_max_shift": ("p = np.exp(s[rows] - m)", "p = np.exp(s[rows])"),
    "normalize_wrong_axis": ("p /= np.sum(p, axis=1, keepdims=True)\n            O[b, h, rows]",
                             "p /= np.sum(p, axis=0, keepdims=True)\n            O[b, h, rows]"),
    "values_are_keys": ("O[b, h, rows] = p @ v[b, h]", "O[b, h, rows] = p @ k[b, h]"),
    "bf16_shift": ("return (x.astype(np.uint32) << 16)", "return (x.astype(np.uint32) << 15)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site for %s no longer in attention.py" % name
    path = tmp_path / ("attention_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("attention_mutant_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with np.errstate(all="ignore"):
        assert run_pins(mod.attention, mod.attention_rows), "mutant %s passed every pin" % name


def test_shapes_and_edges():
    Q = _bf16(50, (1, 1, 4, 8))
    K = _bf16(51, (1, 1, 0, 8))
    assert np.array_equal(att.attention(Q, K, K, 1.0, False), np.zeros((1, 1, 4, 8)))
    # causal with more queries than keys: the first Sq - Skv queries see nothing
    K, V = _bf16(52, (1, 1, 2, 8)), _bf16(53, (1, 1, 2, 8))
    O = att.attention(Q, K, V, 1.0, True)
    assert np.array_equal(O[0, 0, :2], np.zeros((2, 8))) and np.all(np.abs(O[0, 0, 2:]) > 0)
    with pytest.raises(ValueError):
        att.attention(Q, K[:, :, :, :4], V, 1.0, False)
