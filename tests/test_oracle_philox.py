"""Pins of oracle.philox: the Philox4x64-10 block function against numpy's
independent implementation, and the uniform / Gumbel layout against closed
forms."""

import numpy as np
import pytest

from oracle.philox import philox4x64_10, uniforms, uniform_row, gumbel, words_to_uniform


def _numpy_block(counter, key):
    """Block at `counter` from numpy.random.Philox (which increments its
    256-bit counter before producing a block, so start it one below)."""
    c = [int(x) for x in counter]
    v = c[0] | (c[1] << 64) | (c[2] << 128) | (c[3] << 192)
    v -= 1
    prev = np.array([(v >> (64 * j)) & ((1 << 64) - 1) for j in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=prev)
    return g.random_raw(4)


def test_block_matches_numpy_philox():
    rng = np.random.default_rng(123)
    ctrs = rng.integers(0, 2 ** 63, size=(64, 4), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    keys = rng.integers(0, 2 ** 63, size=(64, 2), dtype=np.uint64) * np.uint64(2)
    for c, k in zip(ctrs, keys):
        ours = philox4x64_10(c, (k[0], k[1]))
        np.testing.assert_array_equal(ours, _numpy_block(c, k))


def test_block_matches_numpy_at_small_counters():
    # The counters the verification layout actually uses: small lanes.
    for c in ([1, 0, 0, 0], [5, 17, 1, 3], [65535, 8 * 63 + 7, 1, 12]):
        ours = philox4x64_10(np.array(c, dtype=np.uint64), (np.uint64(7), np.uint64(0)))
        np.testing.assert_array_equal(ours, _numpy_block(c, [7, 0]))


def test_vectorised_equals_scalar():
    rng = np.random.default_rng(5)
    ctrs = rng.integers(0, 2 ** 62, size=(10, 4), dtype=np.uint64)
    batch = philox4x64_10(ctrs, (np.uint64(3), np.uint64(9)))
    for i in range(10):
        np.testing.assert_array_equal(batch[i], philox4x64_10(ctrs[i], (np.uint64(3), np.uint64(9))))


def test_uniform_layout_word_selection():
    # U(s, b, k, i) is 23-bit half i % 2 (0: bits 41..63, 1: bits 9..31) of
    # word (i // 2) % 4 of the block at counter (i // 8, 8b + k, s, offset).
    seed, off, s, b, k = 11, 4, 1, 3, 5
    i = np.arange(37)
    u = uniforms(seed, off, s, b, k, i)
    for j in i:
        blk = philox4x64_10(np.array([j // 8, 8 * b + k, s, off], dtype=np.uint64),
                            (np.uint64(seed), np.uint64(0)))
        w = int(blk[(j // 2) % 4])
        bits = (w >> 41) if j % 2 == 0 else ((w >> 9) & 0x7FFFFF)
        assert u[j] == (bits + 0.5) * 2.0 ** -23
    np.testing.assert_array_equal(uniform_row(seed, off, s, b, k, 37), u)


def test_uniform_range_and_fp32_exact():
    w = np.array([0, 1, 2 ** 41 - 1, 2 ** 41, 2 ** 64 - 1], dtype=np.uint64)
    u = words_to_uniform(w)
    assert u[0] == 0.5 * 2.0 ** -23 and u[-1] == 1.0 - 0.5 * 2.0 ** -23
    assert u[3] == 1.5 * 2.0 ** -23
    # low half: bits 9..31 only
    lo = words_to_uniform(np.array([0, 2 ** 9 - 1, 2 ** 9, 2 ** 32 - 1, 2 ** 64 - 1 - (2 ** 32 - 2 ** 9)],
                                   dtype=np.uint64), 1)
    assert lo[0] == lo[1] == 0.5 * 2.0 ** -23 and lo[2] == 1.5 * 2.0 ** -23
    assert lo[3] == 1.0 - 0.5 * 2.0 ** -23 and lo[4] == 0.5 * 2.0 ** -23
    rowu = uniform_row(1, 2, 1, 0, 1, 1 << 16)
    assert np.all(rowu > 0) and np.all(rowu < 1)
    np.testing.assert_array_equal(rowu.astype(np.float32).astype(np.float64), rowu)


def test_uniform_halves_are_independent():
    # The two halves of the same words: no correlation beyond sampling noise.
    n = 200_000
    u = uniform_row(77, 0, 1, 2, 3, 2 * n)
    hi, lo = u[0::2], u[1::2]
    r = np.corrcoef(hi, lo)[0, 1]
    assert abs(r) < 4 / np.sqrt(n)


def test_uniform_and_gumbel_moments():
    u = uniform_row(2024, 0, 1, 7, 3, 200_000)
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 2e-3
    # Kolmogorov-Smirnov distance against U(0, 1).
    us = np.sort(u)
    ks = np.max(np.abs(us - (np.arange(1, u.size + 1) - 0.5) / u.size))
    assert ks < 1.63 / np.sqrt(u.size)  # alpha = 1 %
    g = gumbel(u)
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 4 * np.sqrt(np.pi ** 2 / 6 / g.size)
    assert abs(g.var() - np.pi ** 2 / 6) < 0.03


def test_streams_are_distinct():
    a = uniform_row(0, 0, 0, 0, 1, 64)
    b = uniform_row(0, 0, 1, 0, 1, 64)
    c = uniform_row(0, 1, 0, 0, 1, 64)
    d = uniform_row(0, 0, 0, 1, 1, 64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
