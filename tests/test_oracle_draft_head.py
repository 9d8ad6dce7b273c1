"""Pins of oracle.draft_head: a one-hot head fixes the orientation, greedy
proposals are the lowest-index argmax, sampled proposals follow
softmax(z / T) (chi-square over independent offsets), a vanishing
temperature reduces sampling to the argmax, and draws use stream 2 (the
verification streams give other draws); the proposal rows' softmax statistics
match scipy's logsumexp and closed forms."""

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.draft_head import DRAFT_STREAM, draft_sample_ref, head_logits_ref
from oracle.philox import gumbel, uniform_row


def test_head_orientation_one_hot():
    rng = np.random.default_rng(0)
    y = rng.standard_normal((2, 8, 16))
    w = np.zeros((50, 16))
    w[7, 3] = 1.0
    w[49, 15] = -2.0
    z = head_logits_ref(y, w)
    assert z.shape == (2, 8, 50)
    assert np.array_equal(z[:, :, 7], y[:, :, 3])
    assert np.array_equal(z[:, :, 49], -2.0 * y[:, :, 15])
    assert np.count_nonzero(np.delete(z, [7, 49], axis=2)) == 0


def test_greedy_is_lowest_index_argmax():
    z = np.zeros((1, 8, 10))
    z[0, 1, [3, 6]] = 5.0          # tie: lowest index wins
    z[0, 2, 9] = 1.0
    z[0, 3, 0] = -1.0              # all others 0: index 1 (first zero after the -1)
    d, gap = draft_sample_ref(z, [0.0])
    assert d[0, 0] == 3 and d[0, 1] == 9 and d[0, 2] == 1
    assert d[0, 3:].tolist() == [0, 0, 0, 0]
    assert np.all(np.isinf(gap))


def test_sampled_proposals_follow_softmax():
    # Every sequence b and row k draws from its own counters (8b + k), so one
    # call over N sequences whose seven rows hold the same logits gives 7N
    # independent draws.
    V, T, N = 8, 0.7, 3000
    row = np.array([1.5, 0.2, -0.4, 0.9, 0.0, 2.1, -1.3, 0.6])
    z = np.broadcast_to(row, (N, 8, V)).copy()
    d, _ = draft_sample_ref(z, np.full(N, T), seed=5, offset=0)
    p = np.exp(row / T)
    p /= p.sum()
    counts = np.bincount(d.reshape(-1), minlength=V)
    n = d.size
    chi2 = np.sum((counts - n * p) ** 2 / (n * p))
    assert stats.chi2.sf(chi2, V - 1) > 1e-3


def test_vanishing_temperature_is_argmax():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 8, 64))
    d_hot, _ = draft_sample_ref(z, [1e-6] * 3, seed=9, offset=4)
    d_greedy, _ = draft_sample_ref(z, [0.0] * 3)
    assert np.array_equal(d_hot, d_greedy)


def test_draws_use_stream_two():
    rng = np.random.default_rng(2)
    V, T = 4096, 1.0
    z = rng.standard_normal((1, 8, V))
    d, _ = draft_sample_ref(z, [T], seed=3, offset=11)
    for k in range(1, 8):
        keys = {s: z[0, k] / T + gumbel(uniform_row(3, 11, s, 0, k, V)) for s in (0, 1, 2)}
        assert int(np.argmax(keys[DRAFT_STREAM])) == d[0, k - 1]
    # with V = 4096 the three streams' draws differ in at least one of the seven rows
    other = [[int(np.argmax(z[0, k] / T + gumbel(uniform_row(3, 11, s, 0, k, V)))) for k in range(1, 8)] for s in (0, 1)]
    assert other[0] != d[0].tolist() and other[1] != d[0].tolist()


def test_draft_stats_closed_forms_and_library():
    # s is the softmax normaliser at temperature T relative to the row max:
    # log(s) + m / T = logsumexp(z / T) (scipy); constant rows give s = V;
    # one logit far above the rest gives s = 1; greedy rows carry none.
    from scipy.special import logsumexp
    rng = np.random.default_rng(12)
    B, V = 4, 600
    z = 3.0 * rng.standard_normal((B, 8, V))
    temp = np.array([0.7, 0.0, 1.0, 2.5])
    st = oracle.draft_stats_ref(z, temp)
    for b in (0, 2, 3):
        T = temp[b]
        np.testing.assert_array_equal(st[b, :, 0], z[b, 1:].max(axis=-1))
        np.testing.assert_allclose(np.log(st[b, :, 1]) + st[b, :, 0] / T, logsumexp(z[b, 1:] / T, axis=-1),
                                   rtol=1e-13)
        # q_k(x) = exp((z - m) / T) / s sums to one, and matches softmax(z / T)
        q = np.exp((z[b, 1:] - st[b, :, :1]) / T) / st[b, :, 1:]
        np.testing.assert_allclose(q.sum(axis=-1), 1.0, rtol=1e-13)
    assert np.all(st[1, :, 0] == -np.inf) and np.all(st[1, :, 1] == 0)
    flat = np.zeros((1, 8, V))
    np.testing.assert_allclose(oracle.draft_stats_ref(flat, [0.8])[0, :, 1], V)
    spike = np.zeros((1, 8, V))
    spike[0, :, 7] = 1e4
    np.testing.assert_allclose(oracle.draft_stats_ref(spike, [1.0])[0, :, 1], 1.0)
    # row 0 (the anchor) is not a proposal row
    z2 = z.copy()
    z2[:, 0] += 100.0
    np.testing.assert_array_equal(oracle.draft_stats_ref(z2, temp), st)
