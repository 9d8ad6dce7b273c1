"""Pins of oracle.dflash2: the block convolution reduces to numpy's 1-D
convolution per channel and a one-step shift kernel fixes its direction and
zero padding; with a zero kernel the layer is the plain draft layer; row
statistics match scipy's entropy and log-softmax and a stable sort (ties to
the lower id); the beam's top-P paths equal brute-force enumeration of every
path (continuous log-probabilities, and bf16-grid logits with many exactly
tied sums, compared as integers), -inf candidates order after finite ones,
the single best path is the per-position argmax, and lambda shifts
every score by lambda times the summed entropy without reordering."""

import itertools

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle.dflash2 import conv_mlp_ref, depthwise_conv_ref, path_select_ref, row_stats_ref, top_paths_ref


@pytest.mark.parametrize("k", [3, 5])
def test_conv_is_causal_convolution_per_channel(k):
    rng = np.random.default_rng(k)
    B, T, D = 3, 8, 16
    h = rng.standard_normal((B, T, D))
    w = rng.standard_normal((k, D))
    b = rng.standard_normal(D)
    out = depthwise_conv_ref(h, w, b)
    for bb in range(B):
        for c in range(D):
            ref = np.convolve(h[bb, :, c], w[:, c])[:T] + b[c]
            np.testing.assert_allclose(out[bb, :, c], ref, rtol=0, atol=1e-12)


def test_conv_shift_kernel_fixes_direction_and_padding():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((2, 8, 4))
    w = np.zeros((3, 4))
    w[1] = 1.0                                   # out[t] = h[t - 1]
    out = depthwise_conv_ref(h, w, np.zeros(4))
    assert np.array_equal(out[:, 1:], h[:, :-1])
    assert np.all(out[:, 0] == 0.0)              # nothing before the anchor
    w = np.zeros((5, 4))
    w[4] = 1.0
    out = depthwise_conv_ref(h, w, np.full(4, 0.5))
    assert np.array_equal(out[:, 4:], h[:, :4] + 0.5)
    assert np.all(out[:, :4] == 0.5)


def test_zero_kernel_layer_is_plain_draft_layer():
    rng = np.random.default_rng(2)
    B, D, I = 2, 32, 24
    x = rng.standard_normal((B, 8, D))
    o = rng.standard_normal((B, 2, 8, 8))        # 2 heads x 8 dims = 16 inputs of W_O
    w_o = 0.1 * rng.standard_normal((D, 16))
    g = 1 + 0.1 * rng.standard_normal(D)
    w_gu = 0.1 * rng.standard_normal((2 * I, D))
    w_d = 0.1 * rng.standard_normal((D, I))
    for bf16 in (False, True):
        a = conv_mlp_ref(x, o, w_o, np.zeros((3, D)), np.zeros(D), g, w_gu, w_d, g_final=g, bf16=bf16)
        r = oracle.mlp_ref(x, o, w_o, g, w_gu, w_d, g_final=g, bf16=bf16)
        np.testing.assert_array_equal(a["x_out"], r["x_out"])
        np.testing.assert_array_equal(a["y"], r["y"])
    # A conv that cancels h (w_0 = -1) leaves h' = b in every row: every row's
    # feed-forward input is the same.
    b = rng.standard_normal(D)
    w = np.zeros((3, D))
    w[0] = -1.0
    a = conv_mlp_ref(x, o, w_o, w, b, g, w_gu, w_d, bf16=False)
    np.testing.assert_allclose(a["h_conv"], np.broadcast_to(b, a["h_conv"].shape), atol=1e-12)
    np.testing.assert_allclose(a["c"], np.broadcast_to(a["c"][0], a["c"].shape), atol=1e-12)


def test_row_stats_match_library_and_ties():
    rng = np.random.default_rng(3)
    z = 2.5 * rng.standard_normal((4, 7, 300))
    z[0, 0, [10, 20, 30]] = 50.0                 # three-way tie on top: ids in increasing order
    ids, logp, ent = row_stats_ref(z, 5)
    np.testing.assert_allclose(ent, stats.entropy(special.softmax(z, axis=-1), axis=-1), rtol=1e-12, atol=1e-12)
    ls = special.log_softmax(z, axis=-1)
    np.testing.assert_allclose(logp, np.take_along_axis(ls, ids, axis=-1), rtol=0, atol=1e-12)
    assert ids[0, 0, :3].tolist() == [10, 20, 30]
    order = np.argsort(-z, axis=-1, kind="stable")[..., :5]
    assert np.array_equal(ids, order)
    assert np.all(np.diff(logp, axis=-1) <= 0)
    _, _, e_uniform = row_stats_ref(np.zeros((1, 1000)), 1)
    np.testing.assert_allclose(e_uniform, np.log(1000), rtol=1e-14)


@pytest.mark.parametrize("m,P", [(2, 7), (3, 20), (3, 2187), (4, 1)])
def test_beam_equals_brute_force(m, P):
    rng = np.random.default_rng(m * 100 + P)
    J = 7
    logp = np.sort(np.log(rng.dirichlet(np.ones(12), size=J))[:, :m], axis=-1)[:, ::-1]
    logp[2, 1] = logp[2, 0]                      # a tie between ranks at one position
    ids = rng.integers(0, 1000, size=(J, m))
    ent = rng.uniform(0, 3, size=J)
    toks, scores, ranks = top_paths_ref(ids, logp, ent, P, 0.0)
    allp = []
    for r in itertools.product(range(m), repeat=J):
        allp.append((-sum(logp[j, r[j]] for j in range(J)), r))
    allp.sort()
    best = allp[:P]
    assert ranks.tolist() == [list(r) for _, r in best]
    np.testing.assert_allclose(scores, [-s for s, _ in best], rtol=0, atol=1e-12)
    assert np.array_equal(toks, ids[np.arange(J)[None, :], ranks])


def _bf16_grid(rng, shape, scale):
    """Values on the bf16 grid of N(0, scale^2) draws (8 significant bits)."""
    x = scale * rng.standard_normal(shape)
    e = np.floor(np.log2(np.abs(x)))
    q = 2.0 ** (e - 7)
    return np.round(x / q) * q


def _brute_force_ranks(vals, P):
    """Every rank tuple, ordered by the integer sum of its candidates (values
    scaled to integers: exact), larger first, ties by the tuple."""
    J, m = vals.shape
    unit = 2.0 ** -40                            # every value in these tests is a multiple of it
    iv = [[int(round(v / unit)) for v in row] for row in vals]
    assert all(float(a) * unit == v for row, vrow in zip(iv, vals) for a, v in zip(row, vrow))
    allp = sorted(itertools.product(range(m), repeat=J), key=lambda r: (-sum(iv[j][r[j]] for j in range(J)), r))
    return [list(r) for r in allp[:P]]


def test_paths_on_tied_bf16_logits_equal_brute_force():
    # Stored bf16 logits: distinct candidate combinations often have equal
    # sums.  The order must follow the exact sums and the rank tuples; a
    # score rounded in floating point (the sum of fp64 log-probabilities
    # z - zmax - log Z) lets rounding decide those ties, and does so wrongly
    # on a good share of these cases -- the check below makes sure the
    # inputs contain such cases.
    rng = np.random.default_rng(17)
    J, m, P = 7, 3, 30
    naive_wrong = 0
    for case in range(60):
        z = _bf16_grid(rng, (J, 40), 2.0)
        ids, logp, ent = row_stats_ref(z, m)
        vals = np.take_along_axis(z, ids.astype(np.int64), axis=-1)
        lse = oracle.dflash2.log_normaliser_ref(z)
        toks, scores, ranks = top_paths_ref(ids, vals, ent, P, 0.4, lse)
        assert ranks.tolist() == _brute_force_ranks(vals, P), case
        own = vals[np.arange(J)[None, :], ranks].sum(axis=1) - lse.sum() + 0.4 * ent.sum()
        np.testing.assert_allclose(scores, own, rtol=0, atol=1e-9)
        naive = sorted(itertools.product(range(m), repeat=J),
                       key=lambda r: (-sum(logp[j, r[j]] for j in range(J)), r))[:P]
        naive_wrong += [list(r) for r in naive] != ranks.tolist()
    assert naive_wrong >= 5


def test_paths_with_neg_inf_candidates():
    # Rows with fewer finite logits than candidates: paths through a -inf
    # candidate come after every finite path, by their number of -inf
    # candidates, then by the exact sum of the finite ones, then by tuple.
    rng = np.random.default_rng(23)
    J, m, P = 7, 3, 600                          # 2 * 3^5 = 486 finite paths, then -inf ones
    z = _bf16_grid(rng, (J, 16), 1.5)
    z[1, 2:] = -np.inf                           # two finite entries: rank 2 is -inf
    z[4, 1:] = -np.inf                           # one finite entry
    ids, logp, ent = row_stats_ref(z, m)
    vals = np.take_along_axis(z, ids.astype(np.int64), axis=-1)
    toks, scores, ranks = top_paths_ref(ids, vals, ent, P, 0.0)
    unit = 2.0 ** -40
    allp = []
    for r in itertools.product(range(m), repeat=J):
        v = [vals[j, r[j]] for j in range(J)]
        n_inf = sum(x == -np.inf for x in v)
        allp.append(((n_inf, -sum(int(round(x / unit)) for x in v if x != -np.inf), r), r))
    allp.sort()
    assert ranks.tolist() == [list(r) for _, r in allp[:P]]
    finite = np.isfinite(scores)
    assert finite.sum() == 2 * 3 ** 5 and np.all(finite[:2 * 3 ** 5])
    assert np.all(scores[~finite] == -np.inf)
    with pytest.raises(ValueError):
        top_paths_ref(ids, np.where(vals == -np.inf, np.inf, vals), ent, P, 0.0)


def test_single_path_is_argmax_and_lambda_shifts():
    rng = np.random.default_rng(5)
    z = 2.0 * rng.standard_normal((3, 8, 500))
    ids, logp, ent, toks, scores, ranks = path_select_ref(z, 4, 1, 0.0)
    assert np.array_equal(toks[:, 0], np.argmax(z[:, 1:], axis=-1))
    assert np.all(ranks == 0)
    _, _, _, toks0, s0, _ = path_select_ref(z, 4, 30, 0.0)
    _, _, _, toks1, s1, _ = path_select_ref(z, 4, 30, 0.7)
    assert np.array_equal(toks0, toks1)
    np.testing.assert_allclose(s1 - s0, 0.7 * ent.sum(axis=-1, keepdims=True) + 0 * s0, atol=1e-12)
