"""Pins of oracle.spec_verify: the length bound, greedy equals step-by-step
argmax decoding on a toy target, chi-square tests of the output law, the
closed-form accept-length law, and planted special cases."""

import numpy as np
import pytest
from scipy import stats

from oracle.spec_verify import spec_verify_ref


def _rand_case(rng, B, V, sigma=3.0, noise=1.0):
    zt = rng.standard_normal((B, 8, V)) * sigma
    zd = zt[:, :7] + rng.standard_normal((B, 7, V)) * noise
    return zt, zd


def test_length_always_in_1_8_and_padding():
    rng = np.random.default_rng(0)
    B, V = 64, 64
    zt, zd = _rand_case(rng, B, V, noise=2.0)
    d = rng.integers(0, V, size=(B, 7))
    d[::3] = np.argmax(zd[::3], axis=-1)
    T = np.where(np.arange(B) % 2 == 0, 0.0, rng.uniform(0.3, 2.0, B))
    tr = spec_verify_ref(zt, zd, d, T, seed=3, offset=9)
    assert np.all((tr.out_len >= 1) & (tr.out_len <= 8))
    assert np.array_equal(tr.out_len, tr.n_acc + 1)
    for b in range(B):
        n = tr.out_len[b]
        assert np.all(tr.out_tokens[b, n:] == -1)
        assert np.all((tr.out_tokens[b, :n] >= 0) & (tr.out_tokens[b, :n] < V))
        np.testing.assert_array_equal(tr.out_tokens[b, :n - 1], d[b, :n - 1])


def _toy_logits(prefix, V):
    """Deterministic toy target: logits depend on the last three tokens."""
    key = hash(tuple(int(t) for t in prefix[-3:])) & 0xFFFFFFFF
    return np.random.default_rng(key).standard_normal(V) * 3.0


def test_greedy_equals_step_by_step_argmax_decoding():
    V, N = 40, 120
    rng = np.random.default_rng(1)
    prompt = [1, 2, 3]
    ref = list(prompt)
    while len(ref) < len(prompt) + N:
        ref.append(int(np.argmax(_toy_logits(ref, V))))
    seq = list(prompt)
    cycles = 0
    while len(seq) < len(prompt) + N:
        # An imperfect drafter: right with probability 0.7 given its own prefix.
        d = []
        ctx = list(seq)
        for _ in range(7):
            t = int(np.argmax(_toy_logits(ctx, V)))
            if rng.random() > 0.7:
                t = int(rng.integers(V))
            d.append(t)
            ctx.append(t)
        zt = np.stack([_toy_logits(seq + d[:r], V) for r in range(8)])[None]
        tr = spec_verify_ref(zt, zt[:, :7], np.array([d]), np.array([0.0]))
        seq.extend(int(x) for x in tr.out_tokens[0, :tr.out_len[0]])
        cycles += 1
    assert seq[:len(ref)] == ref
    assert cycles < N  # speculation actually accepted something


def _fixed_rows(rng, V, sharp=1.5):
    p = np.exp(rng.standard_normal((8, V)) * sharp)
    q = np.exp(rng.standard_normal((7, V)) * sharp)
    return np.log(p / p.sum(1, keepdims=True)), np.log(q / q.sum(1, keepdims=True))


@pytest.mark.slow
def test_chi_square_output_law_and_accept_length_law():
    """Rows fixed across trials; drafts d_k ~ q_k from an independent
    generator.  out[0] ~ p_0; out[1] | accepted d_1 ~ p_1; the number of
    accepted proposals follows prod(beta) (1 - beta) with
    beta_k = sum_x min(p_{k-1}(x), q_k(x))."""
    V, B = 6, 12000
    rng = np.random.default_rng(2)
    lp, lq = _fixed_rows(rng, V)
    p, q = np.exp(lp), np.exp(lq)
    zt = np.broadcast_to(lp, (B, 8, V))
    zd = np.broadcast_to(lq, (B, 7, V))
    draw = np.random.default_rng(99)
    d = np.stack([draw.choice(V, size=B, p=q[k]) for k in range(7)], axis=1)
    tr = spec_verify_ref(zt, zd, d, np.ones(B), seed=7, offset=1, seq_block=256)

    def chi2_p(counts, probs):
        exp = probs * counts.sum()
        return stats.chisquare(counts, exp).pvalue

    c0 = np.bincount(tr.out_tokens[:, 0], minlength=V)
    assert chi2_p(c0, p[0]) > 1e-3
    acc1 = tr.out_tokens[:, 0] == d[:, 0]
    assert np.array_equal(acc1, tr.n_acc >= 1)
    c1 = np.bincount(tr.out_tokens[acc1, 1], minlength=V)
    assert chi2_p(c1, p[1]) > 1e-3
    beta = np.minimum(p[:7], q).sum(axis=1)
    law = np.empty(8)
    run = 1.0
    for n in range(7):
        law[n] = run * (1 - beta[n])
        run *= beta[n]
    law[7] = run
    hist = np.bincount(tr.n_acc, minlength=8)
    keep = law * B > 5
    exp = law[keep] * B
    obs = hist[keep]
    pval = stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue
    assert pval > 1e-3


@pytest.mark.slow
def test_bonus_gumbel_sampler_law():
    """q == p accepts all seven proposals; the bonus token then follows
    softmax(z_7 / T) (Gumbel-max sampler check)."""
    V, B = 7, 12000
    rng = np.random.default_rng(3)
    z7 = rng.standard_normal(V) * 2.0
    T = 1.7
    zt = np.zeros((B, 8, V))
    zt[:, 7] = z7
    zd = zt[:, :7].copy()
    d = np.zeros((B, 7), dtype=int)
    tr = spec_verify_ref(zt, zd, d, np.full(B, T), seed=11, seq_block=512)
    assert np.all(tr.out_len == 8) and np.all(tr.kind == 2)
    pz = np.exp(z7 / T)
    pz /= pz.sum()
    c = np.bincount(tr.out_tokens[:, 7], minlength=V)
    assert stats.chisquare(c, pz * B).pvalue > 1e-3


def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(4)
    B, V = 16, 300
    zt = rng.standard_normal((B, 8, V)) * 4
    d = rng.integers(0, V, (B, 7))
    tr = spec_verify_ref(zt, zt[:, :7].copy(), d, np.full(B, 0.7))
    assert np.all(tr.out_len == 8)
    assert np.all(tr.rho[~np.isnan(tr.rho)] == pytest.approx(1.0, abs=1e-12))


def test_planted_greedy_cases():
    rng = np.random.default_rng(5)
    B, V = 8, 500
    zt = rng.standard_normal((B, 8, V))
    am = np.argmax(zt, axis=-1)
    d = am[:, :7].copy()
    tr = spec_verify_ref(zt, zt[:, :7], d, np.zeros(B))
    assert np.all(tr.out_len == 8)
    np.testing.assert_array_equal(tr.out_tokens[:, 7], am[:, 7])
    for k in range(1, 8):
        d2 = d.copy()
        d2[:, k - 1] = (am[:, k - 1] + 1) % V
        tr = spec_verify_ref(zt, zt[:, :7], d2, np.zeros(B))
        assert np.all(tr.out_len == k)
        np.testing.assert_array_equal(tr.out_tokens[:, k - 1], am[:, k - 1])


def test_greedy_ties_go_to_lowest_index():
    zt = np.zeros((1, 8, 10))
    zt[0, :, [3, 6]] = 2.0
    d = np.full((1, 7), 6)
    tr = spec_verify_ref(zt, zt[:, :7], d, np.zeros(1))
    assert tr.out_len[0] == 1 and tr.out_tokens[0, 0] == 3


def test_planted_sampled_rejection_position():
    """p puts (almost) no mass on d_k while q puts almost all: rejection at k,
    and the replacement never equals d_k."""
    rng = np.random.default_rng(6)
    B, V = 32, 50
    zt = rng.standard_normal((B, 8, V))
    zd = zt[:, :7].copy()
    d = rng.integers(0, V, (B, 7))
    k = 4
    for b in range(B):
        zt[b, k - 1, d[b, k - 1]] = -60.0
        zd[b, k - 1, d[b, k - 1]] = 60.0
        # Rows before k agree exactly, so proposals 1..k-1 are accepted.
    tr = spec_verify_ref(zt, zd, d, np.full(B, 1.0), seed=5)
    assert np.all(tr.out_len == k)
    assert np.all(tr.kind == 1)
    assert np.all(tr.out_tokens[:, k - 1] != d[:, k - 1])


def test_temperature_is_a_logit_scale():
    rng = np.random.default_rng(7)
    B, V = 16, 200
    zt, zd = _rand_case(rng, B, V)
    d = rng.integers(0, V, (B, 7))
    d[:, :3] = np.argmax(zd[:, :3], -1)
    a = spec_verify_ref(zt, zd, d, np.full(B, 2.0), seed=1)
    b = spec_verify_ref(zt / 2.0, zd / 2.0, d, np.full(B, 1.0), seed=1)
    np.testing.assert_array_equal(a.out_tokens, b.out_tokens)


def test_out_of_range_proposals_are_rejected():
    rng = np.random.default_rng(8)
    B, V = 4, 100
    zt = rng.standard_normal((B, 8, V))
    d = np.argmax(zt[:, :7], -1)
    d[:, 2] = V + 5
    d[1, 2] = -1
    g = spec_verify_ref(zt, zt[:, :7], d, np.zeros(B))
    s = spec_verify_ref(zt, zt[:, :7], d, np.ones(B))
    assert np.all(g.out_len == 3) and np.all(s.out_len == 3)
    assert np.all((s.out_tokens[:, 2] >= 0) & (s.out_tokens[:, 2] < V))
