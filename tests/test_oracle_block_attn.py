"""Pins of oracle.block_attn: brute force on tiny shapes, permutation
equivariance of the non-causal block (RoPE off), context permutation
invariance, closed forms, LSE merge, GQA grouping and the non-causality
probe."""

import math

import numpy as np

from oracle.block_attn import block_attn_ref, attend, prep_block

EPS, THETA = 1e-6, 1e6


def _inputs(rng, B, S_list, dtype=np.float64):
    q = rng.standard_normal((B, 32, 8, 128))
    kb = rng.standard_normal((B, 8, 8, 128))
    vb = rng.standard_normal((B, 8, 8, 128))
    gq = 1 + 0.1 * rng.standard_normal(128)
    gk = 1 + 0.1 * rng.standard_normal(128)
    kc = [rng.standard_normal((S, 8, 128)) for S in S_list]
    vc = [rng.standard_normal((S, 8, 128)) for S in S_list]
    return q, kb, vb, gq, gk, kc, vc, np.array(S_list)


def _brute(q, kb, vb, gq, gk, kc, vc, S, rope=True):
    """Pure-Python loops: norm, rotate, score, softmax, weighted sum."""
    def norm_rot(x, g, pos):
        ms = sum(v * v for v in x) / len(x)
        y = [g[i] * x[i] / math.sqrt(ms + EPS) for i in range(len(x))]
        if not rope:
            return y
        out = list(y)
        for i in range(64):
            phi = pos * THETA ** (-2.0 * i / 128)
            out[i] = y[i] * math.cos(phi) - y[i + 64] * math.sin(phi)
            out[i + 64] = y[i + 64] * math.cos(phi) + y[i] * math.sin(phi)
        return out

    out = np.zeros((32, 8, 128))
    for h in range(32):
        g = h // 4
        keys = [list(kc[t, g]) for t in range(S)] + [norm_rot(list(kb[g, j]), gk, S + j) for j in range(8)]
        vals = [list(vc[t, g]) for t in range(S)] + [list(vb[g, j]) for j in range(8)]
        for j in range(8):
            qq = norm_rot(list(q[h, j]), gq, S + j)
            s = [sum(qq[i] * k[i] for i in range(128)) / math.sqrt(128) for k in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for i in range(128):
                out[h, j, i] = sum(e[t] * vals[t][i] for t in range(len(vals))) / z
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    for S in (0, 5, 16):
        q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [S])
        out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl, EPS, THETA)
        ref = _brute(q[0], kb[0], vb[0], gq, gk, kc[0], vc[0], S)
        np.testing.assert_allclose(out[0], ref, atol=1e-12)


def test_block_permutation_equivariance_rope_off():
    rng = np.random.default_rng(1)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [40])
    out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl, rope=False)
    perm = rng.permutation(8)
    out_p, _ = block_attn_ref(q[:, :, perm], kb[:, :, perm], vb[:, :, perm], gq, gk, kc, vc, cl, rope=False)
    np.testing.assert_allclose(out_p, out[:, :, perm], atol=1e-12)


def test_context_permutation_invariance():
    rng = np.random.default_rng(2)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [50])
    out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl)
    perm = rng.permutation(50)
    out_p, _ = block_attn_ref(q, kb, vb, gq, gk, [kc[0][perm]], [vc[0][perm]], cl)
    np.testing.assert_allclose(out_p, out, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [21])
    q[:] = 0.0
    out, lse = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl)
    for g in range(8):
        mean = (vc[0][:, g].sum(0) + vb[0, g].sum(0)) / (21 + 8)
        for hh in range(4):
            np.testing.assert_allclose(out[0, 4 * g + hh], np.broadcast_to(mean, (8, 128)), atol=1e-12)
    np.testing.assert_allclose(lse, np.log(29.0), rtol=1e-14)


def test_lse_merge_of_chunks_equals_one_shot():
    rng = np.random.default_rng(4)
    qr = rng.standard_normal((8, 128))
    keys = rng.standard_normal((300, 128))
    vals = rng.standard_normal((300, 128))
    o, lse = attend(qr, keys, vals)
    parts = [attend(qr, keys[a:b], vals[a:b]) for a, b in ((0, 7), (7, 190), (190, 300))]
    M = np.max([p[1] for p in parts], axis=0)
    w = [np.exp(p[1] - M) for p in parts]
    merged = sum(wi[:, None] * p[0] for wi, p in zip(w, parts)) / sum(w)[:, None]
    np.testing.assert_allclose(merged, o, atol=1e-12)
    np.testing.assert_allclose(M + np.log(sum(w)), lse, atol=1e-12)


def test_identical_heads_in_group_identical_outputs():
    rng = np.random.default_rng(5)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [33])
    q[0, 8:12] = q[0, 8]
    out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl)
    for hh in range(1, 4):
        np.testing.assert_array_equal(out[0, 8 + hh], out[0, 8])
    assert not np.allclose(out[0, 12], out[0, 8])


def test_non_causal_probe_mask_value_reaches_anchor():
    rng = np.random.default_rng(6)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 1, [10])
    out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl)
    vb2 = vb.copy()
    vb2[0, 3, 7] += 5.0            # last mask position, KV head 3
    out2, _ = block_attn_ref(q, kb, vb2, gq, gk, kc, vc, cl)
    assert np.max(np.abs(out2[0, 12:16, 0] - out[0, 12:16, 0])) > 1e-3   # anchor moves
    np.testing.assert_array_equal(out2[0, :12], out[0, :12])            # other groups do not


def test_empty_context_and_window():
    rng = np.random.default_rng(7)
    q, kb, vb, gq, gk, kc, vc, cl = _inputs(rng, 2, [0, 100])
    out, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl)
    qh = prep_block(q[0], gq, 0, EPS, THETA)
    kk = prep_block(kb[0], gk, 0, EPS, THETA)
    o0, _ = attend(qh[9], kk[2], vb[0, 2])
    np.testing.assert_allclose(out[0, 9], o0, atol=1e-12)
    outw, _ = block_attn_ref(q, kb, vb, gq, gk, kc, vc, cl, window=30)
    trunc_k = [kc[0], kc[1][70:]]
    trunc_v = [vc[0], vc[1][70:]]
    # Truncating the cache to the last 30 tokens while keeping positions.
    ref = np.empty_like(out[1])
    qh1 = prep_block(q[1], gq, 100, EPS, THETA)
    kb1 = prep_block(kb[1], gk, 100, EPS, THETA)
    for h in range(32):
        g = h // 4
        ref[h], _ = attend(qh1[h], np.concatenate([trunc_k[1][:, g], kb1[g]]),
                           np.concatenate([trunc_v[1][:, g], vb[1, g]]))
    np.testing.assert_allclose(outw[1], ref, atol=1e-12)
    np.testing.assert_allclose(outw[0], out[0], atol=0)
