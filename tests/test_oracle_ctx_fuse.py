"""Pins of oracle.ctx_fuse: one-hot probes fix the concatenation order, the
W_c orientation and the layer-major [K | V] split; closed forms fix the
norms and RoPE placement."""

import numpy as np

from oracle.ctx_fuse import ctx_fuse_ref, fuse, project_kv, concat_capture
from oracle.common import bf16_round, rope_rotate_half

D = 2560


def _weights(rng, L=2):
    wc = rng.standard_normal((D, 5 * D)) * 0.02
    wkv = rng.standard_normal((L * 2048, D)) * 0.02
    return wc, wkv


def test_concat_order_one_hot():
    rng = np.random.default_rng(0)
    wc, _ = _weights(rng, 1)
    gc = np.ones(D)
    for j, c in ((0, 5), (2, 2559), (4, 1000)):
        hs = [np.zeros((2, D)) for _ in range(5)]
        hs[j][1, c] = 3.0
        hs[(j + 1) % 5][0, 7] = 1.0
        x = concat_capture(hs)
        assert x[1, j * D + c] == 3.0
        ht = fuse(hs, wc, gc, 0.0)
        col = wc[:, j * D + c]
        np.testing.assert_allclose(ht[1], col / np.sqrt(np.mean(col ** 2)), rtol=1e-12)


def test_fusion_norm_rms_one_and_gain():
    rng = np.random.default_rng(1)
    wc, _ = _weights(rng, 1)
    hs = [rng.standard_normal((4, D)) for _ in range(5)]
    ht = fuse(hs, wc, np.ones(D), 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(ht ** 2, axis=1)), 1.0, rtol=1e-6)
    g = 1 + 0.1 * rng.standard_normal(D)
    np.testing.assert_allclose(fuse(hs, wc, g, 1e-6), ht * g, rtol=1e-12)


def test_kv_split_one_hot_layer_major():
    rng = np.random.default_rng(2)
    L = 3
    wkv = rng.standard_normal((L * 2048, D)) * 0.02
    c = 321
    ht = np.zeros((1, D))
    ht[0, c] = 1.0
    gk = np.ones((L, 128))
    K, V = project_kv(ht, wkv, gk, np.array([0]), 0.0, 1e6)
    for l in range(L):
        for h in (0, 5, 7):
            kcol = wkv[2048 * l + 128 * h: 2048 * l + 128 * (h + 1), c]
            vcol = wkv[2048 * l + 1024 + 128 * h: 2048 * l + 1024 + 128 * (h + 1), c]
            np.testing.assert_allclose(V[l, 0, h], vcol, rtol=1e-14)
            # K at position 0: RoPE is the identity, k_norm makes RMS 1.
            np.testing.assert_allclose(K[l, 0, h], kcol / np.sqrt(np.mean(kcol ** 2)), rtol=1e-12)


def test_k_norm_gain_then_rope_at_row_position():
    rng = np.random.default_rng(3)
    L = 2
    wkv = rng.standard_normal((L * 2048, D)) * 0.02
    ht = rng.standard_normal((3, D))
    gk = 1 + 0.1 * rng.standard_normal((L, 128))
    pos = np.array([0, 17, 131071])
    K, V = project_kv(ht, wkv, gk, pos, 1e-6, 1e6)
    K0, V0 = project_kv(ht, wkv, gk, np.zeros(3, dtype=int), 1e-6, 1e6)
    np.testing.assert_array_equal(V, V0)
    for m in range(3):
        np.testing.assert_allclose(K[:, m], rope_rotate_half(K0[:, m], pos[m], 1e6), atol=1e-12)
    # Before RoPE each head equals gk * k / rms(k).
    raw = (ht @ wkv[:1024].T).reshape(3, 8, 128)
    exp0 = gk[0] * raw / np.sqrt(np.mean(raw ** 2, axis=-1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(K0[0], exp0, rtol=1e-12)


def test_full_path_bf16_storage_point():
    rng = np.random.default_rng(4)
    wc, wkv = _weights(rng, 2)
    hs = [rng.standard_normal((3, D)) for _ in range(5)]
    gc = 1 + 0.1 * rng.standard_normal(D)
    gk = 1 + 0.1 * rng.standard_normal((2, 128))
    pos = np.array([5, 6, 7])
    ht, hts, K, V = ctx_fuse_ref(hs, wc, gc, wkv, gk, pos)
    np.testing.assert_array_equal(hts, bf16_round(ht))
    K2, V2 = project_kv(hts, wkv, gk, pos, 1e-6, 1e6)
    np.testing.assert_array_equal(K, K2)
    np.testing.assert_array_equal(V, V2)
    _, hts32, _, _ = ctx_fuse_ref(hs, wc, gc, wkv, gk, pos, ht_bf16=False)
    np.testing.assert_array_equal(hts32, ht)
