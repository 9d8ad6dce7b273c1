"""Pins of oracle.draft_layer: the layer shapes reproduce the parameter count
the pages print, one-hot probes fix the Q/K/V head layout and the attention
output's transposition, closed forms fix the residuals, SiLU and the norms,
and a pure-Python brute force on tiny dimensions fixes the composition."""

import json
import math
import os

import numpy as np
import pytest

from oracle.common import bf16_round
from oracle.draft_layer import (BLOCK, D, INTER, embed_block, layer_weight_shapes, mlp_ref, qkv_ref, silu)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_figures.json")))


def test_layer_shapes_reproduce_parameter_count():
    # [E4B] "The parameter count exposes the real cost": 1,031,568,640 logical
    # parameters = output head + W_c + five layers + fusion and final norms.
    V = 262144
    per_layer = sum(int(np.prod(s)) for s in layer_weight_shapes().values())
    total = V * D + 5 * D * D + 5 * per_layer + 2 * D
    assert total == GOLD["draft_parameters"]["value"]


def test_embed_block_anchor_then_mask_rows():
    rng = np.random.default_rng(0)
    emb = rng.standard_normal((50, 12))
    out = embed_block(emb, [3, 49, 0], mask_id=7)
    assert out.shape == (3, BLOCK, 12)
    for b, a in enumerate([3, 49, 0]):
        assert np.array_equal(out[b, 0], emb[a])
        for j in range(1, BLOCK):
            assert np.array_equal(out[b, j], emb[7])


def test_qkv_head_layout_one_hot():
    # W_QKV row r reads input column c: q[b, h, j, d] for r = 128 h + d,
    # k for r = 4096 + 128 g + d, v for r = 5120 + 128 g + d.
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, BLOCK, D))
    w = np.zeros((6144, D))
    probes = {("q", 5, 17): (128 * 5 + 17, 11), ("k", 3, 0): (4096 + 128 * 3, 2559),
              ("v", 7, 127): (5120 + 128 * 7 + 127, 100), ("q", 31, 127): (4095, 0)}
    for (_, _, _), (r, c) in probes.items():
        w[r, c] = 1.0
    q, k, v, a = qkv_ref(x, np.ones(D), w, eps=0.0, bf16=False)
    assert q.shape == (2, 32, BLOCK, 128) and k.shape == (2, 8, BLOCK, 128) and v.shape == k.shape
    got = {"q": q, "k": k, "v": v}
    arows = a.reshape(2, BLOCK, D)
    for (t, hh, dd), (r, c) in probes.items():
        np.testing.assert_allclose(got[t][:, hh, :, dd], arows[:, :, c], rtol=0, atol=0)
    # Everything else is zero.
    total = sum(np.count_nonzero(g) for g in got.values())
    assert total == len(probes) * 2 * BLOCK


def test_qkv_input_norm_rms_one():
    rng = np.random.default_rng(2)
    x = 3.0 * rng.standard_normal((1, BLOCK, D))
    _, _, _, a = qkv_ref(x, np.ones(D), np.zeros((6144, D)), eps=1e-6, bf16=False)
    np.testing.assert_allclose(np.sqrt(np.mean(a ** 2, axis=1)), 1.0, rtol=1e-6)


def test_mlp_zero_projections_are_identity():
    # With W_O = 0 and W_D = 0 both residual branches vanish: x' = h = x.
    rng = np.random.default_rng(3)
    x = bf16_round(rng.standard_normal((2, BLOCK, D)))
    o = rng.standard_normal((2, 32, BLOCK, 128))
    w_gu = rng.standard_normal((2 * INTER, D)) * 0.02
    for bf16 in (False, True):
        r = mlp_ref(x, o, np.zeros((D, 4096)), np.ones(D), w_gu, np.zeros((D, INTER)), bf16=bf16)
        assert np.array_equal(r["h"], x.reshape(-1, D))
        assert np.array_equal(r["x_out"], x.reshape(-1, D))


def test_attention_output_transposition_one_hot():
    # o[b, h, j, d] = 1 adds column 128 h + d of W_O to row 8 b + j of h.
    rng = np.random.default_rng(4)
    x = np.zeros((2, BLOCK, D))
    w_o = rng.standard_normal((D, 4096))
    o = np.zeros((2, 32, BLOCK, 128))
    o[1, 9, 6, 33] = 1.0
    r = mlp_ref(x, o, w_o, np.ones(D), np.zeros((2 * INTER, D)), np.zeros((D, INTER)), bf16=False)
    expect = np.zeros((2 * BLOCK, D))
    expect[8 + 6] = w_o[:, 128 * 9 + 33]
    assert np.array_equal(r["h"], expect)


def test_silu_closed_forms():
    x = np.linspace(-30, 30, 601)
    s = silu(x)
    assert silu(0.0) == 0.0
    np.testing.assert_allclose(s - silu(-x), x, rtol=0, atol=1e-12)  # x*sig(x) - (-x)*sig(-x) = x
    np.testing.assert_allclose(s[x >= 20], x[x >= 20], rtol=1e-8)
    assert np.all(np.abs(s[x <= -20]) < 1e-6)


def test_swiglu_one_hot():
    # Gate row i reads column a, up row i reads column b, W_D = one-hot column i:
    # x'[m, e] = h[m, e] + silu(c[m, a]) * c[m, b] for output e.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, BLOCK, D))
    w_gu = np.zeros((2 * INTER, D))
    w_d = np.zeros((D, INTER))
    i, a, b, e = 17, 3, 2000, 901
    w_gu[i, a] = 1.0
    w_gu[INTER + i, b] = 1.0
    w_d[e, i] = 1.0
    r = mlp_ref(x, np.zeros((1, 32, BLOCK, 128)), np.zeros((D, 4096)), np.ones(D), w_gu, w_d, bf16=False)
    c = r["c"]
    delta = r["x_out"] - r["h"]
    np.testing.assert_allclose(delta[:, e], silu(c[:, a]) * c[:, b], rtol=1e-14)
    assert np.count_nonzero(np.delete(delta, e, axis=1)) == 0


def test_final_norm_rms_one_and_gain():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, BLOCK, D))
    g = 1 + 0.1 * rng.standard_normal(D)
    args = (x, np.zeros((1, 32, BLOCK, 128)), np.zeros((D, 4096)), np.ones(D),
            rng.standard_normal((2 * INTER, D)) * 0.02, rng.standard_normal((D, INTER)) * 0.02)
    r1 = mlp_ref(*args, g_final=np.ones(D), bf16=False)
    np.testing.assert_allclose(np.sqrt(np.mean(r1["y"] ** 2, axis=1)), 1.0, rtol=1e-6)
    r2 = mlp_ref(*args, g_final=g, bf16=False)
    np.testing.assert_allclose(r2["y"], r1["y"] * g, rtol=1e-12)


# ---- brute force on tiny dimensions ----

def _rms(row, g, eps):
    ms = sum(v * v for v in row) / len(row)
    return [g[i] * row[i] / math.sqrt(ms + eps) for i in range(len(row))]


def _matvec(w, v):
    return [sum(w[r][c] * v[c] for c in range(len(v))) for r in range(len(w))]


def _rnd(vals, bf16):
    return [float(bf16_round(v)) for v in vals] if bf16 else list(vals)


@pytest.mark.parametrize("bf16", [False, True])
def test_brute_force_tiny_layer(bf16):
    d, hq, hkv, hd, inter, B, eps = 6, 2, 1, 4, 3, 2, 1e-6
    rng = np.random.default_rng(7)
    x = bf16_round(rng.standard_normal((B, BLOCK, d))) if bf16 else rng.standard_normal((B, BLOCK, d))
    g_in, g_post, g_fin = (1 + 0.1 * rng.standard_normal(d) for _ in range(3))
    w_qkv = rng.standard_normal(((hq + 2 * hkv) * hd, d)) * 0.5
    w_o = rng.standard_normal((d, hq * hd)) * 0.5
    w_gu = rng.standard_normal((2 * inter, d)) * 0.5
    w_d = rng.standard_normal((d, inter)) * 0.5
    o = rng.standard_normal((B, hq, BLOCK, hd))

    q, k, v, _ = qkv_ref(x, g_in, w_qkv, eps, bf16=bf16, hq=hq, hkv=hkv, head_dim=hd)
    r = mlp_ref(x, o, w_o, g_post, w_gu, w_d, eps, g_final=g_fin, bf16=bf16)

    for b in range(B):
        for j in range(BLOCK):
            row = list(x[b, j])
            a = _rnd(_rms(row, g_in, eps), bf16)
            y = _matvec(w_qkv, a)
            for h in range(hq):
                for dd in range(hd):
                    assert abs(q[b, h, j, dd] - y[h * hd + dd]) < 1e-12
            for g in range(hkv):
                for dd in range(hd):
                    assert abs(k[b, g, j, dd] - y[hq * hd + g * hd + dd]) < 1e-12
                    assert abs(v[b, g, j, dd] - y[(hq + hkv) * hd + g * hd + dd]) < 1e-12
            ocat = [o[b, h, j, dd] for h in range(hq) for dd in range(hd)]
            proj = _matvec(w_o, ocat)
            hrow = [row[i] + proj[i] for i in range(d)]
            hs = _rnd(hrow, bf16)
            c = _rnd(_rms(hs, g_post, eps), bf16)
            gu = _matvec(w_gu, c)
            s = [gu[i] / (1 + math.exp(-gu[i])) * gu[inter + i] for i in range(inter)]
            down = _matvec(w_d, _rnd(s, bf16))
            xo = [hs[i] + down[i] for i in range(d)]
            yv = _rms(_rnd(xo, bf16), g_fin, eps)
            m = b * BLOCK + j
            for i in range(d):
                assert abs(r["h"][m, i] - hrow[i]) < 1e-12
                assert abs(r["x_out"][m, i] - xo[i]) < 1e-12
                assert abs(r["y"][m, i] - yv[i]) < 1e-12
            for i in range(inter):
                assert abs(r["s"][m, i] - s[i]) < 1e-12
