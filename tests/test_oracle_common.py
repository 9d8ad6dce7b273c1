"""Pins of oracle.common: bf16 rounding against torch's CPU conversion and
hand-worked ties, RMSNorm and RoPE against closed forms and invariants."""

import numpy as np
import pytest
import torch

from oracle.common import bf16_round, rms_norm, rope_rotate_half, rope_angles


def test_bf16_round_hand_cases():
    one = 1.0
    ulp = 2.0 ** -7
    assert bf16_round(one) == one
    assert bf16_round(one + ulp / 2) == one                   # tie -> even (1.0)
    assert bf16_round(one + 3 * ulp / 2) == one + 2 * ulp     # tie -> even
    assert bf16_round(one + ulp / 2 + 1e-12) == one + ulp     # just above the tie
    assert bf16_round(-3.0) == -3.0
    assert bf16_round(0.0) == 0.0
    assert bf16_round(2.0 ** 100 * 1.2) == 2.0 ** 100 * 1.203125


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), ref)


def test_rms_norm_closed_forms():
    x = np.full((3, 128), -2.5)
    np.testing.assert_allclose(rms_norm(x, 1.0, 0.0), -1.0, rtol=1e-15)
    g = np.linspace(0.5, 1.5, 128)
    y = rms_norm(np.full(128, 4.0), g, 0.0)
    np.testing.assert_allclose(y, g, rtol=1e-15)
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 2560)) * 7.0
    out = rms_norm(z, 1.0, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-6)
    # Scale invariance (eps = 0).
    np.testing.assert_allclose(rms_norm(3 * z, g[:1], 0.0), rms_norm(z, g[:1], 0.0), rtol=1e-12)
    # eps enters under the square root: x = 0 stays 0, tiny x gets damped.
    np.testing.assert_array_equal(rms_norm(np.zeros(8), 1.0, 1e-6), 0.0)
    np.testing.assert_allclose(rms_norm(np.full(8, 1e-3), 1.0, 1e-6), 1e-3 / np.sqrt(2e-6), rtol=1e-12)


def test_rope_unit_vectors_closed_form():
    theta = 1e6
    pos = 1234
    for i in (0, 1, 17, 32, 63):
        e = np.zeros(128)
        e[i] = 1.0
        phi = pos * theta ** (-2 * i / 128)
        y = rope_rotate_half(e, pos, theta)
        expect = np.zeros(128)
        expect[i] = np.cos(phi)
        expect[i + 64] = np.sin(phi)
        np.testing.assert_allclose(y, expect, atol=1e-15)
        e2 = np.zeros(128)
        e2[i + 64] = 1.0
        y2 = rope_rotate_half(e2, pos, theta)
        expect2 = np.zeros(128)
        expect2[i] = -np.sin(phi)
        expect2[i + 64] = np.cos(phi)
        np.testing.assert_allclose(y2, expect2, atol=1e-15)
    # Frequencies: i = 32 turns at pos / sqrt(theta).
    np.testing.assert_allclose(rope_angles(1000.0, theta)[32], 1.0, rtol=1e-14)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 128))
    np.testing.assert_array_equal(rope_rotate_half(x, 0, 1e6), x)
    y = rope_rotate_half(x, 131071, 1e6)
    np.testing.assert_allclose(x[:, :64] ** 2 + x[:, 64:] ** 2,
                               y[:, :64] ** 2 + y[:, 64:] ** 2, rtol=1e-12)
    # Scores depend only on the position difference.
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    a = rope_rotate_half(q, 100, 1e6) @ rope_rotate_half(k, 37, 1e6)
    b = rope_rotate_half(q, 100 + 5000, 1e6) @ rope_rotate_half(k, 37 + 5000, 1e6)
    assert abs(a - b) < 1e-10
    # Composition: rotating by m then n equals rotating by m + n.
    np.testing.assert_allclose(rope_rotate_half(rope_rotate_half(x, 11, 1e6), 29, 1e6),
                               rope_rotate_half(x, 40, 1e6), atol=1e-12)
