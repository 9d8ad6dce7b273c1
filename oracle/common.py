"""Shared float64 building blocks of the oracle: bf16 rounding, RMSNorm, RoPE.

Test infrastructure only (see the package docstring).
"""

import numpy as np

HEAD_DIM = 128
HALF = HEAD_DIM // 2


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored).  Writing
    x = m * 2**e with m in [0.5, 1), the rounded value is
    rint(m * 256) * 2**(e - 8); numpy's rint rounds halves to even.  This is
    the rounding applied wherever a bf16 intermediate is stored (the fused
    context H_t, cache entries); the pages do not state rounding points, so
    this is the plainest reading of "BF16 K/V" in [E4B] "Cache and latency
    have separate break-even points".
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def rms_norm(x, g, eps):
    """RMSNorm over the last axis: g * x / sqrt(mean(x^2) + eps).

    Used for the fusion norm of [DF2] 4.1 (H_t = RMSNorm(W_c [...])) and for
    the per-head Q/K normalisation of [E4B] "Five target states become
    persistent draft context" ("Per-head Q/K RMS normalization is applied
    before RoPE").
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope_angles(pos, theta, head_dim=HEAD_DIM):
    """Rotation angles phi[..., i] = pos * theta**(-2 i / head_dim), i < head_dim/2.

    The pages call the drafter "Qwen3-style" ([E4B], opening section) and
    say only that Q/K normalisation happens before RoPE; the frequency
    schedule theta**(-2i/d) with theta = 1e6 is the standard one for that
    family.  Computed in float64 so that long positions (131072) keep full
    angle accuracy.
    """
    half = head_dim // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope_rotate_half(x, pos, theta):
    """Rotate-half RoPE on the last axis (pairs (i, i + d/2)).

    (a, b) = (x_i, x_{i+d/2}) -> (a cos phi_i - b sin phi_i,
                                  b cos phi_i + a sin phi_i).
    ``pos`` broadcasts against x.shape[:-1].  Reading of [E4B] "Five target
    states become persistent draft context" (RoPE after per-head RMSNorm);
    the pairing convention is not printed on the pages.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    phi = rope_angles(pos, theta, d)
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
