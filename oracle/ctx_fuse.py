"""Context fusion and K/V injection -- float64 reference.

Test infrastructure only (see the package docstring).

Follows [DF2] 4.1 "Target Context Feature Konditionierung via KV-Injection":
the five captured target states are concatenated on the feature axis,
projected by W_c (D x 5D) and RMS-normalised into H_t; H_t is then projected
by every draft layer's W_K / W_V and written into that layer's cache,
bypassing the layer's Q, O and FFN.  [E4B] "Five target states become
persistent draft context" fixes the shapes (5 states of width 2560, draft
width 2560, 8 KV heads of 128) and the per-head K RMSNorm before RoPE.

Readings where the pages are silent (listed in the design notes as well):
* the fusion RMSNorm has a learned weight g_c and eps (1e-6);
* W_c is stored [out = 2560, in = 12800]; feature j*2560 + c of the
  concatenation is column c of capture j, captures in order 5, 11, 17, 23, 35
  ([E4B] "The released serving cycle");
* W_KV is layer-major: rows [2048 l, 2048 l + 1024) are layer l's W_K
  (8 heads x 128), the next 1024 rows its W_V; no biases anywhere;
* context K gets the layer's per-head k_norm then RoPE at the token's
  position; V is stored as projected;
* in bf16 mode H_t is stored rounded to bf16 before the K/V projection.
"""

import numpy as np

from .common import bf16_round, rms_norm, rope_rotate_half

D = 2560
N_CAPTURE = 5
HKV = 8
HEAD_DIM = 128
KV_ROWS_PER_LAYER = 2 * HKV * HEAD_DIM  # 2048


def concat_capture(hs):
    """[H^(l1); ...; H^(l5)] on the feature axis: list of 5 [M, D] -> [M, 5D]."""
    if len(hs) != N_CAPTURE:
        raise ValueError("expected five captured states")
    return np.concatenate([np.asarray(h, dtype=np.float64) for h in hs], axis=1)


def fuse(hs, wc, gc, eps):
    """H_t = RMSNorm(W_c [H1; ...; H5]) in float64 ([DF2] 4.1, first equation)."""
    x = concat_capture(hs)
    y = x @ np.asarray(wc, dtype=np.float64).T
    return rms_norm(y, gc, eps)


def project_kv(ht, wkv, gk, pos, eps, theta):
    """Per-layer context K/V of [DF2] 4.1 (second equation, context half).

    ht: [M, D]; wkv: [L*2048, D]; gk: [L, 128]; pos: [M].
    Returns K, V as [L, M, 8, 128] float64, K after k_norm and RoPE.
    """
    ht = np.asarray(ht, dtype=np.float64)
    wkv = np.asarray(wkv, dtype=np.float64)
    L = wkv.shape[0] // KV_ROWS_PER_LAYER
    M = ht.shape[0]
    K = np.empty((L, M, HKV, HEAD_DIM))
    V = np.empty((L, M, HKV, HEAD_DIM))
    for l in range(L):
        base = l * KV_ROWS_PER_LAYER
        k = (ht @ wkv[base:base + HKV * HEAD_DIM].T).reshape(M, HKV, HEAD_DIM)
        v = (ht @ wkv[base + HKV * HEAD_DIM:base + KV_ROWS_PER_LAYER].T).reshape(M, HKV, HEAD_DIM)
        k = rms_norm(k, np.asarray(gk, dtype=np.float64)[l], eps)
        k = rope_rotate_half(k, np.asarray(pos)[:, None], theta)
        K[l] = k
        V[l] = v
    return K, V


def ctx_fuse_ref(hs, wc, gc, wkv, gk, pos, eps=1e-6, theta=1e6, ht_bf16=True):
    """Full context fusion + K/V injection.

    Returns (ht, ht_stored, K, V): ht is the float64 fused context, ht_stored
    the value the K/V projection consumes (bf16-rounded when ``ht_bf16``),
    K/V are [L, M, 8, 128] float64 before any cache rounding.
    """
    ht = fuse(hs, wc, gc, eps)
    ht_stored = bf16_round(ht) if ht_bf16 else ht
    K, V = project_kv(ht_stored, wkv, gk, pos, eps, theta)
    return ht, ht_stored, K, V
