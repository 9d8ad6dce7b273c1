"""Non-causal draft block attention -- float64 reference.

Test infrastructure only (see the package docstring).

Follows [E4B] "Five target states become persistent draft context": for the
eight block positions (one anchor + seven masks, [E4B] "The released serving
cycle") each draft layer forms Q [B, 32, 8, 128] and K/V [B, 8, 8, 128],
applies per-head RMSNorm to Q and K and then RoPE, and attends over the
cached (injected) context followed by the block's own keys; four query heads
share each KV head.  "Non-causal" means the block positions attend to each
other bidirectionally (same section and [E4B] training paragraph), so there is
no mask at all inside the block.  [DF2] 4.1 gives K = [W_K H_t ; W_K H_d]_seq,
i.e. keys are context followed by block.

Readings (the pages are silent): block position j (0 = anchor) sits at
position S_b + j; softmax scale 1/sqrt(128); query head h uses KV head
h // 4; an optional window keeps only the latest ``window`` context tokens
([E4B] mentions a 1,024-token draft attention span).
"""

import numpy as np

from .common import rms_norm, rope_rotate_half

HQ, HKV, HEAD_DIM, BLOCK = 32, 8, 128, 8
GROUP = HQ // HKV


def prep_block(x, g, start_pos, eps, theta, rope=True):
    """Per-head RMSNorm then RoPE of block rows x [heads, 8, 128] at start_pos + j."""
    y = rms_norm(x, g, eps)
    if rope:
        y = rope_rotate_half(y, (start_pos + np.arange(x.shape[-2]))[None, :], theta)
    return y


def attend(q, keys, vals, scale=1.0 / np.sqrt(HEAD_DIM)):
    """Plain softmax attention of rows q [n, d] over keys/vals [t, d].

    Returns (o [n, d], lse [n]) with lse = log sum_t exp(scale q.k_t).
    """
    s = (np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T) * scale
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    o = (e / z) @ np.asarray(vals, np.float64)
    return o, (m + np.log(z))[:, 0]


def block_attn_ref(q, k_blk, v_blk, gq, gk, k_ctx, v_ctx, ctx_len, eps=1e-6,
                   theta=1e6, window=0, rope=True):
    """One draft layer's block attention for a batch.

    q: [B, 32, 8, 128]; k_blk, v_blk: [B, 8, 8, 128] (before norm / RoPE);
    gq, gk: [128]; k_ctx[b], v_ctx[b]: [>= ctx_len[b], 8, 128] cached context
    (already normalised and rotated when it was injected); ctx_len: [B].
    Returns out [B, 32, 8, 128] and lse [B, 32, 8] (natural log).
    """
    B = q.shape[0]
    out = np.empty((B, HQ, BLOCK, HEAD_DIM))
    lse = np.empty((B, HQ, BLOCK))
    for b in range(B):
        S = int(ctx_len[b])
        t0 = max(0, S - window) if window else 0
        qh = prep_block(q[b], gq, S, eps, theta, rope)
        kb = prep_block(k_blk[b], gk, S, eps, theta, rope)
        vb = np.asarray(v_blk[b], np.float64)
        for g in range(HKV):
            keys = np.concatenate([np.asarray(k_ctx[b][t0:S, g], np.float64).reshape(-1, HEAD_DIM),
                                   kb[g]], axis=0)
            vals = np.concatenate([np.asarray(v_ctx[b][t0:S, g], np.float64).reshape(-1, HEAD_DIM),
                                   vb[g]], axis=0)
            for hh in range(GROUP):
                h = g * GROUP + hh
                out[b, h], lse[b, h] = attend(qh[h], keys, vals)
    return out, lse
