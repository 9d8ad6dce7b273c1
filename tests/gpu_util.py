"""Helpers of the GPU parity tests: host<->device conversion and the
comparison rules for verification outputs."""

import sys

import numpy as np
import torch

from oracle.spec_verify import DRAW_TERMS

BF16, F32 = torch.bfloat16, torch.float32
TOL = {BF16: 2e-2, F32: 1e-4}   # max abs error bars on attention / projection outputs

# ---- error model of the GPU's fp32 Gumbel-max keys --------------------------
# The kernels compute a draw's key in fp32 from the exact stored logits and
# the exact 23-bit uniforms u; only the arithmetic differs from the oracle's
# fp64.  Per entry, to first order:
#   G = -ln(-ln u), two hardware logs (log2 times ln 2): relative error
#       EPS_HW + 2u of the inner log gives that much absolute error in G,
#       and the outer log adds |G| (EPS_HW + 2u)
#   scaled logit w = z * fl(1/T): two roundings, 2u |w|
#   exponent x = (z - max) * log2(e) / T as an fma on a split scale:
#       2u |x| (one rounding, and one more for fp32 logits' difference)
#   exp2: EPS_HW relative; a row normaliser sums such terms in fp32 along
#       a chain of at most NSUM additions and rescalings, relative error
#       EPS_HW + 2u E_p|x| + NSUM u
#   p = exp2(x) * fl(1/S): + 2u; r = p - q: + u r; ln r: |dr| / r plus
#       (EPS_HW + 2u) |ln r|
#   key = fl(w + G): u (|w| + |G|)
# EPS_HW = 2^-21 allows four ulps of fp32 for the hardware log2 / exp2
# (specified to about one).
U32 = 2.0 ** -24
EPS_HW = 2.0 ** -21
NSUM = 64
_T = {name: i for i, name in enumerate(DRAW_TERMS)}


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def exact(t):
    """Exact stored values of a device tensor as float64."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_step(v):
    """Spacing of bf16 values at |v|: 2^(e-7) for 2^e <= |v| < 2^(e+1)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def bf16_err(gpu, ref, extra=0.0):
    """Largest error of a stored bf16 output against the oracle's unrounded
    value, as a fraction of its bound max(2e-2, 1.1 * 2^-8 |ref|) + extra
    (pass: <= 1).  The first term is the storage rounding (half a step);
    extra carries one-step differences of stored intermediates."""
    gpu, ref = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    bound = np.maximum(TOL[BF16], 1.1 * 2.0 ** -8 * np.abs(ref)) + extra
    return float(np.max(np.abs(gpu - ref) / bound)) if gpu.size else 0.0


def gumbel_err(g):
    """Bound on |G_gpu - G| for G = -ln(-ln u)."""
    return (1.0 + np.abs(g)) * (EPS_HW + 2 * U32)


def scaled_key_err(w, g):
    """Bound on the fp32 error of key = z / T + G (w = z / T)."""
    w, g = np.abs(w), np.abs(g)
    return 2 * U32 * w + gumbel_err(g) + U32 * (w + g)


def draw_key_err(tr, b, j):
    """Bound on the fp32 error of the key of entry j (rank in the oracle's
    list) of sequence b's final draw."""
    t = tr.draw_terms[b, j]
    g, w = t[_T["g"]], t[_T["w"]]
    if tr.kind[b] == 2:
        return float(scaled_key_err(w, g))
    if tr.draw_fallback[b]:                      # keys x_t + G (ln p up to a constant)
        xt = abs(t[_T["x_t"]])
        return float(3 * U32 * xt + gumbel_err(g) + U32 * (xt + abs(g)))
    p, q, r, xt, xq = (t[_T[n]] for n in ("p", "q", "r", "x_t", "x_q"))
    if not r > 0:
        return np.inf
    mt, mq = tr.draw_mean_abs_x[b]
    d_st = EPS_HW + 2 * U32 * mt + NSUM * U32
    d_sq = EPS_HW + 2 * U32 * mq + NSUM * U32
    dp = 2 * U32 * abs(xt) + EPS_HW + d_st + 2 * U32
    dq = 2 * U32 * abs(xq) + EPS_HW + d_sq + 2 * U32
    rel = (dp * p + dq * q + U32 * r) / r
    if rel >= 0.5:
        return np.inf
    lnr = abs(np.log(r))
    return float(rel / (1 - rel) + (EPS_HW + 2 * U32) * lnr + gumbel_err(g) + U32 * (lnr + abs(g)))


def compare_verify(gpu_tokens, gpu_len, tr):
    """Bit-exact comparison of emitted tokens and lengths.

    A sequence whose oracle trace took an acceptance decision with
    |u - p/q| < 1e-6 is compared only up to that decision.  Otherwise lengths
    and every token must match, except that the final token of a sampled
    sequence (its residual or bonus draw) may differ when the two keys lie
    within their fp32 error bounds of each other (draw_key_err): the GPU's
    token must then be among the oracle's best keys, in the residual's
    support, and its key plus its bound must reach the oracle's best key
    minus that key's bound.  Returns the number of sequences excluded by
    either rule."""
    gpu_tokens = np.asarray(gpu_tokens)
    gpu_len = np.asarray(gpu_len)
    excluded = 0
    for b in range(len(gpu_len)):
        k = int(tr.near_tie_k[b])
        if k > 0:
            excluded += 1
            np.testing.assert_array_equal(gpu_tokens[b, :k - 1], tr.out_tokens[b, :k - 1], err_msg=f"seq {b}")
            continue
        n = int(tr.out_len[b])
        assert gpu_len[b] == n, f"seq {b}: len {gpu_len[b]} vs oracle {n}"
        np.testing.assert_array_equal(gpu_tokens[b, :n - 1], tr.out_tokens[b, :n - 1], err_msg=f"seq {b}")
        np.testing.assert_array_equal(gpu_tokens[b, n:], tr.out_tokens[b, n:], err_msg=f"seq {b} padding")
        got, ref = int(gpu_tokens[b, n - 1]), int(tr.out_tokens[b, n - 1])
        if got == ref:
            continue
        assert tr.kind[b] in (1, 2), f"seq {b}: greedy token {got} vs oracle {ref}"
        hit = np.flatnonzero(tr.draw_idx[b] == got)
        assert hit.size, f"seq {b}: drawn token {got} is not among the oracle's best keys"
        j = int(hit[0])
        if tr.kind[b] == 1 and not tr.draw_fallback[b]:
            assert tr.draw_terms[b, j, _T["r"]] > 0, f"seq {b}: token {got} outside the residual's support"
        gap = tr.draw_key[b, 0] - tr.draw_key[b, j]
        bound = draw_key_err(tr, b, j) + draw_key_err(tr, b, 0)
        assert gap <= bound, f"seq {b}: token {got} key {gap:.3e} below the best, bound {bound:.3e}"
        note(f"  seq {b}: draw near-tie, token {got} vs {ref}, key gap {gap:.2e} <= bound {bound:.2e}")
        excluded += 1
    return excluded
