"""DFlash2 variants: depthwise block convolution and the top-m path
selector -- float64 reference.

Test infrastructure only (see the package docstring).

What the pages fix ([DF2] "DFlash & DFlash2: Block-Diffusion LLM-Speedup",
section "DFlash2", items 1 and 2):
* A depthwise 1-D convolution of kernel width k in {3, 5} sits between the
  drafter's attention and feed-forward sublayers; over a block of hidden
  states H (one row per block position) output row t is the sum over
  j = 0..k-1 of W_j (elementwise) H_{t-j}, plus a bias b.  Its cost is
  linear in k, the block length and the width.
* Instead of one token per block position the head yields the top-m
  candidates per position, and a path is scored as the sum over positions
  of log P_draft(chosen candidate) plus lambda times the entropy of
  P_draft at that position; unlikely branches are pruned and the best
  path(s) are handed to the target.

Readings (listed in the design notes as well):
* The convolution is a residual branch on the post-attention residual
  stream: h' = h + conv(h), applied to the stored h; positions before the
  anchor (t - j < 0) contribute zero, since the block is convolved on its
  own (the context lives only in the K/V cache).  Only the depthwise part
  the formula gives is applied (no pointwise mixing).  h' is stored, and
  the feed-forward half reads it in place of h.
* Scores use the draft head's own distribution P = softmax(z) of the stored
  logits of rows 1..7 (temperature 1).  The drafter proposes a whole block
  in one forward, so P at a position does not depend on the candidates
  chosen before it and a path's score separates per position.  The top-P
  paths of a separable score are then exactly what a beam of width P keeps
  position by position (a full path in the top P has its prefix in the top
  P of its length).  log P(x) = z(x) - lse of the position, and the lse
  terms and lambda * entropy shift every path by the same amount, so paths
  are ranked by the exact sum of their stored candidate logits; equal sums
  order by the candidate ranks, first position first (the lexicographically
  smaller rank tuple wins).  Exactness matters: stored bf16 logits lie on a
  coarse grid, different candidate combinations often have equal sums, and
  any rounding of a per-path score would decide those ties instead of the
  rule.  Candidates of a position order by logit, ties to the lower token
  id.
"""

from fractions import Fraction

import numpy as np

from .common import bf16_round
from .draft_layer import ffn_ref, o_proj_residual_ref


def depthwise_conv_ref(h, w_conv, b_conv):
    """conv(h)[b, t] = sum_{j < k, t - j >= 0} w_conv[j] * h[b, t - j] + b_conv.

    h: [B, T, D]; w_conv: [k, D]; b_conv: [D].  Returns [B, T, D] float64
    (the branch alone; the layer adds it to h)."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w_conv, dtype=np.float64)
    out = np.zeros_like(h) + np.asarray(b_conv, dtype=np.float64)
    T = h.shape[1]
    for t in range(T):
        for j in range(w.shape[0]):
            if t - j >= 0:
                out[:, t] += w[j] * h[:, t - j]
    return out


def conv_mlp_ref(x, o, w_o, w_conv, b_conv, g_post, w_gu, w_d, eps=1e-6, g_final=None, bf16=True):
    """The layer after attention with the convolution between its halves:
    h = x + o' W_O^T (stored), h' = h + conv(h) (stored), then the
    feed-forward half on h'.  x: [B, 8, D]; o: [B, hq, 8, hd].  Returns the
    dict of ffn_ref plus h and h_conv, all unrounded float64 [B*8, .]."""
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    h = o_proj_residual_ref(x, o, w_o)
    h_s = bf16_round(h) if bf16 else h
    hc = h_s + depthwise_conv_ref(h_s.reshape(B, T, D), w_conv, b_conv).reshape(B * T, D)
    out = ffn_ref(bf16_round(hc) if bf16 else hc, g_post, w_gu, w_d, eps, g_final, bf16)
    out["h"] = h
    out["h_conv"] = hc
    return out


def row_stats_ref(z, m):
    """Per row of logits z [..., V]: the top-m candidates (token ids, ordered
    by logit, ties to the lower id), their log-probabilities under
    softmax(z), and the entropy of softmax(z).  Returns (ids int32 [..., m],
    logp [..., m], entropy [...])."""
    z = np.asarray(z, dtype=np.float64)
    zmax = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    Z = np.sum(e, axis=-1, keepdims=True)
    p = e / Z
    logp_all = (z - zmax) - np.log(Z)
    with np.errstate(invalid="ignore"):
        ent = -np.sum(np.where(p > 0, p * logp_all, 0.0), axis=-1)
    # stable sort of -z: equal logits keep increasing id order
    ids = np.argsort(-z, axis=-1, kind="stable")[..., :m]
    logp = np.take_along_axis(logp_all, ids, axis=-1)
    return ids.astype(np.int32), logp, ent


def log_normaliser_ref(z):
    """lse = log sum_i e^(z_i) per row of z [..., V] (float64)."""
    z = np.asarray(z, dtype=np.float64)
    zmax = np.max(z, axis=-1)
    return zmax + np.log(np.sum(np.exp(z - zmax[..., None]), axis=-1))


def _path_order(n_neg_inf, total, ranks):
    """Sort key of a (partial) path: fewer -inf candidates first, then the
    larger exact sum of its finite candidate logits, then the
    lexicographically smaller rank tuple."""
    return (n_neg_inf, -total, ranks)


def top_paths_ref(ids, vals, entropy, P, lam, lse=None):
    """Top-P paths of one sequence through its positions.

    ids, vals: [J, m] candidates per position in rank order (token ids and
    their stored logits); entropy: [J]; lse: [J] log-normalisers of the
    positions (default 0).  log P of candidate r at position j is
    vals[j, r] - lse[j], so the score of the path with ranks (r_1..r_J),
    sum_j (vals[j, r_j] - lse[j]) + lam * sum_j entropy[j], differs between
    paths only by sum_j vals[j, r_j]: paths are ordered by that sum, taken
    EXACTLY (Fractions of the stored values, so that equal real sums are
    equal here), best first, equal sums by the lexicographically smaller
    rank tuple.  A -inf logit makes a path's sum -inf; such paths come after
    every finite one, ordered by their number of -inf candidates and then by
    the sum of their finite ones (the refinement keeps the order additive
    over positions, which is what makes the beam exact).  +inf and NaN
    logits are outside the domain.  Returns (tokens int32 [P, J], scores
    [P], ranks int32 [P, J]) via a beam of width P."""
    ids = np.asarray(ids)
    vals = np.asarray(vals, dtype=np.float64)
    J, m = vals.shape
    if np.any(np.isnan(vals)) or np.any(vals == np.inf):
        raise ValueError("candidate logits must be finite or -inf")
    lse = np.zeros(J) if lse is None else np.asarray(lse, dtype=np.float64)
    exact = [[None if v == -np.inf else Fraction(float(v)) for v in row] for row in vals]
    beam = [((), 0, Fraction(0))]            # (rank tuple, -inf count, exact finite sum)
    for j in range(J):
        ext = []
        for r, n, s in beam:
            for c in range(m):
                v = exact[j][c]
                ext.append((r + (c,), n + 1, s) if v is None else (r + (c,), n, s + v))
        ext.sort(key=lambda e: _path_order(e[1], e[2], e[0]))
        beam = ext[:P]
    shift = lam * float(np.sum(entropy)) - float(np.sum(lse))
    ranks = np.array([r for r, _, _ in beam], dtype=np.int32).reshape(len(beam), J)
    scores = np.array([-np.inf if n else float(s) + shift for _, n, s in beam])
    tokens = np.take_along_axis(ids[None, :, :].repeat(len(beam), 0), ranks[:, :, None], axis=2)[:, :, 0]
    return tokens.astype(np.int32), scores, ranks


def path_select_ref(z, m, P, lam):
    """The selector over a batch: z [B, 8, V] stored block logits; rows
    1..7 are the proposal positions.  Returns per sequence the candidates
    (ids [B, 7, m], logp [B, 7, m]), entropies [B, 7] and the top-P paths
    (tokens [B, P, 7], scores [B, P], ranks [B, P, 7])."""
    z = np.asarray(z, dtype=np.float64)
    ids, logp, ent = row_stats_ref(z[:, 1:], m)
    vals = np.take_along_axis(z[:, 1:], ids.astype(np.int64), axis=-1)
    lse = log_normaliser_ref(z[:, 1:])
    B = z.shape[0]
    toks, scores, ranks = [], [], []
    for b in range(B):
        t, s, r = top_paths_ref(ids[b], vals[b], ent[b], P, lam, lse[b])
        toks.append(t)
        scores.append(s)
        ranks.append(r)
    return ids, logp, ent, np.stack(toks), np.stack(scores), np.stack(ranks)
