"""Exact speculative verification -- float64 reference.

Test infrastructure only (see the package docstring).

Follows [E4B] "Why exact verification preserves the target" and [DF2] 4.4
"Garantie mathematischer Verlustfreiheit":

* sampled: proposal x_k is accepted with probability min(1, p(x)/q(x)); on
  rejection (uniform r > acceptance) the block stops and a replacement is
  drawn from normalize(max(0, p - q)); applied in order over the block it
  accepts the longest valid prefix;
* greedy (T = 0): proposals are accepted while they equal the target argmax;
  at the first mismatch the target token is taken;
* the block is eight long, so a cycle emits at most eight tokens including the
  target's correction or next (bonus) token ([E4B] "The released serving
  cycle").

Temperature: [DF2] 9 (FAQ Q3) says temperature scaling is applied to both the
draft and the target logits before the ratio is formed; its printed formula
(a ratio of p^(1/T)) is not normalised, so the reading used here is
p = softmax(z_target / T), q = softmax(z_draft / T); T <= 0 means greedy.

Row alignment (reading): draft row k-1 holds q for proposal d_k (k = 1..7);
target row k-1 holds p for the position of d_k; target row 7 is the bonus
position after all seven proposals.

Sampling (reading; any exact sampler has the right law, parity needs one
fixed sampler): the correction / bonus token is the Gumbel-max
argmax_i [ln r_i + G_i] over i with r_i > 0, G_i = -ln(-ln U(1, b, k, i));
the bonus uses ln p_i up to a constant, i.e. argmax_i [z_i / T + G_i] with
k = 8.  If the residual is identically zero it falls back to p.  Acceptance
compares u = U(0, b, k, 0) < p(d_k) / q(d_k) (q(d_k) = 0 gives +inf).  Greedy
ties go to the lowest index.  Token ids outside [0, V) are never accepted.
"""

from dataclasses import dataclass

import numpy as np

from .philox import uniforms, gumbel

BLOCK = 8
N_PROP = BLOCK - 1
NEAR_TIE = 1e-6
DRAW_TOP = 8
# Exact terms of a draw's key, per entry: p, q and r = max(0, p - q) (residual
# draws; bonus draws give p = q = r = nan), x_t = (z_t - max z_t) / T,
# x_q = (z_q - max z_q) / T (nan for bonus draws), the Gumbel noise G, and the
# log-weight w (key = w + G): ln r, or ln p in the zero-residual fallback, or
# z / T for the bonus.
DRAW_TERMS = ("p", "q", "r", "x_t", "x_q", "g", "w")


@dataclass
class VerifyTrace:
    out_tokens: np.ndarray   # [B, 8] int32, -1 padded
    out_len: np.ndarray      # [B] int32 in [1, 8]
    n_acc: np.ndarray        # [B] accepted proposals, 0..7
    kind: np.ndarray         # [B] 0 greedy, 1 residual draw, 2 bonus draw
    u: np.ndarray            # [B, 7] acceptance uniforms used (nan if unused)
    rho: np.ndarray          # [B, 7] p/q ratios evaluated (nan if unused)
    near_tie_k: np.ndarray   # [B] first k with |u - rho| < 1e-6 (0 = none)
    near_ties: int           # number of such decisions taken
    sample_gap: np.ndarray   # [B] top-2 key gap of the final draw (inf if greedy)
    # The final Gumbel-max draw of a sampled sequence, for checking a draw
    # computed in lower precision: its DRAW_TOP entries with the largest keys
    # (best first; -1 where unused or greedy), their keys and the exact terms
    # behind each key (DRAW_TERMS columns), whether the residual was
    # identically zero (the draw then used p), and the means of |x| under p
    # and q, x = (z - max z) / T, of the two rows a residual draw compares.
    draw_idx: np.ndarray = None    # [B, DRAW_TOP] int64
    draw_key: np.ndarray = None    # [B, DRAW_TOP]
    draw_terms: np.ndarray = None  # [B, DRAW_TOP, len(DRAW_TERMS)]
    draw_fallback: np.ndarray = None  # [B] bool
    draw_mean_abs_x: np.ndarray = None  # [B, 2] E_p|x_t|, E_q|x_q| (residual draws)


def _softmax(z):
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _top2(keys):
    """Index of the maximum (lowest index on ties) and the gap to the runner-up."""
    i = int(np.argmax(keys))
    best = keys[i]
    rest = np.delete(keys, i)
    second = np.max(rest) if rest.size else -np.inf
    return i, float(best - second)


def _record_draw(tr, b, keys, terms, fallback=False, mean_abs_x=(np.nan, np.nan)):
    """Keep the DRAW_TOP largest keys of a draw (ties to the lower index) and
    the exact terms of those entries."""
    order = np.argsort(-keys, kind="stable")[:DRAW_TOP]
    n = len(order)
    tr.draw_idx[b, :n] = order
    tr.draw_key[b, :n] = keys[order]
    tr.draw_terms[b, :n] = np.stack([terms[name][order] for name in DRAW_TERMS], axis=-1)
    tr.draw_fallback[b] = fallback
    tr.draw_mean_abs_x[b] = mean_abs_x


def spec_verify_ref(zt, zd, d, temperature, seed=0, offset=0, seq_block=4, batch_offset=0):
    """Verify one draft block per sequence.

    zt: target logits [B, 8, V]; zd: draft logits [B, 7, V]; d: proposals
    [B, 7]; temperature: [B] (0 = greedy).  Logits are taken as the exact
    stored values.  Sequences are processed ``seq_block`` at a time to bound
    memory; each sequence follows the sequential rule independently.
    ``batch_offset`` is the batch index of row 0 (it enters the random
    counters), so a slice of a batch can be verified on its own.
    """
    B, _, V = zt.shape
    d = np.asarray(d, dtype=np.int64)
    temperature = np.asarray(temperature, dtype=np.float64)
    tr = VerifyTrace(
        out_tokens=np.full((B, BLOCK), -1, dtype=np.int32),
        out_len=np.zeros(B, dtype=np.int32),
        n_acc=np.zeros(B, dtype=np.int32),
        kind=np.zeros(B, dtype=np.int32),
        u=np.full((B, N_PROP), np.nan),
        rho=np.full((B, N_PROP), np.nan),
        near_tie_k=np.zeros(B, dtype=np.int32),
        near_ties=0,
        sample_gap=np.full(B, np.inf),
        draw_idx=np.full((B, DRAW_TOP), -1, dtype=np.int64),
        draw_key=np.full((B, DRAW_TOP), -np.inf),
        draw_terms=np.full((B, DRAW_TOP, len(DRAW_TERMS)), np.nan),
        draw_fallback=np.zeros(B, dtype=bool),
        draw_mean_abs_x=np.full((B, 2), np.nan),
    )
    # Acceptance uniforms U(0, b, k, 0) for every sequence and k = 1..7.
    bb, kk = np.meshgrid(batch_offset + np.arange(B), np.arange(1, BLOCK), indexing="ij")
    u_all = uniforms(seed, offset, 0, bb, kk, np.zeros_like(bb))

    for s0 in range(0, B, seq_block):
        for b in range(s0, min(B, s0 + seq_block)):
            _verify_one(b, batch_offset + b, np.asarray(zt[b], np.float64), np.asarray(zd[b], np.float64),
                        d[b], float(temperature[b]), seed, offset, u_all[b], tr)
    return tr


def _verify_one(b, gb, zt, zd, d, T, seed, offset, u_b, tr):
    """Sequence at trace row b; gb is its batch index in the random counters."""
    V = zt.shape[-1]
    emitted = []
    if not T > 0.0:
        # Greedy (T <= 0): accept while d_k equals the target argmax of row k-1.
        n = 0
        for k in range(1, BLOCK):
            a = int(np.argmax(zt[k - 1]))
            if d[k - 1] == a:
                emitted.append(a)
                n += 1
            else:
                emitted.append(a)
                break
        else:
            emitted.append(int(np.argmax(zt[BLOCK - 1])))
        tr.kind[b] = 0
    else:
        n = 0
        done = False
        for k in range(1, BLOCK):
            p = _softmax(zt[k - 1] / T)
            q = _softmax(zd[k - 1] / T)
            x = int(d[k - 1])
            if 0 <= x < V:
                rho = p[x] / q[x] if q[x] > 0 else np.inf
            else:
                rho = 0.0
            u = u_b[k - 1]
            tr.u[b, k - 1] = u
            tr.rho[b, k - 1] = rho
            if abs(u - rho) < NEAR_TIE:
                tr.near_ties += 1
                if tr.near_tie_k[b] == 0:
                    tr.near_tie_k[b] = k
            if u < rho:
                emitted.append(x)
                n += 1
                continue
            r = np.maximum(0.0, p - q)
            fallback = not np.any(r > 0)
            if fallback:
                r = p
            g = gumbel(uniforms(seed, offset, 1, gb, k, np.arange(V)))
            with np.errstate(divide="ignore"):
                w = np.where(r > 0, np.log(r), -np.inf)
            keys = w + g
            x_new, gap = _top2(keys)
            emitted.append(x_new)
            tr.sample_gap[b] = gap
            tr.kind[b] = 1
            xt = (zt[k - 1] - np.max(zt[k - 1])) / T
            xq = (zd[k - 1] - np.max(zd[k - 1])) / T
            _record_draw(tr, b, keys, {"p": p, "q": q, "r": r, "x_t": xt, "x_q": xq, "g": g, "w": w},
                         fallback, (float(np.sum(p * np.abs(xt))), float(np.sum(q * np.abs(xq)))))
            done = True
            break
        if not done:
            g = gumbel(uniforms(seed, offset, 1, gb, BLOCK, np.arange(V)))
            w = zt[BLOCK - 1] / T
            keys = w + g
            x_new, gap = _top2(keys)
            emitted.append(x_new)
            tr.sample_gap[b] = gap
            tr.kind[b] = 2
            nan = np.full(V, np.nan)
            _record_draw(tr, b, keys, {"p": nan, "q": nan, "r": nan, "x_t": (zt[BLOCK - 1] - np.max(zt[BLOCK - 1])) / T,
                                       "x_q": nan, "g": g, "w": w})
    tr.n_acc[b] = n
    tr.out_len[b] = len(emitted)
    tr.out_tokens[b, :len(emitted)] = emitted
