"""Shared LM head and draft sampling -- float64 reference.

Test infrastructure only (see the package docstring).

What the pages fix:
* [E4B] "The parameter count exposes the real cost": the drafter's output
  head is a copy of the target head, [262144, 2560] (65.1% of its
  parameters), because it must score the target's vocabulary; [DF2] 4.2:
  the target's unembedding head projects the output states back to
  vocabulary logits.
* [E4B] "The released serving cycle": one forward over the eight block
  positions predicts all seven future positions in parallel.

Readings (listed in the design notes as well):
* The head is applied to all eight block rows of the final-norm output
  (row 0, the anchor, is computed and not used); logits are stored in the
  storage type, and sampling reads the stored values.
* The normaliser of q_k = softmax(z_k / T) (the drafter's distribution that
  sampled verification divides by) is a statistic of the same stored row,
  so the head can hand it to verification, which then reads no draft row
  for it ([E4B] "Why exact verification preserves the target": the
  acceptance ratio p / q).
* Proposal k = 1..7 of sequence b comes from row k: greedy (T <= 0) takes
  the argmax (lowest index on ties); sampled takes the Gumbel-max draw
  argmax_i z_i / T + G_i with G_i = -ln(-ln U(2, b, k, i)) -- stream 2 of
  the verification uniform layout, reserved for draft sampling -- which is
  an exact draw from softmax(z / T).
"""

import numpy as np

from .philox import gumbel, uniform_row

DRAFT_STREAM = 2


def head_logits_ref(y, w_head):
    """z = y W_head^T: y [B, 8, D] -> [B, 8, V] float64 (unrounded)."""
    return np.asarray(y, dtype=np.float64) @ np.asarray(w_head, dtype=np.float64).T


def draft_keys(row, T, seed, offset, b, k):
    """Keys whose first maximum is proposal k of sequence b: the logits
    themselves when greedy (T <= 0), else z_i / T + G_i with the stream-2
    Gumbel noise of (b, k)."""
    row = np.asarray(row, dtype=np.float64)
    if not T > 0:
        return row
    return row / T + gumbel(uniform_row(seed, offset, DRAFT_STREAM, b, k, row.shape[0]))


def draft_stats_ref(z, temperature):
    """Softmax statistics of the proposal rows at each sequence's temperature,
    the normaliser of q_k = softmax(z[b, k] / T_b) that verification needs:
    for k = 1..7, m = max_i z[b, k, i] and s = sum_i exp((z[b, k, i] - m) / T_b),
    from the stored logits z [B, 8, V].  Greedy sequences (T <= 0) need none:
    (-inf, 0).  Returns float64 [B, 7, 2]."""
    z = np.asarray(z, dtype=np.float64)
    B = z.shape[0]
    out = np.zeros((B, 7, 2))
    for b in range(B):
        T = float(temperature[b])
        if not T > 0:
            out[b, :, 0] = -np.inf
            continue
        rows = z[b, 1:]
        m = np.max(rows, axis=-1)
        out[b, :, 0] = m
        out[b, :, 1] = np.sum(np.exp((rows - m[:, None]) / T), axis=-1)
    return out


def draft_sample_ref(z, temperature, seed=0, offset=0):
    """Proposals d [B, 7] int32 from stored logits z [B, 8, V] and the gap
    between the two largest keys of each draw (inf for greedy rows, where
    ties resolve to the lowest index exactly)."""
    z = np.asarray(z, dtype=np.float64)
    B, _, V = z.shape
    d = np.empty((B, 7), dtype=np.int32)
    gap = np.full((B, 7), np.inf)
    for b in range(B):
        T = float(temperature[b])
        for k in range(1, 8):
            row = z[b, k]
            if not T > 0:
                d[b, k - 1] = int(np.argmax(row))     # first maximum = lowest index
                continue
            keys = draft_keys(row, T, seed, offset, b, k)
            i = int(np.argmax(keys))
            d[b, k - 1] = i
            gap[b, k - 1] = keys[i] - np.max(np.delete(keys, i)) if V > 1 else np.inf
    return d, gap
