"""Sliding-window draft cache on a ring of pages -- plain reference.

Test infrastructure only (see the package docstring).

[E4B] "Five target states become persistent draft context": the drafter's
own attention is limited to the latest 1,024 tokens; [E4B] "Cache and latency
have separate break-even points": five layers, eight KV heads, a 1,024-token
window, head width 128 and bf16 K/V make the per-sequence payload
(20 MiB).  A cache that only ever needs the latest W tokens can hold them in
a fixed ring of pages per sequence.

Readings (listed in the design notes as well):
* Logical token t of a sequence lives in logical page t // 16, slot t % 16;
  logical page p is stored in physical page ring[p mod R].  Attention reads
  logical pages through a block table whose entry p is ring[p mod R].
* Appending the rows verified in a cycle (verify's out_len of them) writes
  tokens ctx_len .. ctx_len + n - 1 and then advances ctx_len; only verified
  tokens enter the draft cache (block K/V are per cycle), so nothing is ever
  rolled back.
* Page p mod R with slot t % 16 makes the ring a ring of 16 R tokens:
  writing token t overwrites token t - 16 R, which is older than the window
  [S - W, S) whenever 16 R >= W.  So R = ceil(W / 16) pages per sequence
  suffice (for W = 1024, 64 pages: exactly the 20 MiB the pages give), and
  one page fewer does not (both pinned by simulation).  The first and the
  last page of a window may share a physical page; their window tokens sit
  in disjoint slots.
"""

import numpy as np

PAGE = 16


def ring_pages(window, page=PAGE):
    """Physical pages per sequence for a window of W tokens."""
    return -(-int(window) // page)


def ring_block_table(ring, max_pages):
    """Block table [B, max_pages] with entry p = ring[b][p mod R]."""
    ring = np.asarray(ring, dtype=np.int64)
    R = ring.shape[1]
    p = np.arange(max_pages)
    return ring[:, p % R].astype(np.int32)


def ring_append(ring, ctx_len, n_new, rows_per_seq):
    """Cache slots and positions of the rows appended this cycle.

    ring: [B, R] physical page ids; ctx_len: [B] tokens cached before the
    append; n_new: [B] rows appended (clamped to [0, rows_per_seq]).  Row
    rows_per_seq * b + j (j < n_new[b]) holds token ctx_len[b] + j: slot
    ring[b][(t // 16) mod R] * 16 + t % 16 and position t; the other rows get
    slot -1 (not written) and position 0.  Returns (slot int64, pos int32,
    new ctx_len int32).
    """
    ring = np.asarray(ring, dtype=np.int64)
    B, R = ring.shape
    slot = np.full(B * rows_per_seq, -1, dtype=np.int64)
    pos = np.zeros(B * rows_per_seq, dtype=np.int32)
    new_len = np.array(ctx_len, dtype=np.int64).copy()
    for b in range(B):
        n = min(max(int(n_new[b]), 0), rows_per_seq)
        for j in range(n):
            t = int(ctx_len[b]) + j
            slot[rows_per_seq * b + j] = ring[b, (t // PAGE) % R] * PAGE + t % PAGE
            pos[rows_per_seq * b + j] = t
        new_len[b] += n
    return slot, pos, new_len.astype(np.int32)
