"""Philox4x64-10 and the uniform / Gumbel layout of verification.

Test infrastructure only (see the package docstring).

The pages fix that rejection uses a uniform r ~ U(0, 1) ([DF2] 4.4,
"Garantie mathematischer Verlustfreiheit") but give no generator.  Both the
oracle and the GPU implement Philox4x64 with 10 rounds from its published
definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11): a 4 x 64-bit counter, a 2 x 64-bit key, per round two
64x64->128-bit products with the multipliers below, and a Weyl key schedule.
This module is pinned against numpy's independent Philox implementation.

Layout (a reading chosen here; the pages are silent):

    U(stream, b, k, i) = 23-bit half (i mod 2) of word ((i // 2) mod 4) of
        Philox4x64-10 with
        key     = (seed, 0)
        counter = (i // 8, 8*b + k, stream, offset)
    half 0: bits 41..63 of the word, half 1: bits 9..31
    u = (bits + 0.5) * 2**-23             -- exact in fp32, inside (0, 1)

so one Philox block serves eight consecutive entries (the two halves of a
uniformly random 64-bit word are independent uniform 32-bit values; each
keeps its top 23 bits).

stream 0: acceptance uniforms (i = 0, k = 1..7)
stream 1: Gumbel noise of the correction / bonus sample (k = 1..8, i < V)
stream 2: draft sampling (the proposals of rows 1..7 of the draft head).
"""

import numpy as np

M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = np.uint64(0x9E3779B97F4A7C15)
W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, b):
    """Full 64x64 -> 128-bit product of uint64 arrays, as (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.uint64(b)
    lo = a * b  # wraps mod 2**64
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    a0b0 = a0 * b0
    a0b1 = a0 * b1
    a1b0 = a1 * b0
    a1b1 = a1 * b1
    mid = (a0b0 >> _S32) + (a0b1 & _LO32) + (a1b0 & _LO32)
    hi = a1b1 + (a0b1 >> _S32) + (a1b0 >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64-10 block function.

    counter: uint64 array [..., 4]; key: pair (k0, k1) of uint64 (scalars or
    arrays broadcasting against counter[..., 0]).  Returns uint64 [..., 4].
    One round maps (x0, x1, x2, x3) to
        (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0))
    and the key is bumped by (W0, W1) between rounds.
    """
    with np.errstate(over="ignore"):
        c = np.asarray(counter, dtype=np.uint64)
        x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0 = np.asarray(key[0], dtype=np.uint64)
        k1 = np.asarray(key[1], dtype=np.uint64)
        for _ in range(10):
            hi0, lo0 = _mulhilo(x0, M0)
            hi1, lo1 = _mulhilo(x2, M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
            k0 = k0 + W0
            k1 = k1 + W1
        return np.stack([x0, x1, x2, x3], axis=-1)


def words_to_uniform(w, half=0):
    """u = (bits + 0.5) * 2**-23 of a word's 23-bit half (0: bits 41..63,
    1: bits 9..31), as float64 (exactly an fp32 value)."""
    w = np.asarray(w, dtype=np.uint64)
    half = np.asarray(half, dtype=np.uint64)
    shift = np.where(half == 0, np.uint64(41), np.uint64(9))
    bits = (w >> shift) & np.uint64(0x7FFFFF)
    return (bits.astype(np.float64) + 0.5) * 2.0 ** -23


def uniforms(seed, offset, stream, b, k, i):
    """U(stream, b, k, i) for broadcastable integer arrays b, k, i."""
    b, k, i = np.broadcast_arrays(np.asarray(b, dtype=np.uint64),
                                  np.asarray(k, dtype=np.uint64),
                                  np.asarray(i, dtype=np.uint64))
    ctr = np.stack([i >> np.uint64(3),
                    np.uint64(8) * b + k,
                    np.full(i.shape, stream, dtype=np.uint64),
                    np.full(i.shape, offset, dtype=np.uint64)], axis=-1)
    w = philox4x64_10(ctr, (np.uint64(seed), np.uint64(0)))
    word_idx = ((i >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(w, word_idx[..., None], axis=-1)[..., 0]
    return words_to_uniform(word, i & np.uint64(1))


def uniform_row(seed, offset, stream, b, k, n):
    """U(stream, b, k, i) for i = 0 .. n-1 (one Philox block per 8 entries)."""
    nb = (n + 7) // 8
    c0 = np.arange(nb, dtype=np.uint64)
    ctr = np.stack([c0,
                    np.full(nb, 8 * b + k, dtype=np.uint64),
                    np.full(nb, stream, dtype=np.uint64),
                    np.full(nb, offset, dtype=np.uint64)], axis=-1)
    w = philox4x64_10(ctr, (np.uint64(seed), np.uint64(0))).reshape(-1)   # words in order
    hi = words_to_uniform(w, 0)
    lo = words_to_uniform(w, 1)
    return np.stack([hi, lo], axis=-1).reshape(-1)[:n]                   # entry 2j: half 0 of word j


def gumbel(u):
    """Standard Gumbel noise G = -ln(-ln u) for u in (0, 1)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))
