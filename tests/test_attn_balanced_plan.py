"""CPU check of the bookkeeping of block attention's balanced pieces
(split_tokens = DFLASH_SPLIT_BALANCED), restated from the kernel's rules:

* sequence b contributes ceil((S_b - a0_b) / 32) context tiles plus its
  block tile; the tiles of all sequences lie end to end, TT in all;
* piece p (of 64) spans global tiles [floor(W_p TT / 1664), floor(W_(p+1) TT / 1664)),
  W_p = 52 floor(p / 2) + 27 (p mod 2): pieces on even XCDs (p even) take 27
  shares of the tiles, those on odd XCDs 25;
* a segment that holds a whole sequence is written directly; any other
  segment leaves a partial in slot 0 of its piece if its sequence is the
  piece's first, else slot 1;
* the merge of sequence b reads, for each non-empty piece P0..P1 it
  touches, slot 0, except in P0 where it reads slot 1 when P0 starts before
  b's first tile.

Every partial the merge reads must have been written for the same sequence,
none twice, every written partial must be read, and every sequence inside
one piece must be written directly."""

import random

K = 64


def _w(p):
    return 52 * (p // 2) + 27 * (p % 2)


def _tiles(S):
    return (S + 31) // 32 + 1 if S > 0 else 1


def _check(lens):
    B = len(lens)
    pref = [0]
    for S in lens:
        pref.append(pref[-1] + _tiles(S))
    TT = pref[-1]

    def lo(p):
        return _w(p) * TT // 1664

    def piece_of(t):                         # the last piece starting at or before t
        return max(p for p in range(K) if lo(p) <= t)

    writes, direct = {}, set()
    for piece in range(K):
        a, b_end = lo(piece), lo(piece + 1)
        if a >= b_end:
            continue
        first = max(b for b in range(B) if pref[b] <= a)
        b = first
        while b < B and pref[b] < b_end:
            nt = _tiles(lens[b]) - 1
            g0, g1 = max(a, pref[b]) - pref[b], min(b_end, pref[b + 1]) - pref[b]
            if g0 == 0 and g1 > nt:
                direct.add(b)
            else:
                key = (piece, 0 if b == first else 1)
                assert key not in writes
                writes[key] = b
            b += 1
    reads = {}
    for b in range(B):
        t0, t1 = pref[b], pref[b + 1] - 1
        P0, P1 = piece_of(t0), piece_of(t1)
        if P0 == P1:
            assert b in direct
            continue
        assert b not in direct
        slot0 = 0 if lo(P0) == t0 else 1
        for p in range(P0, P1 + 1):
            if lo(p) >= lo(p + 1):
                continue                     # empty piece: wrote nothing
            key = (p, slot0 if p == P0 else 0)
            assert writes.get(key) == b
            assert key not in reads
            reads[key] = b
    assert set(reads) == set(writes)


def test_balanced_plan_fixed_shapes():
    for lens in ([0, 1, 37, 300, 129], [8192] * 64, [131072] * 4, [0], [5], [0] * 70, [3000] * 3, [40] * 1024):
        _check(lens)


def test_balanced_plan_random_lengths():
    rng = random.Random(1)
    for _ in range(1500):
        n = rng.randint(1, 200)
        top = rng.choice([40, 700, 9000])
        _check([rng.randint(0, top) for _ in range(n)])


def test_piece_shares_follow_the_xcd_weights():
    # 64 pieces cover every tile once; even pieces hold 27/26 and odd ones
    # 25/26 of the mean share, to within a tile, and no piece exceeds the
    # bound the host plan sizes the page-id staging for (TT * 27 / 1664 + 2).
    for TT in (64, 1000, 16448, 262144):
        lo = [_w(p) * TT // 1664 for p in range(K + 1)]
        assert lo[0] == 0 and lo[K] == TT
        for p in range(K):
            size = lo[p + 1] - lo[p]
            share = TT / K * (27 if p % 2 == 0 else 25) / 26
            assert abs(size - share) <= 1
            assert size <= TT * 27 // 1664 + 2
