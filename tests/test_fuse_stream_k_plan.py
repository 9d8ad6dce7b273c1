"""CPU check of the stream-K schedule of the context fusion's first GEMM at
large M (256 x 256 tiles, 200 k-tiles of 64 each), restated from the
kernel's, the plan's and the norm kernel's rules:

* tiles are ordered in groups of 8 row tiles, row tile fastest within a
  group; their k-tiles are laid end to end, unit u = tile * 200 + k;
* with T tiles not a multiple of 256, q = ceil(200 T / 256) and the workgroup
  at position p (workgroup L sits at p = (L mod 8) * 32 + L div 8) takes units
  [p q, p q + q), writing each tile's piece to slot p - floor(t * 200 / q);
* the norm kernel adds, for tile t, slots 0 .. n_t - 1 with
  n_t = floor(((t + 1) 200 - 1) / q) - floor(t 200 / q) + 1.

Every unit must be computed exactly once, every slot the norm reads must have
been written for that tile, no two pieces may share a (tile, slot), and the
plan's slot count must bound them all."""

import pytest

NK, G, GROUP, TN = 200, 256, 8, 10


def tile_of(t, tiles_m):
    in_group = GROUP * TN
    first_m = t // in_group * GROUP
    gm = min(tiles_m - first_m, GROUP)
    q = t % in_group
    return first_m + q % gm, q // gm


def index_of(tm, tn, tiles_m):
    first_m = tm // GROUP * GROUP
    gm = min(tiles_m - first_m, GROUP)
    return first_m * TN + tn * gm + (tm - first_m)


@pytest.mark.parametrize("M", [4096, 4097, 6144, 8191, 8192, 8200, 8292, 12345, 20000, 40000, 131072])
def test_stream_k_runs_cover_every_unit_once(M):
    tiles_m = (M + 255) // 256
    T = tiles_m * TN
    for t in range(T):
        assert index_of(*tile_of(t, tiles_m), tiles_m) == t
    if T % G == 0:
        return  # whole rounds: one tile per workgroup, no stream-K
    q = -(-T * NK // G)
    slots = max(((t + 1) * NK - 1) // q - t * NK // q + 1 for t in range(T))
    assert slots <= 4
    seen, written = set(), {}
    per = G // 8
    for L in range(G):
        p = (L % 8) * per + L // 8
        u, end = p * q, min(T * NK, p * q + q)
        while u < end:
            t, kb = divmod(u, NK)
            ke = min(NK, kb + end - u)
            slot = p - t * NK // q
            assert 0 <= slot < slots
            assert (t, slot) not in written
            written[(t, slot)] = (kb, ke)
            for k in range(kb, ke):
                assert (t, k) not in seen
                seen.add((t, k))
            u += ke - kb
    assert len(seen) == T * NK
    for t in range(T):
        n = ((t + 1) * NK - 1) // q - t * NK // q + 1
        assert sorted(s for (tt, s) in written if tt == t) == list(range(n))
