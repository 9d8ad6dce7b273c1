"""CPU check of how block attention's fixed-split launch deals its work units
to the XCDs, restated from the launch and the kernel's index rules:

* units u = c + nsplit (hp + 4 b) for split c, KV-head pair hp, sequence b;
* the grid is the unit count rounded up to a multiple of 8 (the XCDs), and
  workgroup L (which the hardware places on XCD L mod 8) takes unit
  (L mod 8) per + L div 8 with per = grid / 8, doing nothing past the last
  unit.

Every unit must be taken by exactly one workgroup, each XCD's units must
form one contiguous range, and at the serving shape (one split, B = 64)
each XCD must hold whole sequences with all four head pairs."""

import pytest

XCDS = 8


def _deal(nsplit, B):
    units = nsplit * 4 * B
    grid = (units + XCDS - 1) // XCDS * XCDS
    per = grid // XCDS
    taken = {}
    for L in range(grid):
        u = (L % XCDS) * per + L // XCDS
        if u < units:
            assert u not in taken
            taken[u] = L % XCDS
    return units, taken


@pytest.mark.parametrize("nsplit,B", [(1, 1), (1, 3), (1, 64), (1, 65), (2, 5), (16, 4), (3, 7), (1, 1024)])
def test_every_unit_once_and_contiguous_per_xcd(nsplit, B):
    units, taken = _deal(nsplit, B)
    assert sorted(taken) == list(range(units))
    for x in range(XCDS):
        mine = sorted(u for u, xx in taken.items() if xx == x)
        if mine:
            assert mine == list(range(mine[0], mine[-1] + 1))


def test_serving_shape_whole_sequences_per_xcd():
    units, taken = _deal(1, 64)
    for x in range(XCDS):
        seqs = {}
        for u, xx in taken.items():
            if xx == x:
                hp, b = u % 4, u // 4
                seqs.setdefault(b, set()).add(hp)
        assert len(seqs) == 8 and all(h == {0, 1, 2, 3} for h in seqs.values())
