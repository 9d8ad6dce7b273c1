"""Pins of oracle.window_cache: the ring of ceil(W/16) pages holds every
token of the window through any sequence of appends, one page fewer does
not, the window payload is the pages' 20 MiB per sequence, and the append
rule writes exactly the verified rows."""

import json
import os

import numpy as np
import pytest

from oracle.window_cache import PAGE, ring_append, ring_block_table, ring_pages

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_figures.json")))


def test_window_payload_matches_pages():
    # [E4B] "Cache and latency have separate break-even points": 5 layers,
    # 8 KV heads, 1024-token window, head width 128, bf16 K and V.
    W = 1024
    R = ring_pages(W)
    assert R == 64
    per_token = 5 * 8 * 128 * 2 * 2
    assert R * PAGE * per_token / 2 ** 20 == GOLD["cache_payload_per_seq_MiB"]["value"]
    assert ring_pages(100) == 7 and ring_pages(16) == 1


def _simulate(R, W, appends, start=0):
    """Write tokens through the ring and check that every token of the
    window [S - W, S) still sits in its slot after each append; returns the
    first failure (step, token) or None."""
    ring = np.arange(R)[None, :] + 1000          # one sequence, arbitrary page ids
    held = {}                                    # physical slot -> token it holds
    S = 0
    table = ring_block_table(ring, 4096)
    for step, n in enumerate([start] + list(appends)):
        rows = max(n, 1)
        slot, pos, new_len = ring_append(ring, [S], [n], rows)
        for j in range(n):
            held[int(slot[j])] = int(pos[j])
        S = int(new_len[0])
        for t in range(max(0, S - W), S):
            phys = int(table[0, t // PAGE]) * PAGE + t % PAGE
            if held.get(phys) != t:
                return step, t
    return None


@pytest.mark.parametrize("W", [16, 100, 256, 1024])
def test_ring_keeps_the_window(W):
    rng = np.random.default_rng(W)
    for trial in range(20):
        appends = rng.integers(0, 9, size=400)
        start = int(rng.integers(0, 3 * W))
        assert _simulate(ring_pages(W), W, appends, start) is None


@pytest.mark.parametrize("W", [40, 100, 256, 1024])
def test_one_page_fewer_loses_window_tokens(W):
    rng = np.random.default_rng(W + 1)
    failures = 0
    for trial in range(20):
        appends = rng.integers(1, 9, size=400)
        failures += _simulate(ring_pages(W) - 1, W, appends, int(rng.integers(0, 3 * W))) is not None
    assert failures > 0


def test_append_rows_positions_and_lengths():
    ring = np.array([[5, 9, 2], [7, 1, 3]])
    slot, pos, new_len = ring_append(ring, [30, 0], [3, 12], 8)   # 12 clamps to 8
    # sequence 0: tokens 30, 31 (page 1 -> ring[1] = 9), 32 (page 2 -> ring[2] = 2)
    assert slot[:3].tolist() == [9 * 16 + 14, 9 * 16 + 15, 2 * 16 + 0]
    assert pos[:3].tolist() == [30, 31, 32]
    assert (slot[3:8] == -1).all() and (pos[3:8] == 0).all()
    # sequence 1: tokens 0..7 on page 0 -> ring[0] = 7
    assert slot[8:16].tolist() == [7 * 16 + j for j in range(8)]
    assert new_len.tolist() == [33, 8]
    # no rows: nothing written, length unchanged
    s2, _, l2 = ring_append(ring, [30, 4], [0, -2], 8)
    assert (s2 == -1).all() and l2.tolist() == [30, 4]


def test_block_table_wraps():
    ring = np.array([[4, 8, 6]])
    t = ring_block_table(ring, 7)
    assert t.tolist() == [[4, 8, 6, 4, 8, 6, 4]]
