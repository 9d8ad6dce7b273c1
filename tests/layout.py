"""Test-side packing of logical K/V into the paged cache layout that
include/dflash.h documents, and the inverse.  Written from the header's
formulas, independently of the kernels."""

import numpy as np

PAGE, HKV, HEAD_DIM = 16, 8, 128


def k_offsets():
    """[16, 128] element offsets of (token t, dim d) inside a K (page, head) block."""
    t = np.arange(PAGE)[:, None]
    d = np.arange(HEAD_DIM)[None, :]
    return 256 * ((d & 63) >> 3) + 8 * (t + 16 * (d >> 6)) + (d & 7)


def v_offsets():
    t = np.arange(PAGE)[:, None]
    d = np.arange(HEAD_DIM)[None, :]
    return 512 * (d >> 5) + 256 * ((t >> 2) & 1) + 8 * (d & 31) + (((t >> 3) << 2) | (t & 3))


def pack(logical, table_row, cache, offsets):
    """Write logical [S, 8, 128] tokens of one sequence into cache [P, 8, 2048]."""
    S = logical.shape[0]
    for t0 in range(0, S, PAGE):
        page = table_row[t0 // PAGE]
        n = min(PAGE, S - t0)
        blk = cache[page]  # [8, 2048]
        for h in range(HKV):
            blk[h, offsets[:n].reshape(-1)] = logical[t0:t0 + n, h].reshape(-1)


def unpack(cache, table_row, S, offsets):
    """Read logical [S, 8, 128] tokens of one sequence from cache [P, 8, 2048]."""
    t = np.arange(S)
    pages = np.asarray(table_row)[t // PAGE]
    idx = offsets[t % PAGE]  # [S, 128]
    return cache[pages[:, None, None], np.arange(HKV)[None, :, None], idx[:, None, :]]


def read_slots(cache, slots, offsets):
    """Gather [M, 8, 128] entries at physical token slots from cache [P, 8, 2048]."""
    slots = np.asarray(slots)
    page, t = slots // PAGE, slots % PAGE
    idx = offsets[t]  # [M, 128]
    return np.stack([cache[page[m]][:, idx[m]] for m in range(len(slots))])
