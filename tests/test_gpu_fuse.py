"""GPU parity of dflash_ctx_fuse against the oracle: the fused context H_t
and the K/V written at each slot (max abs error 2e-2 bf16, 1e-4 fp32)."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, TOL, dev, exact, note
from tests.layout import k_offsets, v_offsets, read_slots

pytestmark = pytest.mark.gpu


def _run(M, L, dtype, seed, npages, slots, pos, rows=None, sentinel=-7.0):
    import block_speculative_decoding_amd as dfl
    hs_np = synth.capture_states(seed, M)
    w = synth.fuse_weights(seed, L)
    hs = [dev(h, dtype) for h in hs_np]
    del hs_np
    wc, gc, wkv, gk = (dev(w[k], dtype) for k in ("wc", "gc", "wkv", "gk"))
    kcs = [torch.full((npages, 8, 2048), sentinel, dtype=dtype, device="cuda") for _ in range(L)]
    vcs = [torch.full((npages, 8, 2048), sentinel, dtype=dtype, device="cuda") for _ in range(L)]
    ht = torch.empty((M, 2560), dtype=dtype, device="cuda")
    dfl.ctx_fuse(hs, wc, gc, wkv, gk, dev(pos, torch.int32), dev(slots, torch.int64), kcs, vcs, ht_out=ht)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else np.asarray(rows)
    rsel = torch.from_numpy(rows).cuda()
    ht_ref, _, K, V = oracle.ctx_fuse_ref([exact(h.index_select(0, rsel)) for h in hs], exact(wc), exact(gc),
                                          exact(wkv), exact(gk), pos[rows], ht_bf16=(dtype == BF16))
    ht_err = np.max(np.abs(exact(ht.index_select(0, rsel)) - ht_ref))
    kv_err = 0.0
    for l in range(L):
        kg = read_slots(exact(kcs[l]), slots[rows], k_offsets())
        vg = read_slots(exact(vcs[l]), slots[rows], v_offsets())
        kv_err = max(kv_err, np.max(np.abs(kg - K[l])), np.max(np.abs(vg - V[l])))
    return ht_err, kv_err, kcs, vcs


def test_fuse_bf16_small_scattered():
    M, L, npages = 40, 2, 8
    rng = np.random.default_rng(0)
    slots = rng.permutation(npages * 16)[:M].astype(np.int64)
    pos = rng.integers(0, 131072, M).astype(np.int32)
    ht_err, kv_err, kcs, _ = _run(M, L, BF16, 1, npages, slots, pos)
    note(f"fuse bf16 M=40 L=2: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]
    # Slots not named keep their contents.
    untouched = np.setdiff1d(np.arange(npages * 16), slots)
    kk = read_slots(exact(kcs[0]), untouched, k_offsets())
    assert np.all(kk == -7.0)


def test_fuse_fp32_tiny_context():
    """M=128 context rows, one draft layer, fp32, positions 0..127."""
    M, L, npages = 128, 1, 8
    slots = np.arange(M, dtype=np.int64)
    pos = np.arange(M, dtype=np.int32)
    ht_err, kv_err, _, _ = _run(M, L, F32, 0, npages, slots, pos)
    note(f"fuse fp32 M=128: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[F32] and kv_err <= TOL[F32]


def test_fuse_skips_out_of_range_slots():
    M, L, npages = 16, 1, 2
    pos = np.arange(M, dtype=np.int32)
    # Every slot is negative or past the cache: nothing may be written.
    import block_speculative_decoding_amd as dfl
    hs = [dev(h, BF16) for h in synth.capture_states(2, M)]
    w = synth.fuse_weights(2, L)
    wc, gc, wkv, gk = (dev(w[k], BF16) for k in ("wc", "gc", "wkv", "gk"))
    kc = torch.full((npages, 8, 2048), -7.0, dtype=BF16, device="cuda")
    vc = torch.full((npages, 8, 2048), -7.0, dtype=BF16, device="cuda")
    bad = np.array([-1, -5, npages * 16, npages * 16 + 100] * 4, dtype=np.int64)
    dfl.ctx_fuse(hs, wc, gc, wkv, gk, dev(pos, torch.int32), dev(bad, torch.int64), [kc], [vc])
    torch.cuda.synchronize()
    assert torch.all(kc == -7.0) and torch.all(vc == -7.0)


def test_fuse_serving_new_rows():
    """Serving shape: 64 sequences x 1..8 newly verified rows (M = sum),
    five layers, appended at ctx_len .. ctx_len + n - 1 of shuffled pages."""
    B = 64
    n = synth.new_rows(2, B)
    M = int(n.sum())
    ctx = np.full(B, 8192, dtype=np.int32)
    table, npages = synth.page_table(2, ctx + 8)
    slots, pos = [], []
    for b in range(B):
        for r in range(n[b]):
            t = ctx[b] + r
            slots.append(table[b, t // 16] * 16 + t % 16)
            pos.append(t)
    slots = np.array(slots, dtype=np.int64)
    pos = np.array(pos, dtype=np.int32)
    ht_err, kv_err, _, _ = _run(M, 5, BF16, 2, npages, slots, pos)
    note(f"fuse serving M={M} L=5: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]


def test_fuse_prefill_full_size_sampled_rows():
    """Prefill shape: M=32768 rows, five layers, positions 0..32767; sampled
    rows checked one by one (fusion is row-independent)."""
    M, L = 32768, 5
    npages = M // 16
    slots = np.arange(M, dtype=np.int64)
    pos = np.arange(M, dtype=np.int32)
    rows = np.random.default_rng(5).choice(M, 48, replace=False)
    rows.sort()
    rows[-1] = M - 1
    ht_err, kv_err, _, _ = _run(M, L, BF16, 4, npages, slots, pos, rows=rows)
    note(f"fuse prefill M=32768 L=5 sampled: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]


def test_fuse_large_ragged_rows_scattered_slots():
    """M = 8292 (large-M kernel path, not a multiple of its 256-row tile), two
    layers, shuffled slots and positions; sampled rows checked."""
    M, L = 8292, 2
    npages = (M + 15) // 16 + 7
    rng = np.random.default_rng(9)
    slots = rng.permutation(npages * 16)[:M].astype(np.int64)
    pos = rng.integers(0, 131072, M).astype(np.int32)
    rows = np.sort(rng.choice(M, 40, replace=False))
    rows[-1] = M - 1
    ht_err, kv_err, _, _ = _run(M, L, BF16, 6, npages, slots, pos, rows=rows)
    note(f"fuse large ragged M={M} L={L}: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]


@pytest.mark.parametrize("M", [4095, 4096, 8191])
def test_fuse_path_boundary(M):
    """M = 4095 is the largest fusion on the split-K kernels, 4096 the
    smallest on the 256x256 kernel with the K/V epilogue (16 full row tiles),
    8191 that kernel with a ragged last row tile; one layer, shuffled slots,
    sampled rows checked."""
    L = 1
    npages = (M + 15) // 16 + 3
    rng = np.random.default_rng(M)
    slots = rng.permutation(npages * 16)[:M].astype(np.int64)
    pos = rng.integers(0, 65536, M).astype(np.int32)
    rows = np.sort(rng.choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ht_err, kv_err, _, _ = _run(M, L, BF16, 8, npages, slots, pos, rows=rows)
    note(f"fuse path boundary M={M}: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]


@pytest.mark.parametrize("M,L", [(384, 5), (385, 5), (2048, 1), (2049, 1)])
def test_fuse_kv_pair_boundary(M, L):
    """The K/V GEMM runs on two k-groups per workgroup with the K/V epilogue
    while its 128x128 tiles number at most 256: M = 384 at five layers and
    M = 2048 at one layer are the largest such fusions, 385 and 2049 the
    smallest on the split-K GEMM + K/V kernel.  Shuffled slots, sampled rows
    and the last row checked; slots not named keep their contents."""
    npages = (M + 15) // 16 + 5
    rng = np.random.default_rng(M + L)
    slots = rng.permutation(npages * 16)[:M].astype(np.int64)
    pos = rng.integers(0, 131072, M).astype(np.int32)
    rows = np.sort(rng.choice(M, 48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ht_err, kv_err, kcs, vcs = _run(M, L, BF16, 10, npages, slots, pos, rows=rows)
    note(f"fuse K/V path boundary M={M} L={L}: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]
    untouched = np.setdiff1d(np.arange(npages * 16), slots)
    assert np.all(read_slots(exact(kcs[L - 1]), untouched, k_offsets()) == -7.0)
    assert np.all(read_slots(exact(vcs[L - 1]), untouched, v_offsets()) == -7.0)


@pytest.mark.parametrize("shift", [16, 8])
def test_fuse_large_contiguous_slots_page_offsets(shift):
    """Large-M path with slots in order starting at `shift`: with 16 every full
    32-row block fills two whole pages (the V granule store), with 8 none does
    (element stores); M = 8200 leaves a partial last block either way.  Slots
    outside the written range must keep their sentinel."""
    M, L = 8200, 1
    npages = (M + shift + 15) // 16 + 2
    slots = shift + np.arange(M, dtype=np.int64)
    pos = np.arange(M, dtype=np.int32) + 5
    rows = np.sort(np.random.default_rng(11).choice(M, 40, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ht_err, kv_err, kcs, vcs = _run(M, L, BF16, 7, npages, slots, pos, rows=rows)
    note(f"fuse contiguous slots shift={shift} M={M}: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]
    untouched = np.setdiff1d(np.arange(npages * 16), slots)
    for cache, offs in ((kcs[0], k_offsets()), (vcs[0], v_offsets())):
        vals = read_slots(exact(cache), untouched, offs)
        assert np.all(vals == -7.0)


def test_fuse_single_stream_context_4096():
    """Single-stream shape: the 4096 context rows of one sequence fused into
    five layers (split-K path), slots and positions 0..4095; sampled rows."""
    M, L = 4096, 5
    npages = M // 16
    slots = np.arange(M, dtype=np.int64)
    pos = np.arange(M, dtype=np.int32)
    rows = np.sort(np.random.default_rng(13).choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ht_err, kv_err, _, _ = _run(M, L, BF16, 8, npages, slots, pos, rows=rows)
    note(f"fuse single stream M=4096 L=5: H_t err {ht_err:.3e}, K/V err {kv_err:.3e}")
    assert ht_err <= TOL[BF16] and kv_err <= TOL[BF16]
