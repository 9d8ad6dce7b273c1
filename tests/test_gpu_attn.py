"""GPU parity of dflash_block_attn against the oracle (max abs error 2e-2 in
bf16, 1e-4 in fp32), on ragged, paged, windowed and split-K cases."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, TOL, dev, exact, note
from tests.layout import k_offsets, v_offsets, pack, unpack

pytestmark = pytest.mark.gpu


def _case(ctx_lens, dtype, seed, window=0, split=0, spare=3):
    """Build a paged cache holding N(0,1) context K/V; unwritten slots and
    unused pages hold NaN, so any read of them shows in the output."""
    import block_speculative_decoding_amd as dfl
    B = len(ctx_lens)
    blk = synth.attn_block(seed, B)
    table, npages = synth.page_table(seed, [max(1, c) for c in ctx_lens], spare_pages=spare)
    kc = np.full((npages, 8, 2048), np.nan, dtype=np.float32)
    vc = np.full((npages, 8, 2048), np.nan, dtype=np.float32)
    kctx, vctx = [], []
    for b, S in enumerate(ctx_lens):
        k = synth.normal(seed, f"kctx{b}", (S, 8, 128))
        v = synth.normal(seed, f"vctx{b}", (S, 8, 128))
        pack(k, table[b], kc, k_offsets())
        pack(v, table[b], vc, v_offsets())
    kc_d, vc_d = dev(kc, dtype), dev(vc, dtype)
    kc_h, vc_h = exact(kc_d), exact(vc_d)
    for b, S in enumerate(ctx_lens):
        kctx.append(unpack(kc_h, table[b], S, k_offsets()))
        vctx.append(unpack(vc_h, table[b], S, v_offsets()))
    q, kb, vb, gq, gk = (dev(blk[n], dtype) for n in ("q", "k_blk", "v_blk", "gq", "gk"))
    cl = np.array(ctx_lens, dtype=np.int32)
    lse = torch.empty((B, 32, 8), dtype=torch.float32, device="cuda")
    out = dfl.block_attn(q, kb, vb, gq, gk, kc_d, vc_d, dev(table, torch.int32), dev(cl, torch.int32),
                         lse_out=lse, window=window, split_tokens=split)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_attn_ref(exact(q), exact(kb), exact(vb), exact(gq), exact(gk), kctx, vctx, cl,
                                         window=window)
    return exact(out), exact(lse), ref, ref_lse


BALANCED = -1   # DFLASH_SPLIT_BALANCED


@pytest.mark.parametrize("split", [0, 128, 256, BALANCED])
def test_attn_bf16_ragged_paged(split):
    lens = [0, 1, 37, 300, 129]
    note(f"attn bf16 lens={lens} split={split}")
    out, lse, ref, ref_lse = _case(lens, BF16, 3, split=split)
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[BF16]
    assert np.max(np.abs(lse - ref_lse)) <= 2e-2


@pytest.mark.parametrize("split", [0, 128, BALANCED])
def test_attn_bf16_window(split):
    lens = [100, 1500, 1024, 1041]
    note(f"attn bf16 window=1024 lens={lens} split={split}")
    out, lse, ref, ref_lse = _case(lens, BF16, 4, window=1024, split=split)
    err = np.max(np.abs(out - ref))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[BF16]


def test_attn_fp32_tiny_context():
    """B=1, S=128, fp32: one draft layer of the tiny configuration."""
    out, lse, ref, ref_lse = _case([128], F32, 0)
    err = np.max(np.abs(out - ref))
    note(f"attn fp32 S=128 max abs err {err:.3e}")
    assert err <= TOL[F32]
    assert np.max(np.abs(lse - ref_lse)) <= 1e-4


def test_attn_fp32_ragged_window():
    out, lse, ref, ref_lse = _case([0, 5, 77], F32, 1, window=40)
    assert np.max(np.abs(out - ref)) <= TOL[F32]


def test_attn_bf16_single_stream_4096():
    """Single-stream shape: B=1, S=4096 (auto split)."""
    out, lse, ref, ref_lse = _case([4096], BF16, 5)
    err = np.max(np.abs(out - ref))
    note(f"attn bf16 S=4096 max abs err {err:.3e}")
    assert err <= TOL[BF16]


def test_attn_bf16_balanced_ragged_batch():
    """Balanced pieces over 20 sequences of 1..3000 cached tokens (about 800
    tiles in 64 pieces per KV-head pair): pieces span several sequences, and
    sequences are cut by one or more piece boundaries."""
    lens = [int(x) for x in np.random.default_rng(21).integers(1, 3000, 20)]
    lens[3], lens[11] = 0, 2999
    note(f"attn bf16 balanced lens={lens}")
    out, lse, ref, ref_lse = _case(lens, BF16, 21, split=BALANCED)
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[BF16]
    assert np.max(np.abs(lse - ref_lse)) <= 2e-2


def _big_case(B, S, seed, check, n_new=None, split=0, also_split=None):
    """Full-size serving / long-context layer: caches filled on the device
    with N(0,1) bf16 (i.i.d., so layout-agnostic); sampled sequences are read
    back through the documented layout and checked against the oracle."""
    import block_speculative_decoding_amd as dfl
    lens = np.full(B, S, dtype=np.int32) if n_new is None else (S + n_new).astype(np.int32)
    table, npages = synth.page_table(seed, lens)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    kc = torch.randn((npages, 8, 2048), generator=gen, device="cuda", dtype=torch.float32).to(BF16)
    vc = torch.randn((npages, 8, 2048), generator=gen, device="cuda", dtype=torch.float32).to(BF16)
    blk = synth.attn_block(seed, B)
    q, kb, vb, gq, gk = (dev(blk[n], BF16) for n in ("q", "k_blk", "v_blk", "gq", "gk"))
    out = dfl.block_attn(q, kb, vb, gq, gk, kc, vc, dev(table, torch.int32), dev(lens, torch.int32),
                         split_tokens=split)
    torch.cuda.synchronize()
    out_h = exact(out)
    assert np.all(np.isfinite(out_h))
    diff = None
    if also_split is not None:
        # Every sequence, through the other work split: both compute the same
        # exact attention, so they may differ by at most the bar between them.
        out2 = dfl.block_attn(q, kb, vb, gq, gk, kc, vc, dev(table, torch.int32), dev(lens, torch.int32),
                              split_tokens=also_split)
        torch.cuda.synchronize()
        diff = float(np.max(np.abs(exact(out2) - out_h)))
        del out2
    errs = []
    for b in check:
        pages = torch.from_numpy(table[b][table[b] >= 0].astype(np.int64)).cuda()
        kb_h = kc.index_select(0, pages).float().cpu().numpy()
        vb_h = vc.index_select(0, pages).float().cpu().numpy()
        local = np.arange(len(pages))
        kctx = unpack(kb_h, local, int(lens[b]), k_offsets()).astype(np.float64)
        vctx = unpack(vb_h, local, int(lens[b]), v_offsets()).astype(np.float64)
        ref, _ = oracle.block_attn_ref(exact(q[b:b + 1]), exact(kb[b:b + 1]), exact(vb[b:b + 1]), exact(gq),
                                       exact(gk), [kctx], [vctx], lens[b:b + 1])
        errs.append(np.max(np.abs(out_h[b] - ref[0])))
        del kb_h, vb_h, kctx, vctx
    return max(errs) if also_split is None else (max(errs), diff)


def test_attn_serving_batch_full_size():
    """B=64, ctx 8192 + new rows (1..8), shuffled 16-token pages."""
    n_new = synth.new_rows(2, 64)
    err = _big_case(64, 8192, 2, check=[0, 31, 63], n_new=n_new)
    note(f"attn serving B=64 S=8192 sampled max abs err {err:.3e}")
    assert err <= TOL[BF16]


def test_attn_long_context_full_size():
    """B=4, S=131072: split-K with many chunks and the LSE merge."""
    err = _big_case(4, 131072, 3, check=[1])
    note(f"attn long context B=4 S=131072 sampled max abs err {err:.3e}")
    assert err <= TOL[BF16]


@pytest.mark.parametrize("shape", ["serving_ragged", "long_context"])
def test_attn_balanced_full_size(shape):
    """Balanced pieces at full size: the serving batch with ragged contexts
    (B = 64, 1024..8192 cached tokens, pieces cutting most sequences) and the
    long context (B = 4, S = 131072: every sequence spread over 16 pieces)."""
    if shape == "serving_ragged":
        # The pieces on even XCDs take 27 shares of the tiles and those on odd
        # ones 25, so nearly every sequence is cut; all 64 are compared with
        # the one-split-per-sequence result as well.
        n_new = synth.ragged_lengths(7, 64, 1024, 8192) - 8192
        err, diff = _big_case(64, 8192, 7, check=[0, 17, 40, 63], n_new=n_new, split=BALANCED, also_split=0)
        note(f"attn balanced {shape}: all 64 sequences within {diff:.3e} of one split per sequence")
        assert diff <= TOL[BF16]
    else:
        err = _big_case(4, 131072, 8, check=[2], split=BALANCED)
    note(f"attn balanced {shape} sampled max abs err {err:.3e}")
    assert err <= TOL[BF16]
