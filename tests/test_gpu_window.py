"""GPU parity of the sliding-window draft cache kept as a ring of pages:
dflash_ring_append against the oracle's append rule (bit-exact), and cycles
of append -> ctx_fuse -> block_attn(window) through a wrapped block table,
with every window token read back against the oracle's fused K/V and the
attention output against the oracle's windowed attention over its own fused
K/V (max abs 2e-2)."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, TOL, dev, exact, note
from tests.layout import k_offsets, unpack, v_offsets

pytestmark = pytest.mark.gpu


def test_ring_append_matches_oracle_over_chained_calls():
    import block_speculative_decoding_amd as dfl
    B, R, rows = 7, 5, 8
    rng = np.random.default_rng(21)
    ring = rng.permutation(B * R + 3)[:B * R].reshape(B, R).astype(np.int32)
    ctx = rng.integers(0, 500, size=B).astype(np.int32)
    ring_d, ctx_d = dev(ring, torch.int32), dev(ctx, torch.int32)
    note("ring_append B=7 R=5 rows=8, 3 calls")
    for call in range(3):
        n_new = rng.integers(-1, 11, size=B).astype(np.int32)   # includes clamped values
        slot, pos = dfl.ring_append(ring_d, ctx_d, dev(n_new, torch.int32), rows)
        torch.cuda.synchronize()
        r_slot, r_pos, r_len = oracle.ring_append(ring, ctx, n_new, rows)
        assert np.array_equal(slot.cpu().numpy(), r_slot)
        assert np.array_equal(pos.cpu().numpy(), r_pos)
        assert np.array_equal(ctx_d.cpu().numpy(), r_len)
        ctx = r_len


def test_windowed_cycles_through_ring_cache():
    import block_speculative_decoding_amd as dfl
    seed, B, L, W = 22, 2, 1, 128
    R = oracle.ring_pages(W)                       # 8 pages per sequence
    npages = B * R + 4
    rng = np.random.default_rng(seed)
    ring = rng.permutation(npages)[:B * R].reshape(B, R).astype(np.int32)
    ring_d = dev(ring, torch.int32)
    ctx_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    kc = torch.full((npages, 8, 2048), float("nan"), dtype=BF16, device="cuda")
    vc = torch.full((npages, 8, 2048), float("nan"), dtype=BF16, device="cuda")
    w = {k: dev(v, BF16) for k, v in synth.fuse_weights(seed, L).items()}
    k_of = [[] for _ in range(B)]                   # oracle K / V of each token, in order
    v_of = [[] for _ in range(B)]
    ctx = np.zeros(B, dtype=np.int32)

    def append(n_new, rows_per_seq, call):
        nonlocal ctx
        slot, pos = dfl.ring_append(ring_d, ctx_d, dev(n_new, torch.int32), rows_per_seq)
        M = B * rows_per_seq
        hs = [dev(h, BF16) for h in synth.capture_states(seed * 100 + call, M)]
        dfl.ctx_fuse(hs, w["wc"], w["gc"], w["wkv"], w["gk"], pos, slot, [kc], [vc])
        torch.cuda.synchronize()
        r_slot, r_pos, r_len = oracle.ring_append(ring, ctx, n_new, rows_per_seq)
        assert np.array_equal(slot.cpu().numpy(), r_slot) and np.array_equal(pos.cpu().numpy(), r_pos)
        hx = [exact(h) for h in hs]
        for b in range(B):
            n = int(r_len[b] - ctx[b])
            sel = slice(rows_per_seq * b, rows_per_seq * b + n)
            _, _, K, V = oracle.ctx_fuse_ref([h[sel] for h in hx], exact(w["wc"]), exact(w["gc"]), exact(w["wkv"]),
                                             exact(w["gk"]), ctx[b] + np.arange(n))
            k_of[b].extend(K[0])
            v_of[b].extend(V[0])
        ctx = r_len

    note("ring cache: prefill 200 tokens per sequence, W=128, R=8")
    for call, n in enumerate([64, 64, 64, 8]):
        append(np.full(B, n, dtype=np.int32), 64, call)
    max_pages = (int(ctx.max()) + 5 * 8 + 15) // 16 + 1
    table = ring[:, np.arange(max_pages) % R]
    table_d = dev(table, torch.int32)
    blk = synth.attn_block(seed, B)
    q, kb, vb, gq, gk = (dev(blk[n], BF16) for n in ("q", "k_blk", "v_blk", "gq", "gk"))
    for cycle in range(5):
        append(rng.integers(1, 9, size=B).astype(np.int32), 8, 10 + cycle)
        note(f"  cycle {cycle}: ctx_len {ctx.tolist()}")
        out = dfl.block_attn(q, kb, vb, gq, gk, kc, vc, table_d, ctx_d, window=W)
        torch.cuda.synchronize()
        # Window tokens read back through the wrapped table against the oracle's fused K/V.
        kh, vh = exact(kc), exact(vc)
        kctx, vctx = [], []
        for b in range(B):
            S = int(ctx[b])
            k_all = unpack(kh, table[b], S, k_offsets())
            v_all = unpack(vh, table[b], S, v_offsets())
            t0 = max(0, S - W)
            err = max(np.max(np.abs(k_all[t0:] - np.stack(k_of[b][t0:S]))),
                      np.max(np.abs(v_all[t0:] - np.stack(v_of[b][t0:S]))))
            assert err <= TOL[BF16], (cycle, b, err)
            # The attention oracle reads the oracle's own fused K/V as stored
            # in bf16 (positions before t0 are outside the window).
            kctx.append(oracle.bf16_round(np.stack(k_of[b][:S])))
            vctx.append(oracle.bf16_round(np.stack(v_of[b][:S])))
        o_ref, _ = oracle.block_attn_ref(exact(q), exact(kb), exact(vb), exact(gq), exact(gk), kctx, vctx, ctx,
                                         window=W)
        e = float(np.max(np.abs(exact(out) - o_ref)))
        note(f"    attention max abs err {e:.3e}")
        assert np.all(np.isfinite(exact(out))) and e <= TOL[BF16]
