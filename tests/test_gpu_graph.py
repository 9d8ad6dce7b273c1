"""A whole draft-verify cycle (ctx_fuse, block_attn per layer, spec_verify)
captured into HIP graphs and replayed: every replay must reproduce the eager
outputs bit for bit, with eager work and synchronisations between replays.
The library's calls only launch kernels (no memset, no allocation, no host
synchronisation), so they can be captured as they are."""

import numpy as np
import pytest
import torch

from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, dev, note

pytestmark = pytest.mark.gpu


def _cycle_inputs(seed=21, B=4, S=1000, L=2, V=4096):
    import block_speculative_decoding_amd as dfl
    n_new = synth.new_rows(seed, B)
    ctx = np.full(B, S, dtype=np.int32)
    lens = (ctx + n_new).astype(np.int32)
    table, npages = synth.page_table(seed, ctx + 8, spare_pages=2)
    g = torch.Generator(device="cuda").manual_seed(seed)
    kc = [torch.randn((npages, 8, 2048), generator=g, device="cuda").to(BF16) for _ in range(L)]
    vc = [torch.randn((npages, 8, 2048), generator=g, device="cuda").to(BF16) for _ in range(L)]
    slots, pos = [], []
    for b in range(B):
        for r in range(n_new[b]):
            t = ctx[b] + r
            slots.append(table[b, t // 16] * 16 + t % 16)
            pos.append(t)
    M = len(slots)
    hs = [dev(h, BF16) for h in synth.capture_states(seed, M)]
    w = {k: dev(v, BF16) for k, v in synth.fuse_weights(seed, L).items()}
    ht = torch.empty((M, 2560), dtype=BF16, device="cuda")
    fuse = dfl.prepare_ctx_fuse(hs, w["wc"], w["gc"], w["wkv"], w["gk"], dev(np.array(pos, np.int32), torch.int32),
                                dev(np.array(slots, np.int64), torch.int64), kc, vc, ht_out=ht)
    attn = []
    for l in range(L):
        blk = {k: dev(v, BF16) for k, v in synth.attn_block(seed, B, layer=l).items()}
        attn.append(dfl.prepare_block_attn(blk["q"], blk["k_blk"], blk["v_blk"], blk["gq"], blk["gk"], kc[l], vc[l],
                                           dev(table, torch.int32), dev(lens, torch.int32)))
    zt, zd = synth.logits(seed, B, V, 4.0, 1.0)
    temp = np.array([0.0, 0.7, 1.0, 0.7], dtype=np.float32)[:B]
    d = synth.sample_drafts(seed, zd.astype(np.float32), temp)
    verify = dfl.prepare_spec_verify(dev(zt, BF16), dev(zd, BF16), dev(d, torch.int32), dev(temp, F32), seed=seed)
    return fuse, attn, verify, (ht, kc, vc)


def _outputs(fuse, attn, verify, bufs):
    ht, kc, vc = bufs
    out = [ht.clone()] + [c.clone() for c in kc] + [c.clone() for c in vc]
    out += [a.out.clone() for a in attn]
    out += [t.clone() for t in verify.outputs[:2]]
    return out


def _step(fuse, attn, verify, offset):
    verify.args.offset = offset
    fuse()
    for a in attn:
        a()
    verify()


def test_cycle_graph_replays_match_eager():
    fuse, attn, verify, bufs = _cycle_inputs()
    eager = {}
    for off in (3, 4):
        _step(fuse, attn, verify, off)
        torch.cuda.synchronize()
        eager[off] = _outputs(fuse, attn, verify, bufs)
    graphs = {}
    for off in (3, 4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _step(fuse, attn, verify, off)
        graphs[off] = g
    torch.cuda.synchronize()
    for rep in range(3):
        for off in (3, 4):
            # eager work of the other offset in between
            _step(fuse, attn, verify, 7 - off)
            torch.cuda.synchronize()
            graphs[off].replay()
            torch.cuda.synchronize()
            got = _outputs(fuse, attn, verify, bufs)
            for i, (a, b) in enumerate(zip(got, eager[off])):
                assert torch.equal(a, b), f"replay {rep} offset {off}: output {i} differs"
    note(f"  3 replays x 2 graphs match eager (verify lengths {eager[3][-1].tolist()} / {eager[4][-1].tolist()})")
