"""Calls enqueued on a side stream keep their library-allocated workspace and
outputs: the wrapper marks them as in use on that stream, so memory
allocated and written on the default stream while the kernels still run
never lands in them."""

import numpy as np
import pytest
import torch

from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, dev, note

pytestmark = pytest.mark.gpu


def test_side_stream_call_with_default_stream_allocations():
    import block_speculative_decoding_amd as dfl
    B, V, seed = 64, 262144, 41
    note("side-stream verify B=64 V=262144")
    zt, zd = synth.logits(seed, B, V, 4.0, 1.0)
    temp = np.where(np.arange(B) % 2 == 0, 0.0, 0.7).astype(np.float32)
    zt_d, zd_d = dev(zt, BF16), dev(zd, BF16)
    del zt, zd
    d = synth.sample_drafts(seed, zd_d.float().cpu().numpy(), temp)
    d_d, t_d = dev(d, torch.int32), dev(temp, F32)
    ref_toks, ref_len, _ = dfl.spec_verify(zt_d, zd_d, d_d, t_d, seed=3, offset=9)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for trial in range(4):
        side.wait_stream(torch.cuda.current_stream())
        toks, lens, _ = dfl.spec_verify(zt_d, zd_d, d_d, t_d, seed=3, offset=9, stream=side)
        # default-stream allocations of the sizes just freed, written at once
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda") for n in (1 << 20, 1 << 16, 1 << 12, 256)]
        junk += [torch.full((B, 8), -7, dtype=torch.int32, device="cuda"), torch.full((B,), -7, dtype=torch.int32, device="cuda")]
        torch.cuda.synchronize()
        assert torch.equal(toks, ref_toks) and torch.equal(lens, ref_len), trial
        del junk
