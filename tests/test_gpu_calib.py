"""Calibration kernels: the copy reproduces its source byte for byte, the
read's per-workgroup xors fold to the xor of the whole buffer, the gather's
to the xor of exactly the listed in-range chunks, and the MFMA loop's FLOP
count follows its grid and round count."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_calib_stream_copy_and_read():
    import block_speculative_decoding_amd as dfl
    sink = dfl.calib_sink()
    x = torch.randint(0, 256, (48 * 1024 * 1024 + 16 * 37,), dtype=torch.uint8, device="cuda")  # ragged tail
    y = torch.zeros_like(x)
    assert dfl.calib_stream(x, sink, dst=y) == x.numel()
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    words = x.view(torch.int32).cpu().numpy().reshape(-1, 4)
    want = np.bitwise_xor.reduce(words, axis=0)
    for grid in (0, 300, 4096):
        dfl.calib_stream(x, sink, grid=grid)
        torch.cuda.synchronize()
        n = grid or 2048
        got = np.bitwise_xor.reduce(sink[: n * 16].view(torch.int32).cpu().numpy().reshape(-1, 4), axis=0)
        assert np.array_equal(got, want), grid


def test_calib_gather_reads_the_listed_chunks():
    import block_speculative_decoding_amd as dfl
    sink = dfl.calib_sink()
    chunk = 8192
    x = torch.randint(0, 256, (64 * chunk + 4096 + 16 * 5,), dtype=torch.uint8, device="cuda")  # ragged last chunk
    nfull = x.numel() // chunk
    g = torch.Generator().manual_seed(3)
    ids = torch.randperm(nfull + 1, generator=g).to(torch.int32)
    ids = torch.cat([ids, torch.tensor([-1, nfull + 7, 2**31 - 1], dtype=torch.int32)])  # read nothing
    ids = ids[torch.randperm(ids.numel(), generator=g)].contiguous()
    words = x.view(torch.int32).cpu().numpy()
    want = np.zeros(4, dtype=np.int32)
    for c in ids.tolist():
        if 0 <= c:
            piece = words[c * chunk // 4: (c + 1) * chunk // 4]
            if piece.size:
                want ^= np.bitwise_xor.reduce(piece.reshape(-1, 4), axis=0)
    idd = ids.cuda()
    for grid in (0, 7, 300):
        assert dfl.calib_gather(x, idd, chunk, sink, grid=grid) == ids.numel() * chunk
        torch.cuda.synchronize()
        n = grid or 2048
        got = np.bitwise_xor.reduce(sink[: n * 16].view(torch.int32).cpu().numpy().reshape(-1, 4), axis=0)
        assert np.array_equal(got, want), grid


def test_calib_mfma_flops():
    import block_speculative_decoding_amd as dfl
    sink = dfl.calib_sink()
    f = dfl.calib_mfma(10, sink)
    torch.cuda.synchronize()
    assert f == 512 * 4 * 10 * 8 * 2 * 32 * 32 * 16
    s = sink[: 512 * 256 * 4].view(torch.float32)
    assert torch.isfinite(s).all() and float(s.abs().max()) > 0
