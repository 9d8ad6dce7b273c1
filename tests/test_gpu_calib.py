"""Calibration kernels: the copy reproduces its source byte for byte, the
read's per-workgroup xors fold to the xor of the whole buffer, and the MFMA
loop's FLOP count follows its grid and round count."""

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


def test_calib_mfma_flops():
    import block_speculative_decoding_amd as dfl
    sink = dfl.calib_sink()
    f = dfl.calib_mfma(10, sink)
    torch.cuda.synchronize()
    assert f == 512 * 4 * 10 * 8 * 2 * 32 * 32 * 16
    s = sink[: 512 * 256 * 4].view(torch.float32)
    assert torch.isfinite(s).all() and float(s.abs().max()) > 0
