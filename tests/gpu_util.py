"""Helpers of the GPU parity tests: host<->device conversion and the
comparison rules for verification outputs."""

import sys

import numpy as np
import torch

BF16, F32 = torch.bfloat16, torch.float32
TOL = {BF16: 2e-2, F32: 1e-4}   # max abs error bars on attention / projection outputs
GAP_TOL = 1e-4                  # final-draw key gaps below this are counted as near-ties


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def exact(t):
    """Exact stored values of a device tensor as float64."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_step(v):
    """Spacing of bf16 values at |v|: 2^(e-7) for 2^e <= |v| < 2^(e+1)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def bf16_err(gpu, ref, extra=0.0):
    """Largest error of a stored bf16 output against the oracle's unrounded
    value, as a fraction of its bound max(2e-2, 1.1 * 2^-8 |ref|) + extra
    (pass: <= 1).  The first term is the storage rounding (half a step);
    extra carries one-step differences of stored intermediates."""
    gpu, ref = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    bound = np.maximum(TOL[BF16], 1.1 * 2.0 ** -8 * np.abs(ref)) + extra
    return float(np.max(np.abs(gpu - ref) / bound)) if gpu.size else 0.0


def compare_verify(gpu_tokens, gpu_len, tr, gap_tol=GAP_TOL):
    """Bit-exact comparison of emitted tokens and lengths.

    A sequence whose oracle trace took an acceptance decision with
    |u - p/q| < 1e-6 is compared only up to that decision; one whose final
    Gumbel-max draw had a top-2 key gap below gap_tol is compared except for
    that last token.  Returns the number of sequences so excluded.
    """
    gpu_tokens = np.asarray(gpu_tokens)
    gpu_len = np.asarray(gpu_len)
    excluded = 0
    for b in range(len(gpu_len)):
        k = int(tr.near_tie_k[b])
        if k > 0:
            excluded += 1
            np.testing.assert_array_equal(gpu_tokens[b, :k - 1], tr.out_tokens[b, :k - 1], err_msg=f"seq {b}")
            continue
        if tr.sample_gap[b] < gap_tol:
            excluded += 1
            assert gpu_len[b] == tr.out_len[b], f"seq {b}"
            n = tr.out_len[b]
            np.testing.assert_array_equal(gpu_tokens[b, :n - 1], tr.out_tokens[b, :n - 1], err_msg=f"seq {b}")
            continue
        assert gpu_len[b] == tr.out_len[b], f"seq {b}: len {gpu_len[b]} vs oracle {tr.out_len[b]}"
        np.testing.assert_array_equal(gpu_tokens[b], tr.out_tokens[b], err_msg=f"seq {b}")
    return excluded
