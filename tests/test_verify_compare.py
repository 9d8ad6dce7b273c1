"""Host logic of the verification parity rule (tests/gpu_util.py): a GPU
output equal to the oracle's passes with no exclusion; a different final
draw passes only inside the fp32 key bound and the residual's support; any
other difference fails.  The GPU outputs here are planted on the CPU."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import compare_verify, draw_key_err

V = 512


def _trace():
    rng = np.random.default_rng(4)
    zt = 3.0 * rng.standard_normal((6, 8, V))
    zd = zt[:, :7] + rng.standard_normal((6, 7, V))
    temp = np.array([0.0, 0.7, 1.0, 0.0, 0.7, 1.3])
    d = np.argmax(zd, axis=-1).astype(np.int32)
    d[1, 3] = (d[1, 3] + 1) % V
    return oracle.spec_verify_ref(zt, zd, d, temp, seed=2, offset=1)


def test_identical_output_has_no_exclusion():
    tr = _trace()
    assert compare_verify(tr.out_tokens.copy(), tr.out_len.copy(), tr) == 0


def test_runner_up_draw_fails_outside_the_bound():
    tr = _trace()
    sampled = [b for b in range(6) if tr.kind[b] in (1, 2)]
    assert sampled
    for b in sampled:
        toks = tr.out_tokens.copy()
        n = tr.out_len[b]
        toks[b, n - 1] = tr.draw_idx[b, 1]
        gap = tr.draw_key[b, 0] - tr.draw_key[b, 1]
        assert gap > draw_key_err(tr, b, 0) + draw_key_err(tr, b, 1)
        with pytest.raises(AssertionError):
            compare_verify(toks, tr.out_len, tr)


def test_near_tie_draw_inside_the_bound_is_counted():
    tr = _trace()
    b = next(b for b in range(6) if tr.kind[b] == 1)
    tr.draw_key[b, 1] = tr.draw_key[b, 0] - 0.5 * draw_key_err(tr, b, 0)   # planted near-tie
    toks = tr.out_tokens.copy()
    toks[b, tr.out_len[b] - 1] = tr.draw_idx[b, 1]
    assert compare_verify(toks, tr.out_len, tr) == 1
    # the same key gap, but the token outside the residual's support, fails
    tr.draw_terms[b, 1, 2] = 0.0
    with pytest.raises(AssertionError):
        compare_verify(toks, tr.out_len, tr)


def test_greedy_and_length_differences_fail():
    tr = _trace()
    b = next(b for b in range(6) if tr.kind[b] == 0)
    toks = tr.out_tokens.copy()
    toks[b, tr.out_len[b] - 1] = (toks[b, tr.out_len[b] - 1] + 1) % V
    with pytest.raises(AssertionError):
        compare_verify(toks, tr.out_len, tr)
    lens = tr.out_len.copy()
    lens[1] += 1 if lens[1] < 8 else -1
    with pytest.raises(AssertionError):
        compare_verify(tr.out_tokens, lens, tr)


def test_bound_is_small_for_typical_keys():
    tr = _trace()
    for b in range(6):
        if tr.kind[b] in (1, 2):
            e = draw_key_err(tr, b, 0)
            assert 1e-7 < e < 1e-4, e
