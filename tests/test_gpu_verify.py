"""GPU parity of dflash_spec_verify against the oracle: bit-exact tokens and
lengths on shared Philox streams (near-ties counted and excluded)."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, dev, exact, compare_verify, note

pytestmark = pytest.mark.gpu


def _run(zt, zd, d, temp, seed, offset, dtype, B_check=None):
    import block_speculative_decoding_amd as dfl
    zt_d, zd_d = dev(zt, dtype), dev(zd, dtype)
    toks, lens, nt = dfl.spec_verify(zt_d, zd_d, dev(d, torch.int32), dev(temp, F32), seed=seed, offset=offset)
    torch.cuda.synchronize()
    sel = np.arange(zt.shape[0]) if B_check is None else np.asarray(B_check)
    tr = oracle.spec_verify_ref(exact(zt_d)[sel], exact(zd_d)[sel], d[sel], temp[sel], seed, offset)
    return toks.cpu().numpy()[sel], lens.cpu().numpy()[sel], int(nt.item()), tr, sel


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_verify_mixed_ragged_vocab(dtype):
    """B=24, V=50000 (ragged against both chunk sizes), temperatures mixed."""
    B, V, seed = 24, 50000, 11
    note(f"verify mixed B={B} V={V} {dtype}")
    zt, zd = synth.logits(seed, B, V, 3.0, 1.0)
    temp = np.array([0.0, 0.7, 1.0, 1.7] * (B // 4), dtype=np.float32)
    d = synth.sample_drafts(seed, exact(dev(zd, dtype)), temp)
    toks, lens, nt, tr, _ = _run(zt, zd, d, temp, 5, 17, dtype)
    excl = compare_verify(toks, lens, tr)
    assert excl <= 2
    assert nt == tr.near_ties
    assert np.all((lens >= 1) & (lens <= 8))


def test_verify_fp32_tiny_vocab():
    """B=1, V=4096, fp32, logits N(0, 3^2): independent draft rows, rows with
    draft = target + N(0,1), and planted matches; greedy and T=1."""
    V = 4096
    for variant in ("independent", "noisy", "planted"):
        rng = np.random.default_rng(0)
        zt = (rng.standard_normal((1, 8, V)) * 3).astype(np.float32)
        if variant == "independent":
            zd = (rng.standard_normal((1, 7, V)) * 3).astype(np.float32)
        else:
            zd = zt[:, :7] + rng.standard_normal((1, 7, V)).astype(np.float32)
        for T in (0.0, 1.0):
            temp = np.array([T], dtype=np.float32)
            if variant == "planted":
                d = np.argmax(zt[:, :7], -1).astype(np.int32)
            else:
                d = synth.sample_drafts(0, zd, temp)
            note(f"verify tiny fp32 {variant} T={T}")
            toks, lens, nt, tr, _ = _run(zt, zd, d, temp, 0, 0, F32)
            compare_verify(toks, lens, tr)
            if variant == "planted" and T == 0.0:
                assert lens[0] == 8


def test_verify_planted_rejections_and_all_accept():
    B, V = 16, 1024
    rng = np.random.default_rng(3)
    zt = rng.standard_normal((B, 8, V)).astype(np.float32)
    zd = zt[:, :7].copy()
    d = rng.integers(0, V, (B, 7)).astype(np.int32)
    # sequences 0..6: sampled rejection forced at k = b + 1; 7..13 greedy mismatch at k = b - 6
    for b in range(7):
        k = b + 1
        zt[b, k - 1, d[b, k - 1]] = -60.0
        zd[b, k - 1, d[b, k - 1]] = 60.0
    am = np.argmax(zt, -1)
    for b in range(7, 14):
        k = b - 6
        d[b] = am[b, :7]
        d[b, k - 1] = (am[b, k - 1] + 1) % V
    d[14] = am[14, :7]            # greedy, all accepted
    temp = np.ones(B, dtype=np.float32)
    temp[7:15] = 0.0              # 15: sampled with q == p -> all accepted, bonus draw
    toks, lens, nt, tr, _ = _run(zt, zd, d, temp, 9, 2, F32)
    compare_verify(toks, lens, tr)
    assert list(lens[:7]) == [1, 2, 3, 4, 5, 6, 7]
    assert list(lens[7:14]) == [1, 2, 3, 4, 5, 6, 7]
    assert lens[14] == 8 and lens[15] == 8


def test_verify_planted_near_tie_is_counted():
    """p(d)/q(d) placed 5e-7 above the acceptance uniform: both sides count it."""
    V = 8
    u = oracle.uniforms(4, 6, 0, 0, 1, 0)  # U(stream 0, b=0, k=1, i=0)
    target = float(u) + 5e-7
    zd = np.zeros((1, 7, V), dtype=np.float32)   # q uniform: q(x) = 1/8
    zt = np.zeros((1, 8, V), dtype=np.float32)
    # p(d) = e^a / (e^a + 7) = target / 8  ->  e^a = 7 target / (8 - target)
    zt[0, 0, 3] = np.float32(np.log(7 * target / (8 - target)))
    d = np.full((1, 7), 3, dtype=np.int32)
    temp = np.ones(1, dtype=np.float32)
    toks, lens, nt, tr, _ = _run(zt, zd, d, temp, 4, 6, F32)
    assert tr.near_ties == 1 and tr.near_tie_k[0] == 1
    assert nt == 1


def test_verify_strided_draft_view_and_determinism():
    """Draft rows given as rows 1..7 of a [B, 8, V] tensor (the drafter's
    output shifted by one row); two runs give identical results."""
    import block_speculative_decoding_amd as dfl
    B, V, seed = 6, 8192, 21
    zt, zd7 = synth.logits(seed, B, V, 4.0, 1.0)
    full = np.concatenate([np.zeros((B, 1, V), np.float32), zd7], axis=1)
    temp = np.array([0.0, 0.7, 1.0, 0.0, 0.7, 1.0], dtype=np.float32)
    zt_d, full_d = dev(zt, BF16), dev(full, BF16)
    zd_view = full_d[:, 1:]
    d = synth.sample_drafts(seed, exact(zd_view), temp)
    outs = [dfl.spec_verify(zt_d, zd_view, dev(d, torch.int32), dev(temp, F32), seed=1, offset=2) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    tr = oracle.spec_verify_ref(exact(zt_d), exact(zd_view), d, temp, 1, 2)
    compare_verify(outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), tr)


def test_verify_serving_batch_full_size():
    """Serving-batch shape: [64, 8, 262144] bf16, N(0, 4^2), draft = target +
    N(0, 1); first half greedy, second half T = 0.7."""
    B, V, seed = 64, 262144, 2
    note("verify serving batch B=64 V=262144")
    zt, zd = synth.logits(seed, B, V, 4.0, 1.0)
    temp = np.where(np.arange(B) < 32, 0.0, 0.7).astype(np.float32)
    zt_d, zd_d = dev(zt, BF16), dev(zd, BF16)
    del zt, zd
    d = synth.sample_drafts(seed, exact(zd_d), temp)
    import block_speculative_decoding_amd as dfl
    toks, lens, nt = dfl.spec_verify(zt_d, zd_d, dev(d, torch.int32), dev(temp, F32), seed=2, offset=5)
    torch.cuda.synchronize()
    toks, lens = toks.cpu().numpy(), lens.cpu().numpy()
    excl = 0
    for b0 in range(0, B, 8):
        sl = slice(b0, b0 + 8)
        tr = oracle.spec_verify_ref(exact(zt_d[sl]), exact(zd_d[sl]), d[sl], temp[sl], 2, 5,
                                    batch_offset=b0)
        excl += compare_verify(toks[sl], lens[sl], tr)
    note(f"  mean out_len {lens.mean():.2f}, excluded {excl}, near-ties {nt}")
    assert excl <= 3


def test_verify_only_step_b256_sampled_sequences():
    """Prefill workload's verify-only step: [256, 8, 262144] bf16 at T = 0.7
    (N(0, 4^2) target, draft = target + N(0, 1)); the GPU verifies all 256
    sequences in one call, the oracle checks 32 of them (every 8th) with their
    batch indices, since the decisions of a sequence depend only on its rows
    and its own counters."""
    B, V, seed = 256, 262144, 12
    note("verify-only B=256 V=262144")
    g = torch.Generator(device="cuda").manual_seed(seed)
    zt_d = (4.0 * torch.randn((B, 8, V), generator=g, device="cuda")).to(BF16)
    zd_d = (zt_d[:, :7].float() + torch.randn((B, 7, V), generator=g, device="cuda")).to(BF16)
    temp = np.full(B, 0.7, dtype=np.float32)
    pick = np.arange(0, B, 8)
    d = np.zeros((B, 7), dtype=np.int32)
    d[pick] = synth.sample_drafts(seed, exact(zd_d[pick]), temp[pick])
    import block_speculative_decoding_amd as dfl
    toks, lens, nt = dfl.spec_verify(zt_d, zd_d, dev(d, torch.int32), dev(temp, F32), seed=seed, offset=3)
    torch.cuda.synchronize()
    toks, lens = toks.cpu().numpy(), lens.cpu().numpy()
    assert np.all((lens >= 1) & (lens <= 8))
    excl = 0
    for b in pick:
        tr = oracle.spec_verify_ref(exact(zt_d[b:b + 1]), exact(zd_d[b:b + 1]), d[b:b + 1], temp[b:b + 1], seed, 3,
                                    batch_offset=int(b))
        excl += compare_verify(toks[b:b + 1], lens[b:b + 1], tr)
    note(f"  checked {len(pick)} sequences, excluded {excl}, near-ties {nt}")
    assert excl <= 2


def test_verify_single_stream_t1():
    """Single-stream shape: B = 1, V = 262144 bf16, N(0, 4^2) target, draft =
    target + N(0, 1), T = 1, four Philox offsets."""
    B, V, seed = 1, 262144, 31
    zt, zd = synth.logits(seed, B, V, 4.0, 1.0)
    temp = np.ones(B, dtype=np.float32)
    zt_d, zd_d = dev(zt, BF16), dev(zd, BF16)
    d = synth.sample_drafts(seed, exact(zd_d), temp)
    import block_speculative_decoding_amd as dfl
    excl = 0
    for off in range(4):
        toks, lens, nt = dfl.spec_verify(zt_d, zd_d, dev(d, torch.int32), dev(temp, F32), seed=seed, offset=off)
        torch.cuda.synchronize()
        tr = oracle.spec_verify_ref(exact(zt_d), exact(zd_d), d, temp, seed, off)
        excl += compare_verify(toks.cpu().numpy(), lens.cpu().numpy(), tr)
        note(f"  offset {off}: len {int(lens.cpu()[0])}")
    assert excl <= 1


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_verify_with_draft_stats_input(dtype):
    """The draft rows' statistics given as an input (as the shared head
    writes them; here the oracle's, rounded to fp32): verification reads no
    draft row for them and matches the oracle bit for bit."""
    import block_speculative_decoding_amd as dfl
    B, V, seed = 24, 50000, 13
    note(f"verify with draft stats B={B} V={V} {dtype}")
    zt, zd = synth.logits(seed, B, V, 3.0, 1.0)
    temp = np.array([0.0, 0.7, 1.0, 1.7] * (B // 4), dtype=np.float32)
    zt_d, zd_d = dev(zt, dtype), dev(zd, dtype)
    zfull = np.concatenate([np.zeros((B, 1, V)), exact(zd_d)], axis=1)
    st = oracle.draft_stats_ref(zfull, temp)
    d = synth.sample_drafts(seed, exact(zd_d), temp)
    toks, lens, nt = dfl.spec_verify(zt_d, zd_d, dev(d, torch.int32), dev(temp, F32), seed=5, offset=17,
                                     draft_stats=dev(st, F32))
    torch.cuda.synchronize()
    tr = oracle.spec_verify_ref(exact(zt_d), exact(zd_d), d, temp, 5, 17)
    excl = compare_verify(toks.cpu().numpy(), lens.cpu().numpy(), tr)
    assert excl <= 2
    assert int(nt.item()) == tr.near_ties


def test_verify_sampler_statistics_tiny_vocab():
    """The GPU sampler's own statistics, independent of the oracle's draws.

    8192 sequences share one fp32 (target, draft) logit pair at T = 1 and
    V = 64, and each draws its proposals d_k ~ q_k with numpy.  The accepted
    prefix length must follow the closed form P(n) = beta_1 ... beta_n
    (1 - beta_{n+1}), with beta_k = sum_x min(p_{k-1}(x), q_k(x)).  The
    first emitted token must follow p_0 (accepted d_1 or correction).  Where
    d_1 is rejected, the correction must follow max(0, p_0 - q_1)
    normalised.  Each is a chi-square test at p > 1e-4 on fixed seeds."""
    from scipy.stats import chisquare
    import block_speculative_decoding_amd as dfl
    B, V = 8192, 64
    rng = np.random.default_rng(404)
    zt1 = 1.5 * rng.standard_normal((8, V))
    zd1 = zt1[:7] + rng.standard_normal((7, V))
    zt1, zd1 = zt1.astype(np.float32), zd1.astype(np.float32)
    sm = lambda z: np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p, q = sm(zt1.astype(np.float64)), sm(zd1.astype(np.float64))
    d = np.stack([rng.choice(V, size=B, p=q[k]) for k in range(7)], axis=1).astype(np.int32)
    zt = np.broadcast_to(zt1, (B, 8, V)).copy()
    zd = np.broadcast_to(zd1, (B, 7, V)).copy()
    note(f"verify sampler statistics B={B} V={V}")
    toks, lens, _ = dfl.spec_verify(dev(zt, F32), dev(zd, F32), dev(d, torch.int32),
                                    torch.ones(B, dtype=torch.float32, device="cuda"), seed=77, offset=5)
    torch.cuda.synchronize()
    toks, lens = toks.cpu().numpy(), lens.cpu().numpy()

    def chi2(observed, expected):
        # Bins expected below 5 are pooled.
        small = expected < 5
        obs = np.append(observed[~small], observed[small].sum())
        exp_ = np.append(expected[~small], expected[small].sum())
        keep = exp_ > 0
        return chisquare(obs[keep], exp_[keep] * obs[keep].sum() / exp_[keep].sum()).pvalue

    beta = np.array([np.minimum(p[k], q[k]).sum() for k in range(7)])
    law = np.array([np.prod(beta[:n]) * (1 - beta[n]) for n in range(7)] + [np.prod(beta)])
    p_len = chi2(np.bincount(lens - 1, minlength=8).astype(float), B * law)
    p_first = chi2(np.bincount(toks[:, 0], minlength=V).astype(float), B * p[0])
    rej = lens == 1
    resid = np.maximum(p[0] - q[0], 0.0)
    p_resid = chi2(np.bincount(toks[rej, 0], minlength=V).astype(float), rej.sum() * resid / resid.sum())
    note(f"  beta={np.round(beta, 3)} p(len)={p_len:.3g} p(first)={p_first:.3g} "
         f"p(correction)={p_resid:.3g} ({rej.sum()} rejections at k=1)")
    assert np.all((lens >= 1) & (lens <= 8))
    assert p_len > 1e-4 and p_first > 1e-4 and p_resid > 1e-4
