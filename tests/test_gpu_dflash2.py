"""GPU parity of DFlash2's variants against the oracle.

Block convolution (dflash_draft_mlp with conv_k = 3, 5 and the extremes 1, 8): x_out, y and the
stored h' against the oracle's chain from the same synthetic inputs.  bf16
bounds are those of the plain layer, plus one term: the stored h may be one
bf16 step from the oracle's.  A worst-case step in each of the k rows a
convolution output reads passes through the taps into h', and from there
into x_out and y.  fp32: 1e-4.

Path selector (dflash_draft_paths) on synthetic logits:
- candidate ids must match bit for bit; both sides order the same stored
  logits, ties to the lower id.
- log-probabilities and entropies must be within 1e-4.
- every GPU path must score, under the oracle, within 1e-3 of the oracle's
  path of the same rank.  Paths must be distinct.  Paths whose oracle score
  is more than 2e-3 from its neighbours' must match exactly.
- exact ties (duplicate logits) must order by the rank tuple on both sides."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, TOL, bf16_err, bf16_step, dev, exact, note

pytestmark = pytest.mark.gpu


def _conv_extra(h_ref, w_conv, B):
    """Largest move of h' = h + conv(h) from one-step differences of the
    stored h in the rows each output reads: step(h_t) |1 + w_0| +
    sum_{j >= 1} |w_j| step(h_{t-j})."""
    k = w_conv.shape[0]
    st = bf16_step(h_ref).reshape(B, 8, -1)
    e = st * np.abs(1.0 + w_conv[0])
    for j in range(1, k):
        e[:, j:] += np.abs(w_conv[j]) * st[:, :-j]
    return e.reshape(B * 8, -1)


@pytest.mark.parametrize("B,k", [(3, 3), (40, 5), (1, 5), (2, 1), (2, 8)])
def test_conv_layer_bf16(B, k):
    import block_speculative_decoding_amd as dfl
    seed = 40 + k
    w = {n: dev(v, BF16) for n, v in synth.draft_layer_weights(seed).items()}
    wc, bc = (dev(v, BF16) for v in synth.conv_weights(seed, k))
    gf = dev(synth.final_norm(seed), BF16)
    x = dev(synth.normal(seed, "x", (B, 8, 2560)), BF16)
    o = dev(synth.normal(seed, "o", (B, 32, 8, 128)), BF16)
    hc = torch.empty_like(x)
    note(f"draft_mlp + block conv bf16 B={B} k={k}")
    x_out, y, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], g_final=gf, h_out=hc,
                                w_conv=wc, b_conv=bc)
    torch.cuda.synchronize()
    g = exact(gf)
    r = oracle.conv_mlp_ref(exact(x), exact(o), exact(w["w_o"]), exact(wc), exact(bc), exact(w["g_post"]),
                            exact(w["w_gu"]), exact(w["w_d"]), g_final=g, bf16=True)
    e_hc = _conv_extra(r["h"], exact(wc), B)
    e_x = e_hc + bf16_step(r["h_conv"]) + 4.0 * np.sqrt(bf16_step(r["s"]) ** 2 @ (exact(w["w_d"]).T ** 2))
    rms = np.sqrt(np.mean(oracle.bf16_round(r["x_out"]) ** 2, axis=-1, keepdims=True) + 1e-6)
    errs = [bf16_err(exact(hc).reshape(-1, 2560), r["h_conv"], e_hc),
            bf16_err(exact(x_out).reshape(-1, 2560), r["x_out"], e_x),
            bf16_err(exact(y).reshape(-1, 2560), r["y"], np.abs(g) / rms * (bf16_step(r["x_out"]) + e_x))]
    note(f"  error / bound h' / x_out / y: {errs}")
    assert max(errs) <= 1.0


def test_conv_layer_fp32_and_zero_kernel():
    import block_speculative_decoding_amd as dfl
    B, k, seed = 2, 3, 48
    w = {n: dev(v, F32) for n, v in synth.draft_layer_weights(seed).items()}
    wc, bc = (dev(v, F32) for v in synth.conv_weights(seed, k))
    x = dev(synth.normal(seed, "x", (B, 8, 2560)), F32)
    o = dev(synth.normal(seed, "o", (B, 32, 8, 128)), F32)
    hc = torch.empty_like(x)
    note("draft_mlp + block conv fp32 B=2 k=3")
    x_out, _, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], h_out=hc, w_conv=wc, b_conv=bc)
    # A zero kernel and bias give the plain layer, bit for bit.
    z_out, _, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], w_conv=torch.zeros_like(wc),
                                b_conv=torch.zeros_like(bc))
    plain, _, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"])
    torch.cuda.synchronize()
    r = oracle.conv_mlp_ref(exact(x), exact(o), exact(w["w_o"]), exact(wc), exact(bc), exact(w["g_post"]),
                            exact(w["w_gu"]), exact(w["w_d"]), bf16=False)
    e = max(float(np.max(np.abs(exact(hc).reshape(-1, 2560) - r["h_conv"]))),
            float(np.max(np.abs(exact(x_out).reshape(-1, 2560) - r["x_out"]))))
    note(f"  max abs err h' / x_out {e:.3e}")
    assert e <= TOL[F32]
    assert torch.equal(z_out, plain)


def _check_paths(out, z, m, P, lam, tol=1e-3):
    """Compare the selector's outputs with the oracle on the stored logits z
    [B, 8, V] (float64): candidate ids and paths bit-exact (both sides rank
    paths by the exact sum of stored candidate logits, ties by rank tuple),
    log-probabilities, entropies and scores within tol.  Returns the number
    of paths compared."""
    ids, logp, ent, paths, scores = (t.cpu().numpy() for t in out)
    r_ids, r_logp, r_ent, r_toks, r_scores, r_ranks = oracle.path_select_ref(z, m, P, lam)
    assert np.array_equal(ids, r_ids)
    fin = np.isfinite(r_logp)
    assert np.array_equal(np.isfinite(logp), fin) and np.all(logp[~fin] == -np.inf)
    assert float(np.max(np.abs(logp[fin] - r_logp[fin]), initial=0.0)) <= 1e-4
    assert float(np.max(np.abs(ent - r_ent))) <= 1e-4
    for b in range(z.shape[0]):
        bad = [p for p in range(P) if not np.array_equal(paths[b, p], r_toks[b, p])]
        assert not bad, (b, bad[:4], paths[b, bad[0]], r_toks[b, bad[0]])
        fin = np.isfinite(r_scores[b])
        assert np.array_equal(np.isfinite(scores[b]), fin) and np.all(scores[b][~fin] == -np.inf)
        err = float(np.max(np.abs(scores[b][fin] - r_scores[b][fin]), initial=0.0))
        assert err <= tol, err
    return z.shape[0] * P


@pytest.mark.parametrize("dtype,m,P", [(BF16, 4, 16), (BF16, 8, 64), (F32, 2, 7), (BF16, 1, 1), (F32, 3, 64)])
def test_paths_against_oracle(dtype, m, P):
    import block_speculative_decoding_amd as dfl
    B, V, lam = 5, 3 * 8192 + 384, 0.3
    z = synth.normal(60 + m, "zpaths", (B, 8, V), std=2.5)
    z_d = dev(z, dtype)
    note(f"draft_paths {dtype} B={B} V={V} m={m} P={P}")
    out = dfl.draft_paths(z_d, m, P, lam)
    torch.cuda.synchronize()
    n = _check_paths(out, exact(z_d), m, P, lam)
    note(f"  {n} paths bit-exact")


def test_paths_exact_ties_and_strides():
    # Duplicate logits at the top of a row give equal log-probabilities on
    # both sides: tied paths must follow the rank tuple.  The logits are a
    # view into a wider buffer (row stride > V).
    import block_speculative_decoding_amd as dfl
    B, V, m, P = 3, 8192 + 64, 3, 27
    z = synth.normal(70, "zties", (B, 8, V + 32), std=1.0)
    z[:, 1:, [5, 900, 8200]] = 9.0               # three-way tie at every position: 3^7 tied-first paths
    z[0, 3, 900] = 8.5
    zw = dev(z, BF16)
    view = zw[:, :, :V]
    out = dfl.draft_paths(view, m, P, 0.0)
    torch.cuda.synchronize()
    ids = out[0].cpu().numpy()
    assert np.all(ids[1:, :, :] == np.array([5, 900, 8200]))
    assert _check_paths(out, exact(view), m, P, 0.0) == B * P


def test_paths_neg_inf_candidates():
    # Masked rows: positions 1, 3, 4 and 6 have one finite logit, so with
    # m = 3 only 3^3 = 27 paths are finite and the remaining 37 of the top 64
    # run through -inf candidates: they follow, ordered by their number of
    # -inf candidates, the sum of their finite ones, then the rank tuple.
    import block_speculative_decoding_amd as dfl
    B, V, m, P = 2, 8192 + 64, 3, 64
    z = synth.normal(75, "zmask", (B, 8, V), std=2.0)
    for k in (1, 3, 4, 6):
        keep = z[:, k, 4000].copy()
        z[:, k, :] = -np.inf
        z[:, k, 4000] = keep
    z_d = dev(z, BF16)
    out = dfl.draft_paths(z_d, m, P, 0.5)
    torch.cuda.synchronize()
    assert _check_paths(out, exact(z_d), m, P, 0.5) == B * P
    assert int(np.isfinite(out[4].cpu().numpy()).sum()) == B * 27


def test_paths_full_vocabulary_batch64():
    # The serving shape: 64 sequences x 7 positions over V = 262144, m = 4,
    # P = 16; the oracle checks 8 of the 64 sequences in full.
    import block_speculative_decoding_amd as dfl
    B, V, m, P, lam = 64, 262144, 4, 16, 0.2
    note("draft_paths bf16 B=64 V=262144: generating logits")
    z = synth.normal(80, "zpaths_full", (B, 8, V), std=2.5)
    z_d = dev(z, BF16)
    del z
    out = dfl.draft_paths(z_d, m, P, lam)
    torch.cuda.synchronize()
    seqs = [0, 9, 21, 30, 38, 47, 55, 63]
    sub = tuple(t[seqs] for t in out)
    n = _check_paths(sub, exact(z_d[seqs]), m, P, lam)
    note(f"  sequences {seqs}: {n} paths bit-exact")
