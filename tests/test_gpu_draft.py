"""GPU parity of the draft layer around block attention (dflash_draft_embed,
dflash_draft_qkv, dflash_draft_mlp) against the oracle.

The embedding copy is bit-exact.  Every other output is compared with the
oracle's unrounded float64 value, computed by the oracle's own chain from
the synthetic inputs (never from a GPU output).  The bound for fp32 is 1e-4.
For bf16 it is 2e-2 or, at magnitude 8 and above, half a bf16 step
(2^-8 |x|, with 10% slack): storing such a value in bf16 alone can move it
more than 2e-2.

Outputs computed from stored bf16 intermediates get more terms.  Such an
intermediate may be one bf16 step from the oracle's (its value sat near a
rounding midpoint), and the step passes on: one step of h into x_out; steps
of the SwiGLU product through W_D (rounding flips have random signs: 4
standard deviations with every element flipped); x_out's own step and what
reached it into y, scaled by g_final / rms.  In the full draft-layer chain
the attention outputs may be a step off too, which moves h through W_O."""

import numpy as np
import pytest
import torch

import oracle
from block_speculative_decoding_amd import synth
from tests.gpu_util import BF16, F32, TOL, bf16_err, bf16_step, dev, exact, note
from tests.layout import k_offsets, pack, v_offsets

pytestmark = pytest.mark.gpu

def _weights(seed, dtype, layer=0):
    return {k: dev(v, dtype) for k, v in synth.draft_layer_weights(seed, layer).items()}


def _max_err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_draft_embed_copies_rows(dtype):
    import block_speculative_decoding_amd as dfl
    V, B, mask = 4096, 6, 17
    emb = dev(synth.embedding(11, V), dtype)
    anchors = synth.anchors(11, B, V)
    anchors[2], anchors[4] = -1, V          # out of range: zero rows
    note(f"draft_embed {dtype} B={B} V={V}")
    x = dfl.draft_embed(emb, dev(anchors, torch.int32), mask)
    torch.cuda.synchronize()
    valid = (anchors >= 0) & (anchors < V)
    ref = oracle.embed_block(exact(emb), np.where(valid, anchors, 0), mask)
    ref[~valid, 0] = 0.0
    assert np.array_equal(exact(x), ref)


@pytest.mark.parametrize("B", [1, 3, 40, 80])
def test_draft_qkv_bf16_ragged_rows(B):
    # 8, 24, 320 and 640 block rows: one partial 128-row tile up to 5 tiles;
    # 640 rows run unsplit on two k-groups with the head-layout epilogue.
    import block_speculative_decoding_amd as dfl
    w = _weights(12, BF16)
    x = dev(synth.normal(12, "x", (B, 8, 2560)), BF16)
    note(f"draft_qkv bf16 B={B}")
    q, k, v = dfl.draft_qkv(x, w["g_in"], w["w_qkv"])
    torch.cuda.synchronize()
    qr, kr, vr, _ = oracle.qkv_ref(exact(x), exact(w["g_in"]), exact(w["w_qkv"]), bf16=True)
    err = max(bf16_err(exact(q), qr), bf16_err(exact(k), kr), bf16_err(exact(v), vr))
    note(f"  max error / bound {err:.3f}")
    assert err <= 1.0


def test_draft_qkv_fp32_tiny():
    import block_speculative_decoding_amd as dfl
    B = 2
    w = _weights(13, F32)
    x = dev(synth.normal(13, "x", (B, 8, 2560)), F32)
    note("draft_qkv fp32 B=2")
    q, k, v = dfl.draft_qkv(x, w["g_in"], w["w_qkv"])
    torch.cuda.synchronize()
    qr, kr, vr, _ = oracle.qkv_ref(exact(x), exact(w["g_in"]), exact(w["w_qkv"]), bf16=False)
    err = max(_max_err(exact(q), qr), _max_err(exact(k), kr), _max_err(exact(v), vr))
    note(f"  max abs err {err:.3e}")
    assert err <= TOL[F32]


def _mlp_check(x_in, o_in, w, g_final, h, x_out, y, chained):
    """Errors / bound of the GPU's h, x_out (and y) against the oracle's chain
    from the stored inputs x_in [B, 8, 2560] and o_in [B, 32, 8, 128]
    (float64).  Each stored intermediate may be one bf16 step from the
    oracle's: h moves x_out by its step; the SwiGLU product s moves it
    through W_D (4 standard deviations of random-sign steps in every
    element); x_out's own step and that move pass into y scaled by g / rms.
    Chained, o itself may be a step off anywhere, which moves h through W_O
    the same way."""
    gf = None if g_final is None else exact(g_final)
    r = oracle.mlp_ref(x_in, o_in, exact(w["w_o"]), exact(w["g_post"]), exact(w["w_gu"]), exact(w["w_d"]),
                       g_final=gf, bf16=True)
    h_ref, x_ref = r["h"], r["x_out"]
    e_h = 0.0
    if chained:
        a_o = np.asarray(o_in).transpose(0, 2, 1, 3).reshape(-1, 4096)
        e_h = 4.0 * np.sqrt(bf16_step(a_o) ** 2 @ (exact(w["w_o"]).T ** 2))
    e_x = bf16_step(h_ref) + e_h + 4.0 * np.sqrt(bf16_step(r["s"]) ** 2 @ (exact(w["w_d"]).T ** 2))
    errs = [bf16_err(exact(h).reshape(-1, 2560), h_ref, e_h), bf16_err(exact(x_out).reshape(-1, 2560), x_ref, e_x)]
    if gf is not None:
        rms = np.sqrt(np.mean(oracle.bf16_round(x_ref) ** 2, axis=-1, keepdims=True) + 1e-6)
        errs.append(bf16_err(exact(y).reshape(-1, 2560), r["y"], np.abs(gf) / rms * (bf16_step(x_ref) + e_x)))
    return errs


@pytest.mark.parametrize("B,final", [(1, False), (3, True), (40, True), (65, False), (128, True)])
def test_draft_mlp_bf16_ragged_rows(B, final):
    import block_speculative_decoding_amd as dfl
    w = _weights(14, BF16)
    gf = dev(synth.final_norm(14), BF16) if final else None
    x = dev(synth.normal(14, "x", (B, 8, 2560)), BF16)
    o = dev(synth.normal(14, "o", (B, 32, 8, 128)), BF16)
    h = torch.empty_like(x)
    note(f"draft_mlp bf16 B={B} final={final}")
    x_out, y, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], g_final=gf, h_out=h)
    # Without h_out the result is the same, bit for bit.
    x_out2, y2, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], g_final=gf)
    torch.cuda.synchronize()
    assert torch.equal(x_out, x_out2) and (y is None or torch.equal(y, y2))
    errs = _mlp_check(exact(x), exact(o), w, gf, h, x_out, y, chained=False)
    note(f"  max error / bound h / x_out / y: {errs}")
    assert max(errs) <= 1.0


def test_draft_mlp_fp32_tiny_against_composed_oracle():
    import block_speculative_decoding_amd as dfl
    B = 2
    w = _weights(15, F32)
    gf = dev(synth.final_norm(15), F32)
    x = dev(synth.normal(15, "x", (B, 8, 2560)), F32)
    o = dev(synth.normal(15, "o", (B, 32, 8, 128)), F32)
    note("draft_mlp fp32 B=2")
    x_out, y, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], g_final=gf)
    torch.cuda.synchronize()
    r = oracle.mlp_ref(exact(x), exact(o), exact(w["w_o"]), exact(w["g_post"]), exact(w["w_gu"]),
                       exact(w["w_d"]), g_final=exact(gf), bf16=False)
    errs = [_max_err(exact(x_out).reshape(-1, 2560), r["x_out"]), _max_err(exact(y).reshape(-1, 2560), r["y"])]
    note(f"  max abs err x_out / y: {errs}")
    assert max(errs) <= TOL[F32]


def test_draft_mlp_in_place_matches_out_of_place():
    import block_speculative_decoding_amd as dfl
    B = 5
    w = _weights(16, BF16)
    x = dev(synth.normal(16, "x", (B, 8, 2560)), BF16)
    o = dev(synth.normal(16, "o", (B, 32, 8, 128)), BF16)
    note("draft_mlp in place B=5")
    ref, _, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"])
    xi = x.clone()
    dfl.draft_mlp(xi, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], x_out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, ref)


def test_draft_layer_serving_batch_chain():
    """The serving batch (B = 64, 512 block rows) through embed -> qkv ->
    block_attn -> mlp (+ final norm), ragged short contexts on shuffled pages;
    every stage checked against the oracle's own chain from the same inputs."""
    import block_speculative_decoding_amd as dfl
    seed, B, V = 17, 64, 4096
    w = _weights(seed, BF16)
    gf = dev(synth.final_norm(seed), BF16)
    emb = dev(synth.embedding(seed, V), BF16)
    anchors = synth.anchors(seed, B, V)
    note("draft layer chain B=64")
    x = dfl.draft_embed(emb, dev(anchors, torch.int32), 3)
    q, kb, vb = dfl.draft_qkv(x, w["g_in"], w["w_qkv"])

    lens = synth.ragged_lengths(seed, B, 0, 96)
    table, npages = synth.page_table(seed, [max(1, int(c)) for c in lens])
    kc = np.zeros((npages, 8, 2048), dtype=np.float32)
    vc = np.zeros((npages, 8, 2048), dtype=np.float32)
    kctx, vctx = [], []
    for b, S in enumerate(lens):
        k_b = synth.normal(seed, f"kctx{b}", (int(S), 8, 128))
        v_b = synth.normal(seed, f"vctx{b}", (int(S), 8, 128))
        pack(k_b, table[b], kc, k_offsets())
        pack(v_b, table[b], vc, v_offsets())
        kctx.append(oracle.bf16_round(k_b))        # the cache as stored in bf16
        vctx.append(oracle.bf16_round(v_b))
    kc_d, vc_d = dev(kc, BF16), dev(vc, BF16)
    blk = synth.attn_block(seed, B)
    gq, gk = dev(blk["gq"], BF16), dev(blk["gk"], BF16)
    o = dfl.block_attn(q, kb, vb, gq, gk, kc_d, vc_d, dev(table, torch.int32), dev(lens, torch.int32))
    h = torch.empty_like(x)
    x_out, y, _ = dfl.draft_mlp(x, o, w["w_o"], w["g_post"], w["w_gu"], w["w_d"], g_final=gf, h_out=h)
    torch.cuda.synchronize()

    # The oracle's chain: each stage reads the previous stage's value as the
    # oracle stores it (rounded to bf16).
    ref_x = oracle.embed_block(exact(emb), anchors, 3)
    assert np.array_equal(exact(x), ref_x)
    qr, kr, vr, _ = oracle.qkv_ref(ref_x, exact(w["g_in"]), exact(w["w_qkv"]), bf16=True)
    e_qkv = max(bf16_err(exact(q), qr), bf16_err(exact(kb), kr), bf16_err(exact(vb), vr))
    o_ref, _ = oracle.block_attn_ref(oracle.bf16_round(qr), oracle.bf16_round(kr), oracle.bf16_round(vr),
                                     exact(gq), exact(gk), kctx, vctx, lens)
    e_attn = bf16_err(exact(o), o_ref)
    errs = _mlp_check(ref_x, oracle.bf16_round(o_ref), w, gf, h, x_out, y, chained=True)
    note(f"  max error / bound: qkv {e_qkv:.3f} attn {e_attn:.3f} h / x_out / y {errs}")
    assert max([e_qkv, e_attn] + errs) <= 1.0
