"""The rest of a draft layer around block attention -- float64 reference.

Test infrastructure only (see the package docstring).

What the pages fix:
* [E4B] "The released serving cycle": the drafter's block has eight
  positions (the anchor, then seven mask positions) and one non-causal
  five-layer forward covers all of them.
* [DF2] 4.2 "Geteilte Embeddings & LM-Head": the anchor's input
  representation comes from the target's (shared, frozen) embedding table.
* [DF2] 4.1: Q_i = W_i^Q H_d and the block half of K_i / V_i is W_i^K H_d /
  W_i^V H_d, with H_d the draft tokens' hidden states; the context features
  bypass the drafter's Q, output projections and FFNs.
* [E4B] "Five target states become persistent draft context": Q is
  [B,32,8,128], block K/V [B,8,8,128].
* [E4B] opening section: the drafter is a five-layer "Qwen3-style" network;
  [E4B] "The parameter count exposes the real cost": 1,031,568,640 logical
  parameters, reproduced by the shapes below (intermediate width 5120 and
  two extra 2560-wide norm vectors are derived, not printed).

Readings where the pages are silent (listed in the design notes as well):
* "Qwen3-style" is read as the pre-norm decoder layer of that family:
      a  = RMSNorm(x; g_in)
      q, k, v = a W_Q^T, a W_K^T, a W_V^T       (then block attention)
      h  = x + o W_O^T                           (o: the attention output)
      c  = RMSNorm(h; g_post)
      x' = h + (silu(c W_G^T) * (c W_U^T)) W_D^T
  and after the last layer y = RMSNorm(x'; g_final).
* The seven mask positions all take the embedding row of one mask token id.
* Weight layouts, all [out, in] row-major: W_QKV [6144, 2560] = W_Q (head h
  at rows 128h..128h+127) | W_K (8 heads) | W_V (8 heads); W_O [2560, 4096]
  whose input index is 128 h + d for query head h, dim d; W_GU [10240, 2560]
  = W_G | W_U; W_D [2560, 5120].  No biases.
* In bf16 mode every stored activation is rounded to bf16 once, from its
  exact value: a, q/k/v, h, c, the SwiGLU product s = silu(g) * u (computed
  from the unrounded projections), x' and y.  Each function returns the
  unrounded float64 value of its outputs and consumes the rounded values of
  its inputs, so a GPU result is compared against the value it rounded.
"""

import numpy as np

from .common import bf16_round, rms_norm

D = 2560
HQ = 32
HKV = 8
HEAD_DIM = 128
BLOCK = 8
INTER = 5120


def layer_weight_shapes(d=D, hq=HQ, hkv=HKV, head_dim=HEAD_DIM, inter=INTER):
    """Shapes of one draft layer's tensors in the layouts above."""
    return {
        "g_in": (d,), "w_qkv": ((hq + 2 * hkv) * head_dim, d), "gq": (head_dim,), "gk": (head_dim,),
        "w_o": (d, hq * head_dim), "g_post": (d,), "w_gu": (2 * inter, d), "w_d": (d, inter),
    }


def _maybe_round(x, bf16):
    return bf16_round(x) if bf16 else np.asarray(x, dtype=np.float64)


def embed_block(emb, anchors, mask_id):
    """Block input H_d of layer 0: row 0 is the anchor's embedding, rows 1..7
    the mask token's ([E4B] "The released serving cycle", step 2; [DF2] 4.2).

    emb: [V, D]; anchors: [B] token ids; returns [B, 8, D] (an exact copy).
    """
    emb = np.asarray(emb)
    anchors = np.asarray(anchors, dtype=np.int64)
    out = np.empty((len(anchors), BLOCK, emb.shape[1]), dtype=emb.dtype)
    out[:, 0] = emb[anchors]
    out[:, 1:] = emb[int(mask_id)]
    return out


def qkv_ref(x, g_in, w_qkv, eps=1e-6, bf16=True, hq=HQ, hkv=HKV, head_dim=HEAD_DIM):
    """Input RMSNorm and the fused Q/K/V projection of the block ([DF2] 4.1,
    Q = W^Q H_d and the H_d halves of K, V).

    x: [B, 8, D] layer input.  Returns (q [B, hq, 8, hd], k [B, hkv, 8, hd],
    v [B, hkv, 8, hd], a [B*8, D]) in float64, q/k/v unrounded, a unrounded.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, d = x.shape
    a = rms_norm(x.reshape(B * T, d), g_in, eps)
    y = _maybe_round(a, bf16) @ np.asarray(w_qkv, dtype=np.float64).T
    nq, nk = hq * head_dim, hkv * head_dim
    q = y[:, :nq].reshape(B, T, hq, head_dim).transpose(0, 2, 1, 3)
    k = y[:, nq:nq + nk].reshape(B, T, hkv, head_dim).transpose(0, 2, 1, 3)
    v = y[:, nq + nk:nq + 2 * nk].reshape(B, T, hkv, head_dim).transpose(0, 2, 1, 3)
    return q, k, v, a


def silu(x):
    """x * sigmoid(x), the SwiGLU gate of the Qwen3 family."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def o_proj_residual_ref(x, o, w_o):
    """h = x + o' W_O^T, o' row (b, j) = concatenation over query heads h of
    o[b, h, j, :] (input index 128 h + d of W_O).  x: [B, 8, D] layer input;
    o: [B, hq, 8, hd].  Returns h [B*8, D] float64, unrounded."""
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    B, T, d = x.shape
    hq, hd = o.shape[1], o.shape[3]
    a_o = o.transpose(0, 2, 1, 3).reshape(B * T, hq * hd)
    return x.reshape(B * T, d) + a_o @ np.asarray(w_o, dtype=np.float64).T


def ffn_ref(h_s, g_post, w_gu, w_d, eps=1e-6, g_final=None, bf16=True):
    """From the stored residual h_s [M, D]: c = RMSNorm(h_s; g_post),
    s = silu(c W_G^T) * (c W_U^T), x' = h_s + s W_D^T and, when g_final is
    given, y = RMSNorm(x'; g_final).  Returns a dict of unrounded float64
    arrays c, s, x_out (and y); each stage consumes the bf16-rounded value of
    the previous one in bf16 mode."""
    h_s = np.asarray(h_s, dtype=np.float64)
    c = rms_norm(h_s, g_post, eps)
    gu = _maybe_round(c, bf16) @ np.asarray(w_gu, dtype=np.float64).T
    inter = gu.shape[1] // 2
    s = silu(gu[:, :inter]) * gu[:, inter:]
    x_out = h_s + _maybe_round(s, bf16) @ np.asarray(w_d, dtype=np.float64).T
    out = {"c": c, "s": s, "x_out": x_out}
    if g_final is not None:
        out["y"] = rms_norm(_maybe_round(x_out, bf16), g_final, eps)
    return out


def mlp_ref(x, o, w_o, g_post, w_gu, w_d, eps=1e-6, g_final=None, bf16=True):
    """Output projection + residual, post-attention RMSNorm, SwiGLU MLP +
    residual, and (after the last layer) the final RMSNorm: the composition
    of o_proj_residual_ref and ffn_ref on the stored h.

    x: [B, 8, D] layer input (the residual); o: [B, hq, 8, hd] attention
    output.  Returns a dict of float64 arrays, each unrounded, all [B*8, .]:
    h, c, s (the SwiGLU product), x_out and, when g_final is given, y.
    """
    h = o_proj_residual_ref(x, o, w_o)
    out = ffn_ref(_maybe_round(h, bf16), g_post, w_gu, w_d, eps, g_final, bf16)
    out["h"] = h
    return out
