"""Seeded synthetic inputs of the hot-path workloads.

Shared by the tests (for both the HIP path and the CPU oracle) and by the
benchmark.  It draws random tensors and builds page tables; it contains none
of the method's arithmetic.  Every generator is keyed by (seed, tensor name),
so tensors do not shift when shapes elsewhere change.

Distributions follow the workload descriptions: hidden states N(0, 1);
weights N(0, 0.02^2); norm gains 1 + 0.1 N(0, 1); embeddings, block Q/K/V and cache
contents N(0, 1); target logits N(0, sigma^2) and draft logits = target
logits + N(0, noise^2).  Cache pages are physically shuffled.
"""

import zlib

import numpy as np

D, NCAPTURE, HQ, HKV, HEAD_DIM, BLOCK, PAGE, INTER = 2560, 5, 32, 8, 128, 8, 16, 5120


def gen(seed, name):
    return np.random.Generator(np.random.PCG64([int(seed), zlib.crc32(name.encode())]))


def normal(seed, name, shape, std=1.0, mean=0.0):
    x = gen(seed, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def capture_states(seed, M):
    """Five captured target states, each [M, 2560]."""
    return [normal(seed, f"hs{j}", (M, D)) for j in range(NCAPTURE)]


def fuse_weights(seed, num_layers):
    """W_c [2560, 12800], g_c [2560], W_KV [L*2048, 2560], g_k [L, 128]."""
    return {
        "wc": normal(seed, "wc", (D, NCAPTURE * D), std=0.02),
        "gc": normal(seed, "gc", (D,), std=0.1, mean=1.0),
        "wkv": normal(seed, "wkv", (num_layers * 2 * HKV * HEAD_DIM, D), std=0.02),
        "gk": normal(seed, "gk_ctx", (num_layers, HEAD_DIM), std=0.1, mean=1.0),
    }


def attn_block(seed, B, layer=0):
    """Block q [B,32,8,128], k_blk / v_blk [B,8,8,128], gq / gk [128]."""
    t = f"L{layer}"
    return {
        "q": normal(seed, "q" + t, (B, HQ, BLOCK, HEAD_DIM)),
        "k_blk": normal(seed, "kb" + t, (B, HKV, BLOCK, HEAD_DIM)),
        "v_blk": normal(seed, "vb" + t, (B, HKV, BLOCK, HEAD_DIM)),
        "gq": normal(seed, "gq" + t, (HEAD_DIM,), std=0.1, mean=1.0),
        "gk": normal(seed, "gk" + t, (HEAD_DIM,), std=0.1, mean=1.0),
    }


def page_table(seed, capacity_tokens, spare_pages=0):
    """Shuffled physical pages for sequences with the given token capacities.

    Returns (block_table int32 [B, max_pages] with -1 in unused entries,
    num_pages).  Physical page ids are a random permutation of all pages.
    """
    need = [(int(c) + PAGE - 1) // PAGE for c in capacity_tokens]
    max_pages = max(1, max(need))
    total = sum(need) + spare_pages
    perm = gen(seed, "pages").permutation(total).astype(np.int32)
    table = np.full((len(need), max_pages), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[o:o + n]
        o += n
    return table, max(total, 1)


def ragged_lengths(seed, B, lo, hi):
    """Context lengths uniform on [lo, hi]."""
    return gen(seed, "ctx_len").integers(lo, hi + 1, size=B).astype(np.int32)


def new_rows(seed, B, lo=1, hi=8):
    """Newly verified rows per sequence, uniform on [lo, hi]."""
    return gen(seed, "new_rows").integers(lo, hi + 1, size=B).astype(np.int32)


def draft_layer_weights(seed, layer=0):
    """One draft layer around attention: g_in [2560], W_QKV [6144, 2560],
    W_O [2560, 4096], g_post [2560], W_GU [10240, 2560], W_D [2560, 5120]."""
    t = f"L{layer}"
    return {
        "g_in": normal(seed, "g_in" + t, (D,), std=0.1, mean=1.0),
        "w_qkv": normal(seed, "w_qkv" + t, ((HQ + 2 * HKV) * HEAD_DIM, D), std=0.02),
        "w_o": normal(seed, "w_o" + t, (D, HQ * HEAD_DIM), std=0.02),
        "g_post": normal(seed, "g_post" + t, (D,), std=0.1, mean=1.0),
        "w_gu": normal(seed, "w_gu" + t, (2 * INTER, D), std=0.02),
        "w_d": normal(seed, "w_d" + t, (D, INTER), std=0.02),
    }


def conv_weights(seed, k):
    """DFlash2 block convolution: taps [k, 2560] ~ N(0, 0.2^2) and bias
    [2560] ~ N(0, 0.02^2)."""
    return normal(seed, f"w_conv{k}", (k, D), std=0.2), normal(seed, f"b_conv{k}", (D,), std=0.02)


def final_norm(seed):
    """Final RMSNorm gain [2560] after the last draft layer."""
    return normal(seed, "g_final", (D,), std=0.1, mean=1.0)


def embedding(seed, V):
    """Shared embedding table [V, 2560] ~ N(0, 1)."""
    return normal(seed, "emb", (V, D))


def head_weight(seed, V, std=0.05):
    """Shared LM head [V, 2560] ~ N(0, std^2): on unit-RMS states the logits
    have standard deviation std * sqrt(2560) (about 2.5 at the default)."""
    return normal(seed, "w_head", (V, D), std=std)


def head_input(seed, B):
    """Final-norm output of the last draft layer [B, 8, 2560] ~ N(0, 1)."""
    return normal(seed, "y_head", (B, BLOCK, D))


def head_temperatures(seed, B):
    """Per-sequence temperatures: a quarter greedy (0 or -1), the rest
    uniform on [0.3, 1.5]."""
    g = gen(seed, "head_temperature")
    t = g.uniform(0.3, 1.5, size=B).astype(np.float32)
    greedy = g.permutation(B)[:max(1, B // 4)]
    t[greedy] = np.where(np.arange(len(greedy)) % 2 == 0, 0.0, -1.0)
    return t


def anchors(seed, B, V):
    """Last verified token of each sequence, uniform on [0, V)."""
    return gen(seed, "anchors").integers(0, V, size=B).astype(np.int32)


def logits(seed, B, V, sigma, noise):
    """Target logits [B, 8, V] ~ N(0, sigma^2); draft = target[:, :7] + N(0, noise^2)."""
    zt = normal(seed, "zt", (B, BLOCK, V), std=sigma)
    zd = zt[:, :BLOCK - 1] + normal(seed, "zd_noise", (B, BLOCK - 1, V), std=noise)
    return zt, zd


def sample_drafts(seed, zd, temperature):
    """Harness-side proposals d_k: argmax of the draft row when greedy, else a
    draw from softmax(zd / T) by Gumbel-max with numpy's generator."""
    zd = np.asarray(zd, dtype=np.float64)
    B = zd.shape[0]
    d = np.empty((B, BLOCK - 1), dtype=np.int32)
    g = gen(seed, "drafts")
    for b in range(B):
        T = float(temperature[b])
        if T > 0:
            d[b] = np.argmax(zd[b] / T + g.gumbel(size=zd[b].shape), axis=-1)
        else:
            d[b] = np.argmax(zd[b], axis=-1)
    return d
