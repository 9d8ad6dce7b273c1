/*
 * dflash.h -- C ABI of the DFlash draft-verify hot path on AMD MI355X (gfx950).
 *
 * Three operations of the draft-verify hot path, each one call on a
 * caller-supplied HIP stream:
 *
 *   dflash_ctx_fuse    context fusion + K/V injection into the draft caches
 *   dflash_block_attn  one draft layer's non-causal attention for the 8-token block
 *   dflash_spec_verify exact speculative verification of the 7 proposals
 *
 * and the rest of a draft layer around block attention:
 *
 *   dflash_draft_embed anchor + mask embeddings: the first layer's block input
 *   dflash_draft_qkv   input RMSNorm + fused Q/K/V projection of the block
 *   dflash_draft_mlp   output projection + residual, RMSNorm, SwiGLU MLP +
 *                      residual, optional final RMSNorm
 *
 * and the append step of a sliding-window draft cache kept as a ring:
 *
 *   dflash_ring_append slots and positions of a cycle's verified rows
 *
 * and the shared LM head with the draft proposals it samples:
 *
 *   dflash_draft_head  block logits and the seven proposals
 *
 * and DFlash2's candidate path selector (its block convolution is an option
 * of dflash_draft_mlp):
 *
 *   dflash_draft_paths top-m candidates per position, entropies, top-P paths
 *
 * Sources (web pages; cited by title and section):
 *   [E4B] "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash"
 *   [DF2] "DFlash & DFlash2: Block-Diffusion LLM-Speedup"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer named "device" is device memory on the current HIP device,
 *   owned by the caller.  The library never allocates or frees device memory;
 *   scratch space comes in through `workspace`, sized by the matching
 *   *_workspace_size call (0 bytes is valid when that call returns 0).
 *   Device pointers must be 16-byte aligned.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Calls only enqueue work: there is no host synchronisation, outputs stay
 *   on the device, and every pointer must stay valid until the stream has
 *   reached the call.  Results are deterministic for fixed inputs.
 * - Element types: dtype DFLASH_BF16 (bfloat16 storage, fp32 arithmetic) or
 *   DFLASH_F32.  Integer tensors are int32 / int64 as stated.
 * - Return value: DFLASH_OK (0) or a negative code.  On error nothing is
 *   enqueued and dflash_last_error() (thread-local) describes the problem.
 *   Data-dependent conditions that only the device can see never fault: they
 *   are handled as documented on each field (skipped writes, clamped lengths,
 *   rejected proposals).
 * - Calls that share a workspace buffer must be ordered on one stream.
 *
 * Paged KV cache layout (owned by the caller; written by dflash_ctx_fuse,
 * read by dflash_block_attn)
 * ---------------------------------------------------------------------
 * A layer's K cache and V cache are each [num_pages][8 kv heads][2048]
 * elements.  A page holds 16 consecutive tokens; token slot s = page*16 + t.
 * Inside one (page, head) block of 16 tokens x 128 dims the element of token
 * t (0..15) and dim d (0..127) sits at
 *
 *   K:  256*((d & 63) >> 3) + 8*(t + 16*(d >> 6)) + (d & 7)
 *   V:  512*(d >> 5) + 256*((t >> 2) & 1) + 8*(d & 31) + (((t >> 3) << 2) | (t & 3))
 *
 * Both layouts make every 64-lane load of a 32-token tile one contiguous,
 * coalesced 512-byte or 1-KiB run whose lanes land directly in the operand
 * registers of the gfx950 32x32x16 bf16 matrix instruction (keys as the A
 * operand of S^T = K Q^T, values as the A operand of O^T = V^T P^T).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define DFLASH_OK            0
#define DFLASH_EINVAL       (-1)  /* null pointer, bad size/stride, bad constant */
#define DFLASH_EUNSUPPORTED (-2)  /* dtype or shape outside the supported set */
#define DFLASH_EHIP         (-3)  /* a HIP launch failed (message has the HIP error) */
#define DFLASH_EWORKSPACE   (-4)  /* workspace missing or smaller than required */

/* ---- element types ---- */
#define DFLASH_BF16 0
#define DFLASH_F32  1

/* ---- fixed model constants ([E4B] "Five target states become persistent
 *      draft context"; "The released serving cycle") ---- */
#define DFLASH_D          2560   /* draft width = target width */
#define DFLASH_NCAPTURE   5      /* captured target states (layers 5,11,17,23,35) */
#define DFLASH_HQ         32     /* query heads */
#define DFLASH_HKV        8      /* KV heads; 4 query heads share one */
#define DFLASH_HEAD_DIM   128
#define DFLASH_BLOCK      8      /* 1 anchor + 7 mask positions */
#define DFLASH_PAGE       16     /* tokens per cache page */
#define DFLASH_MAX_LAYERS 5      /* draft layers */
#define DFLASH_INTER      5120   /* SwiGLU width (derived from the parameter count) */

#define DFLASH_VERSION 10501     /* 1.5.1: verification workspace sized for 4096-entry draw chunks */

/* dflash_attn_args.split_tokens: cut the context tiles of all sequences,
 * laid end to end (each sequence's 32-token tiles, then its block's keys as
 * one more tile), into equal pieces per pair of KV heads, one workgroup each,
 * and merge the sequences a piece boundary cuts.  For batches whose context
 * lengths differ (the split by sequence waits for the longest).  Falls back to
 * the automatic split when B > 1024 or a piece could exceed 32768 tokens
 * (B * (max_pages * 16 or window) / 64, roughly). */
#define DFLASH_SPLIT_BALANCED (-1)

/*
 * dflash_ctx_fuse -- context fusion and K/V injection.
 * [DF2] 4.1 (H_t = RMSNorm(W_c [H1;...;H5]), K_i/V_i = W_i^K/V H_t injected
 * into every draft layer's cache) and [E4B] "Five target states become
 * persistent draft context" (five 2560-wide states concatenated and projected
 * back to 2560; per-head K RMSNorm before RoPE).
 *
 * For each of the M rows:
 *   y    = [hs0 | hs1 | hs2 | hs3 | hs4] . wc^T           (12800 -> 2560)
 *   H_t  = gc * y / sqrt(mean(y^2) + eps)                  (stored in dtype)
 *   for layer l < num_layers:
 *     k  = H_t . wkv[2048 l      : 2048 l + 1024]^T  -> 8 heads x 128
 *     v  = H_t . wkv[2048 l+1024 : 2048 l + 2048]^T
 *     k  = RoPE(gk[l] * k / sqrt(mean_head(k^2) + eps), pos[row])
 *     k_cache[l], v_cache[l] at slot[row] <- k, v          (rounded to dtype)
 * RoPE is rotate-half over pairs (i, i+64) with angle pos * theta^(-i/64).
 */
typedef struct dflash_fuse_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 (all float tensors) */
    int32_t num_layers;       /* 1..5 draft layers to write */
    int64_t M;                /* rows to fuse; 0 is a valid no-op */
    const void* hs[5];        /* device, each [M][hs_stride], first 2560 used; capture order */
    int64_t hs_stride;        /* elements between rows, >= 2560, multiple of 8, <= 2^22 */
    const void* wc;           /* device [2560][12800] row-major (out, in) */
    const void* gc;           /* device [2560] fusion-norm weight */
    const void* wkv;          /* device [num_layers*2048][2560]; per layer 1024 K rows then 1024 V rows */
    const void* gk;           /* device [num_layers][128] k_norm weights */
    float eps;                /* RMSNorm epsilon (> 0) */
    float rope_theta;         /* RoPE base (> 1) */
    const int32_t* pos;       /* device [M] RoPE positions */
    const int64_t* slot;      /* device [M] cache slot page*16+t; slots < 0 or >= num_pages*16 are skipped */
    void* k_cache[5];         /* device, layer l: [num_pages][8][2048] K layout (entries >= num_layers ignored) */
    void* v_cache[5];         /* device, layer l: [num_pages][8][2048] V layout */
    int64_t num_pages;        /* pages in every layer's cache */
    void* ht_out;             /* optional device [M][2560] copy of H_t (dtype); NULL = not written */
} dflash_fuse_args;

/*
 * dflash_block_attn -- one draft layer's block attention.
 * [E4B] "Five target states become persistent draft context": Q [B,32,8,128],
 * K/V [B,8,8,128], four query heads per KV head, per-head Q/K RMSNorm before
 * RoPE; attention over the cached context plus the block, non-causal inside
 * the block ([E4B] "The released serving cycle"; [DF2] 4.1, K = [K_ctx ; K_blk]).
 *
 * For sequence b with S = ctx_len[b] (clamped to [0, max_pages*16]) and query
 * head h (KV head g = h/4), block position j (0 = anchor) at position S + j:
 *   q^   = RoPE(gq * q / rms(q), S + j),  k^blk = RoPE(gk * k_blk / rms, S + j)
 *   keys = cached tokens [t0, S) of head g, then the 8 block keys
 *          (t0 = 0, or max(0, S - window) when window > 0)
 *   out  = softmax(q^ . keys^T / sqrt(128)) . values       (no mask)
 * Cached tokens are read through block_table[b][t / 16]; entries past the
 * sequence's last page are never read.
 */
typedef struct dflash_attn_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 */
    int32_t B;                /* sequences, >= 1 */
    const void* q;            /* device [B][32][8][128] */
    const void* k_blk;        /* device [B][8][8][128] block keys before norm/RoPE */
    const void* v_blk;        /* device [B][8][8][128] block values */
    const void* gq;           /* device [128] q_norm weight */
    const void* gk;           /* device [128] k_norm weight */
    float eps;
    float rope_theta;
    const void* k_cache;      /* device [num_pages][8][2048] K layout (this layer) */
    const void* v_cache;      /* device [num_pages][8][2048] V layout */
    int64_t num_pages;        /* block_table entries must lie in [0, num_pages) */
    const int32_t* block_table; /* device [B][max_pages] */
    int32_t max_pages;        /* >= 1 */
    const int32_t* ctx_len;   /* device [B] cached tokens per sequence */
    int32_t page_size;        /* must be 16 */
    int32_t block_len;        /* must be 8 */
    int32_t window;           /* 0 = full context; > 0 = latest `window` tokens */
    int32_t split_tokens;     /* 0 = automatic; DFLASH_SPLIT_BALANCED; else tokens per split-K chunk,
                                 multiple of 128, <= 32768 */
    void* out;                /* device [B][32][8][128] (dtype) */
    float* lse_out;           /* optional device [B][32][8] natural-log LSE; NULL = not written */
} dflash_attn_args;

/*
 * dflash_spec_verify -- exact speculative verification of one block.
 * [E4B] "Why exact verification preserves the target" and [DF2] 4.4:
 * sampled proposals are accepted with probability min(1, p/q); on rejection
 * the replacement is drawn from normalize(max(0, p - q)); greedy accepts while
 * the proposal equals the target argmax; at most 8 tokens per cycle including
 * the correction or bonus token ([E4B] "The released serving cycle").
 *
 * Per sequence b with T = temperature[b] (T <= 0: greedy):
 *   p_r = softmax(target[b][r] / T) (r = 0..7), q_k = softmax(draft[b][k-1] / T)
 *   for k = 1..7: greedy  -- accept iff d_k == argmax target[b][k-1] (lowest index on ties)
 *                 sampled -- accept iff u_k < p_{k-1}(d_k) / q_k(d_k),
 *                            u_k = U(0, b, k, 0)
 *   first rejection at k: greedy emits the argmax; sampled emits
 *       argmax_{i: r_i > 0} ln r_i + G_i,  r = max(0, p_{k-1} - q_k)   (r == 0 -> p_{k-1})
 *   all accepted: greedy emits argmax target[b][7]; sampled emits
 *       argmax_i target[b][7][i]/T + G_i  with G from k = 8
 *   G_i = -ln(-ln U(1, b, k, i)).
 * Uniforms: U(s, b, k, i) for stream s, sequence b, position k, entry i.
 * One Philox4x64-10 block (Salmon et al., SC'11: 10 rounds, multipliers
 * 0xD2E7470EE14C6C93 and 0xCA5A826395121157, key increments
 * 0x9E3779B97F4A7C15 and 0xBB67AE8584CAA73B) with key (seed, 0) and counter
 * (floor(i / 8), 8b + k, s, offset) gives four 64-bit words w0..w3 and
 * serves the eight entries 8 floor(i / 8) .. + 7:
 *   w    = word floor(i / 2) mod 4 of the block
 *   bits = (w >> 41) & 0x7FFFFF   when i is even (bits 41..63)
 *          (w >> 9)  & 0x7FFFFF   when i is odd  (bits 9..31)
 *   U    = (bits + 0.5) * 2^-23   (exact in fp32, strictly inside (0, 1))
 * Stream 0 holds the acceptance uniforms (i = 0), stream 1 the Gumbel noise
 * of the correction / bonus draw, stream 2 the draft proposals
 * (dflash_draft_head).
 * Proposal ids outside [0, V) are never accepted.  Decisions with
 * |u - p/q| < 1e-6 are counted into *near_ties (atomically added).
 */
typedef struct dflash_verify_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 logits */
    int32_t B;                /* sequences, >= 1 */
    int64_t V;                /* vocabulary, >= 1, multiple of 8 */
    const void* target_logits;  /* device; row r of sequence b at b*t_batch_stride + r*t_row_stride, 8 rows */
    int64_t t_batch_stride;   /* elements, multiple of 8 */
    int64_t t_row_stride;     /* elements, >= V, multiple of 8 */
    const void* draft_logits;   /* device; row k-1 (proposal k) at b*d_batch_stride + (k-1)*d_row_stride, 7 rows */
    int64_t d_batch_stride;
    int64_t d_row_stride;
    const int32_t* draft_tokens; /* device [B][7] proposals d_1..d_7 */
    const float* temperature;    /* device [B]; <= 0 means greedy */
    uint64_t seed;
    uint64_t offset;             /* per-cycle counter word */
    int32_t* out_tokens;         /* device [B][8]; emitted tokens, -1 padded */
    int32_t* out_len;            /* device [B]; 1..8 */
    unsigned long long* near_ties; /* device [1]; incremented, never cleared */
    const float* draft_stats;    /* optional device [B][7][2]: (m, s) of draft row k-1 (proposal k) at the
                                    sequence's temperature, m = max of the row, s = sum e^((z - m) / T), as
                                    dflash_draft_head writes them for the same rows and temperatures; the
                                    row statistics pass then reads no draft row.  NULL = computed here */
} dflash_verify_args;

/*
 * dflash_draft_embed -- block input of the first draft layer.
 * [E4B] "The released serving cycle" (a block of eight: the anchor, then
 * seven mask positions) and [DF2] 4.2 (input representations come from the
 * target's embedding table, shared with the drafter).
 *   x[b][0] = emb[anchor[b]],  x[b][j] = emb[mask_id] for j = 1..7
 * An anchor id outside [0, V) gives a zero row.
 */
typedef struct dflash_embed_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 */
    int32_t B;                /* sequences, 1..8192 */
    int64_t V;                /* rows of emb, >= 1 */
    const void* emb;          /* device [V][2560] embedding table */
    const int32_t* anchor;    /* device [B] last verified token per sequence */
    int32_t mask_id;          /* mask token id, in [0, V) */
    void* x;                  /* device [B][8][2560] (dtype), copied rows */
} dflash_embed_args;

/*
 * dflash_draft_qkv -- input RMSNorm and fused Q/K/V projection of one draft
 * layer's block.  [DF2] 4.1 (Q_i = W_i^Q H_d; the H_d halves of K_i, V_i) and
 * [E4B] "Five target states become persistent draft context" (Q [B,32,8,128],
 * block K/V [B,8,8,128]); the pre-norm layer is the reading of the drafter as
 * "Qwen3-style" ([E4B], opening section).
 *   a = g_in * x / sqrt(mean(x^2) + eps)                        (stored in dtype)
 *   y = a . w_qkv^T                                             (6144 columns)
 *   q[b][h][j][d] = y[8b+j][128h+d],  k_blk[b][g][j][d] = y[8b+j][4096+128g+d],
 *   v_blk[b][g][j][d] = y[8b+j][5120+128g+d]                     (rounded to dtype)
 * The outputs are the inputs of dflash_block_attn (before its Q/K norm and
 * RoPE).  Outputs must not overlap x.
 */
typedef struct dflash_qkv_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 */
    int32_t B;                /* sequences, 1..8192 */
    const void* x;            /* device [B][8][2560] layer input */
    const void* g_in;         /* device [2560] input-norm weight */
    const void* w_qkv;        /* device [6144][2560] row-major (out, in): W_Q | W_K | W_V */
    float eps;                /* RMSNorm epsilon (> 0) */
    void* q;                  /* device [B][32][8][128] */
    void* k_blk;              /* device [B][8][8][128] */
    void* v_blk;              /* device [B][8][8][128] */
} dflash_qkv_args;

/*
 * dflash_draft_mlp -- the layer after block attention: output projection and
 * residual, post-attention RMSNorm, SwiGLU MLP and residual, and (after the
 * last layer) the final RMSNorm.  Same reading and sources as
 * dflash_draft_qkv; [E4B] "The parameter count exposes the real cost" fixes
 * the shapes (intermediate width 5120, derived).
 *   o'[8b+j][128h+d] = o[b][h][j][d]
 *   h  = x + o' . w_o^T                                          (stored)
 *   c  = g_post * h / sqrt(mean(h^2) + eps)                      (stored)
 *   s  = silu(c . w_gu[0:5120]^T) * (c . w_gu[5120:10240]^T)     (stored)
 *   x_out = h + s . w_d^T                                        (rounded to dtype)
 *   y  = g_final * x_out / sqrt(mean(x_out^2) + eps)  when g_final != NULL
 * Every "stored" value is rounded to dtype once and the next step reads the
 * rounded value.  x_out may be x itself (in place); y_out and h_out must not
 * overlap x, o, x_out or each other.
 *
 * With conv_k > 0, DFlash2's depthwise block convolution ([DF2] "DFlash2",
 * item 1: kernel width 3 or 5 between the attention and feed-forward
 * sublayers) is applied to the stored h as a residual branch, causal over
 * the eight block positions t = 0..7 of each sequence (nothing before the
 * anchor):
 *   h'[t] = h[t] + b_conv + sum_{j < conv_k, t - j >= 0} w_conv[j] * h[t - j]   (stored)
 * and the rest of the layer reads h' in place of h (c, and the residual of
 * x_out); h_out then receives h'.
 */
typedef struct dflash_mlp_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 */
    int32_t B;                /* sequences, 1..8192 */
    const void* x;            /* device [B][8][2560] layer input (the residual) */
    const void* o;            /* device [B][32][8][128] block attention output */
    const void* w_o;          /* device [2560][4096] (out, in = 128*head + dim) */
    const void* g_post;       /* device [2560] post-attention norm weight */
    const void* w_gu;         /* device [10240][2560]: 5120 gate rows, then 5120 up rows */
    const void* w_d;          /* device [2560][5120] */
    const void* g_final;      /* optional device [2560] final-norm weight; NULL = no final norm */
    float eps;                /* RMSNorm epsilon (> 0) */
    void* x_out;              /* device [B][8][2560] layer output */
    void* y_out;              /* device [B][8][2560] final-norm output; required iff g_final != NULL */
    void* h_out;              /* optional device [B][8][2560] copy of h (h' with the convolution) (dtype); NULL = not written */
    int32_t conv_k;           /* 0 = no convolution; else the kernel width, 1..8 */
    const void* w_conv;       /* device [conv_k][2560] per-channel taps (tap j multiplies h[t - j]); required iff conv_k > 0 */
    const void* b_conv;       /* device [2560] bias; required iff conv_k > 0 */
} dflash_mlp_args;

/*
 * dflash_ring_append -- cache slots of the rows a cycle appends to a
 * sliding-window draft cache kept as a ring of pages.  [E4B] "Five target
 * states become persistent draft context" (the drafter attends to the latest
 * 1,024 tokens) and "Cache and latency have separate break-even points"
 * (20 MiB of K/V per sequence at that window).
 * Logical page p of sequence b is physical page ring[b][p mod ring_pages];
 * keeping the slot t % 16, the ring holds the latest 16 * ring_pages tokens,
 * so ceil(W / 16) pages cover a W-token window.  For row rows_per_seq*b + j,
 * with n = clamp(n_new[b], 0, rows_per_seq):
 *   j < n:  t = ctx_len[b] + j,  slot = ring[b][(t/16) mod R] * 16 + t % 16,  pos = t
 *   else:   slot = -1 (dflash_ctx_fuse skips the row),  pos = 0
 * and then ctx_len[b] += n.  slot / pos feed dflash_ctx_fuse with
 * M = B * rows_per_seq rows; dflash_block_attn then reads the ring through a
 * block table whose entry p is ring[b][p mod R], with window = W.  Only
 * verified tokens enter the draft cache (block K/V are per cycle), so there
 * is nothing to roll back.  No workspace.
 */
typedef struct dflash_ring_args {
    int32_t B;                /* sequences, 1..65535 */
    int32_t ring_pages;       /* R >= 1 pages per sequence */
    const int32_t* ring;      /* device [B][R] physical page ids */
    int32_t* ctx_len;         /* device [B] cached tokens; read, then advanced */
    const int32_t* n_new;     /* device [B] rows verified this cycle (e.g. out_len) */
    int32_t rows_per_seq;     /* 1..64 fuse rows reserved per sequence */
    int64_t* slot;            /* device [B * rows_per_seq] */
    int32_t* pos;             /* device [B * rows_per_seq] */
} dflash_ring_args;

/*
 * dflash_draft_head -- the shared LM head over the eight block rows and the
 * seven draft proposals.  [E4B] "The parameter count exposes the real cost"
 * (the drafter's output head is a copy of the target head, [262144, 2560],
 * since it scores the target's vocabulary) and "The released serving cycle"
 * (one forward over the block proposes all seven future tokens); [DF2] 4.2
 * (the target's unembedding head maps output states to vocabulary logits).
 *   logits[b][r] = y[b][r] . w_head^T            r = 0..7, stored in dtype
 *   draft_tokens[b][k-1], k = 1..7, from the STORED row logits[b][k]:
 *     T_b <= 0: argmax_i logits[b][k][i]             (lowest index on ties)
 *     T_b >  0: argmax_i logits[b][k][i] / T_b - ln(-ln u_i)
 * with u_i = U(2, b, k, i), stream 2 of the uniform layout documented at
 * dflash_spec_verify (counter (floor(i / 8), 8b + k, 2, offset), entry i in
 * half i mod 2 of word floor(i / 2) mod 4; streams 0 and 1 belong to
 * verification): a Gumbel-max
 * draw, which is an exact sample from softmax(logits[b][k] / T_b).  Row 0
 * (the anchor) is projected and not sampled.  Rows 1..7 of logits are the
 * draft_logits of dflash_spec_verify for the same cycle (base logits + V,
 * d_batch_stride = 8 V, d_row_stride = V).  Use the same seed and offset as
 * that verify call: draft and verification draws come from disjoint streams.
 */
typedef struct dflash_head_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 */
    int32_t B;                /* sequences, 1..8192 */
    int64_t V;                /* vocabulary, multiple of 128, 128..2^21 */
    const void* y;            /* device [B][8][2560] final-norm output of the last draft layer */
    const void* w_head;       /* device [V][2560] head weight (row i scores token i) */
    const float* temperature; /* device [B]; <= 0 means greedy */
    uint64_t seed;
    uint64_t offset;          /* per-cycle counter word */
    void* logits;             /* device [B][8][V] (dtype), written */
    int32_t* draft_tokens;    /* device [B][7] proposals d_1..d_7, written (-1 if a row has no finite key,
                                 which only non-finite inputs cause; dflash_spec_verify rejects it) */
    float* draft_stats;       /* optional device [B][7][2], written: for proposal row k = 1..7 of a sampled
                                 sequence, m = max_i logits[b][k][i] and s = sum_i e^((logits[b][k][i] - m) / T_b)
                                 of the STORED logits (the normaliser of q_k); (-inf, 0) for greedy
                                 sequences.  Pass it as dflash_spec_verify's draft_stats.  NULL = not computed */
} dflash_head_args;

/*
 * dflash_draft_paths -- DFlash2's top-m candidate path selector.  [DF2]
 * "DFlash2", item 2: the head yields the top-m candidates of every block
 * position, a path (one candidate per position) is scored by the sum of its
 * draft log-probabilities plus lambda times the positions' entropies, and
 * the best paths are handed to the target.  For proposal positions
 * k = 1..7 (rows 1..7 of each sequence's logits), with P_k = softmax of the
 * stored row and H_k its entropy:
 *   cand_ids[b][k-1][r]  = the r-th largest logit's id (r < m; ties to the lower id)
 *   cand_logp[b][k-1][r] = log P_k(cand_ids[b][k-1][r]),   entropy[b][k-1] = H_k
 *   paths[b][0..P)       = the P best rank tuples (r_1..r_7) by
 *                          score = sum_k cand_logp[b][k-1][r_k] + lambda * sum_k H_k,
 *                          best first, equal scores by the lexicographically
 *                          smaller tuple; written as token ids
 *   scores[b][p]         = that score of path p (fp32; -inf if it holds a -inf logit)
 * log P_k(x) = z_k(x) - lse_k, and lse_k and lambda * H_k are the same for
 * every path, so paths are ranked by the EXACT sum of their stored candidate
 * logits (a 128-bit fixed-point sum at the finest unit among the sequence's
 * candidates; exact while they span at most 2^123 in magnitude); equal sums
 * go to the smaller rank tuple.  A path through a -inf logit comes after
 * every finite one (fewer -inf candidates first, then the sum of its finite
 * ones).  +inf and NaN logits are outside the supported domain.  The drafter
 * proposes the block in one forward, so P_k does not depend on the
 * candidates chosen before k: the score separates per position, and a beam
 * of width P keeps exactly the top P.
 * Rows 1..7 of dflash_draft_head's logits are the natural input
 * (batch_stride = 8 V, row_stride = V).
 */
typedef struct dflash_paths_args {
    int32_t dtype;            /* DFLASH_BF16 or DFLASH_F32 logits */
    int32_t B;                /* sequences, 1..8192 */
    int64_t V;                /* vocabulary, multiple of 8, m..2^24 */
    const void* logits;       /* device; row r (0..7) of sequence b at b*batch_stride + r*row_stride; rows 1..7 read */
    int64_t batch_stride;     /* elements, multiple of 8, >= 8 * row_stride */
    int64_t row_stride;       /* elements, multiple of 8, >= V */
    int32_t m;                /* candidates per position, 1..8 */
    int32_t P;                /* paths, 1..64 and <= m^7 */
    float lambda;             /* entropy weight */
    int32_t* cand_ids;        /* device [B][7][m] */
    float* cand_logp;         /* device [B][7][m] */
    float* entropy;           /* device [B][7] */
    int32_t* paths;           /* device [B][P][7] token ids, best path first */
    float* scores;            /* device [B][P] */
} dflash_paths_args;

/* Library version (DFLASH_VERSION of the build). */
int dflash_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* dflash_last_error(void);

/* sizeof of the argument structs as compiled into the library:
 * kind 0 = dflash_fuse_args, 1 = dflash_attn_args, 2 = dflash_verify_args,
 * 3 = dflash_embed_args, 4 = dflash_qkv_args, 5 = dflash_mlp_args,
 * 6 = dflash_ring_args, 7 = dflash_head_args, 8 = dflash_paths_args;
 * returns 0 for any other kind.  Lets bindings check their struct mirrors. */
size_t dflash_args_size(int kind);

/* Workspace bytes the matching call needs for these arguments (only sizes,
 * dtype and flags are read; pointers may be NULL).  Returns a status code. */
int dflash_fuse_workspace_size(const dflash_fuse_args* args, size_t* bytes);
int dflash_attn_workspace_size(const dflash_attn_args* args, size_t* bytes);
int dflash_verify_workspace_size(const dflash_verify_args* args, size_t* bytes);
int dflash_draft_qkv_workspace_size(const dflash_qkv_args* args, size_t* bytes);
int dflash_draft_mlp_workspace_size(const dflash_mlp_args* args, size_t* bytes);
int dflash_draft_head_workspace_size(const dflash_head_args* args, size_t* bytes);
int dflash_draft_paths_workspace_size(const dflash_paths_args* args, size_t* bytes);

/* The three operations.  `workspace` must hold at least the size returned
 * above (it may be NULL when that size is 0); its contents are scratch. */
int dflash_ctx_fuse(const dflash_fuse_args* args, void* workspace,
                    size_t workspace_bytes, void* stream);
int dflash_block_attn(const dflash_attn_args* args, void* workspace,
                      size_t workspace_bytes, void* stream);
int dflash_spec_verify(const dflash_verify_args* args, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Allocation-free dflash_spec_verify, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as dflash_spec_verify; the scratch comes from a fixed device
 * array of dflash_verify_scratch_bytes() bytes (4 MiB) that the library holds
 * on every GPU it runs on until the process ends.  It calls no allocating
 * routine.  Calls whose dflash_verify_workspace_size exceeds that size are
 * rejected with DFLASH_EWORKSPACE (e.g. B = 1409 at V = 262144 still fits).
 * Every allocation-free call on a GPU uses that GPU's one array: calls that
 * overlap on one GPU (concurrent streams, or threads without ordering) race
 * and must not be issued; calls ordered on one stream are fine.  The first
 * call on a device looks up the array's device address (no allocation). */
int dflash_spec_verify_noalloc(const dflash_verify_args* args, void* stream);
int dflash_verify_scratch_bytes(size_t* bytes);

/* The draft layer around block attention (dflash_draft_embed needs no
 * workspace). */
int dflash_draft_embed(const dflash_embed_args* args, void* stream);
int dflash_draft_qkv(const dflash_qkv_args* args, void* workspace,
                     size_t workspace_bytes, void* stream);
int dflash_draft_mlp(const dflash_mlp_args* args, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Sliding-window cache append (no workspace). */
int dflash_ring_append(const dflash_ring_args* args, void* stream);

/* Shared LM head and draft proposals. */
int dflash_draft_head(const dflash_head_args* args, void* workspace,
                      size_t workspace_bytes, void* stream);

/* DFlash2 candidate path selector. */
int dflash_draft_paths(const dflash_paths_args* args, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Calibration: the practical ceilings of the part the hot path runs on, for
 * reading the roofline fractions against measured rather than datasheet
 * peaks.  Not part of the draft-verify cycle.
 *   dflash_calib_stream: reads `bytes` (a positive multiple of 16) of device
 *     memory at src once with 16-byte loads, eight in flight per thread, each
 *     workgroup of 256 threads reading 32 KiB contiguous runs, over `grid`
 *     workgroups (0 = 2048; at most 65536); with dst != NULL also stores
 *     every 16 bytes to dst (a copy).  sink receives one 16-byte xor per
 *     workgroup.
 *   dflash_calib_gather: reads chunks of the `bytes` (a positive multiple
 *     of 16) at src (16-byte aligned) in the order of the device list
 *     chunk_ids[nchunks] (int32): chunk c covers bytes [c chunk_bytes,
 *     (c + 1) chunk_bytes), chunk_bytes a multiple of 4096 in [4096, 2^20].
 *     Pieces of 4 KiB, eight in flight per thread, over `grid` workgroups
 *     (0 = 2048; at most 65536).  A negative id, or the part of a chunk
 *     past `bytes`, reads nothing.  A random permutation of the chunks gives
 *     the access pattern of shuffled cache pages.  sink receives one 16-byte
 *     xor per workgroup.  nchunks times chunk_bytes / 4096 must not exceed
 *     2^31.
 *   dflash_calib_mfma: bf16 32x32x16 matrix instructions on register
 *     operands only, `iters` rounds of eight per wave, two waves per SIMD on
 *     256 CUs; *flops (if not NULL) receives the FLOPs of the launch.  sink
 *     receives one float per thread.
 * sink must hold dflash_calib_sink_bytes() bytes.  Time the calls with
 * events on the stream. */
int dflash_calib_sink_bytes(size_t* bytes);
int dflash_calib_stream(const void* src, void* dst, size_t bytes, int grid, void* sink, void* stream);
int dflash_calib_gather(const void* src, size_t bytes, const int32_t* chunk_ids, int64_t nchunks, int chunk_bytes,
                        int grid, void* sink, void* stream);
int dflash_calib_mfma(int iters, void* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
