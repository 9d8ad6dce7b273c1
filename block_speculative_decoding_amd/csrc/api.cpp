// C ABI of libdflash: argument validation, workspace sizing and launch.
// The operations themselves are documented in include/dflash.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/dflash.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DFLASH_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                                  \
    do {                                                                                \
        if (!(p)) return fail(DFLASH_EINVAL, "%s: null pointer " #p, fn);               \
        if (!aligned16(p)) return fail(DFLASH_EINVAL, "%s: " #p " is not 16-byte aligned", fn); \
    } while (0)

int check_dtype(const char* fn, int dtype) {
    if (dtype != DFLASH_BF16 && dtype != DFLASH_F32)
        return fail(DFLASH_EUNSUPPORTED, "%s: unsupported dtype %d", fn, dtype);
    return DFLASH_OK;
}

int check_ws(const char* fn, size_t need, const void* ws, size_t have) {
    if (need == 0) return DFLASH_OK;
    if (!ws) return fail(DFLASH_EWORKSPACE, "%s: workspace of %zu bytes required, got NULL", fn, need);
    if (have < need) return fail(DFLASH_EWORKSPACE, "%s: workspace of %zu bytes required, got %zu", fn, need, have);
    if (!aligned16(ws)) return fail(DFLASH_EWORKSPACE, "%s: workspace is not 16-byte aligned", fn);
    return DFLASH_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(DFLASH_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------- sizes
int validate_fuse_sizes(const char* fn, const dflash_fuse_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = check_dtype(fn, a->dtype);
    if (rc) return rc;
    if (a->num_layers < 1 || a->num_layers > DFLASH_MAX_LAYERS)
        return fail(DFLASH_EINVAL, "%s: num_layers %d outside [1, %d]", fn, a->num_layers, DFLASH_MAX_LAYERS);
    if (a->M < 0 || a->M > (1 << 24)) return fail(DFLASH_EINVAL, "%s: M %lld outside [0, 2^24]", fn, (long long)a->M);
    return DFLASH_OK;
}

int validate_attn_sizes(const char* fn, const dflash_attn_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = check_dtype(fn, a->dtype);
    if (rc) return rc;
    if (a->B < 1 || a->B > 65535) return fail(DFLASH_EINVAL, "%s: B %d outside [1, 65535]", fn, a->B);
    if (a->max_pages < 1 || (int64_t)a->max_pages * DFLASH_PAGE > INT_MAX / 2)
        return fail(DFLASH_EINVAL, "%s: max_pages %d out of range", fn, a->max_pages);
    if (a->page_size != DFLASH_PAGE) return fail(DFLASH_EINVAL, "%s: page_size must be 16 (got %d)", fn, a->page_size);
    if (a->block_len != DFLASH_BLOCK) return fail(DFLASH_EINVAL, "%s: block_len must be 8 (got %d)", fn, a->block_len);
    if (a->window < 0) return fail(DFLASH_EINVAL, "%s: negative window", fn);
    if (a->split_tokens != DFLASH_SPLIT_BALANCED &&
        (a->split_tokens < 0 || a->split_tokens % 128 != 0 || a->split_tokens > 32768))
        return fail(DFLASH_EINVAL,
                    "%s: split_tokens must be 0, DFLASH_SPLIT_BALANCED or a multiple of 128 up to 32768 (got %d)", fn,
                    a->split_tokens);
    return DFLASH_OK;
}

int validate_verify_sizes(const char* fn, const dflash_verify_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = check_dtype(fn, a->dtype);
    if (rc) return rc;
    if (a->B < 1 || a->B > (1 << 20)) return fail(DFLASH_EINVAL, "%s: B %d outside [1, 2^20]", fn, a->B);
    if (a->V < 8 || a->V > INT_MAX / 2 || a->V % 8 != 0)
        return fail(DFLASH_EINVAL, "%s: V %lld must be a positive multiple of 8 below 2^30", fn, (long long)a->V);
    return DFLASH_OK;
}

// Sizes, pointers and strides of a verification call (defined below).
int validate_verify(const char* fn, const dflash_verify_args* a);

int validate_draft_b(const char* fn, int dtype, int B) {
    int rc = check_dtype(fn, dtype);
    if (rc) return rc;
    if (B < 1 || B > 8192) return fail(DFLASH_EINVAL, "%s: B %d outside [1, 8192]", fn, B);
    return DFLASH_OK;
}

int validate_qkv_sizes(const char* fn, const dflash_qkv_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    return validate_draft_b(fn, a->dtype, a->B);
}

int validate_mlp_sizes(const char* fn, const dflash_mlp_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    return validate_draft_b(fn, a->dtype, a->B);
}

int validate_head_sizes(const char* fn, const dflash_head_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = validate_draft_b(fn, a->dtype, a->B);
    if (rc) return rc;
    if (a->V < 128 || a->V > (1 << 21) || a->V % 128)
        return fail(DFLASH_EINVAL, "%s: V %lld must be a multiple of 128 in [128, 2^21]", fn, (long long)a->V);
    return DFLASH_OK;
}

int validate_paths_sizes(const char* fn, const dflash_paths_args* a) {
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = validate_draft_b(fn, a->dtype, a->B);
    if (rc) return rc;
    if (a->m < 1 || a->m > 8) return fail(DFLASH_EINVAL, "%s: m %d outside [1, 8]", fn, a->m);
    int64_t paths = 1;
    for (int k = 0; k < 7 && paths <= 64; ++k) paths *= a->m;
    if (a->P < 1 || a->P > 64 || a->P > paths)
        return fail(DFLASH_EINVAL, "%s: P %d outside [1, min(64, m^7)]", fn, a->P);
    if (a->V < a->m || a->V > (1 << 24) || a->V % 8)
        return fail(DFLASH_EINVAL, "%s: V %lld must be a multiple of 8 in [m, 2^24]", fn, (long long)a->V);
    if (a->row_stride < a->V || a->row_stride % 8)
        return fail(DFLASH_EINVAL, "%s: row_stride %lld must be a multiple of 8, >= V", fn, (long long)a->row_stride);
    if (a->batch_stride < 8 * a->row_stride || a->batch_stride % 8)
        return fail(DFLASH_EINVAL, "%s: batch_stride %lld must be a multiple of 8, >= 8 * row_stride", fn,
                    (long long)a->batch_stride);
    return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_version(void) { return DFLASH_VERSION; }

const char* dflash_last_error(void) { return g_err.c_str(); }

size_t dflash_args_size(int kind) {
    switch (kind) {
        case 0: return sizeof(dflash_fuse_args);
        case 1: return sizeof(dflash_attn_args);
        case 2: return sizeof(dflash_verify_args);
        case 3: return sizeof(dflash_embed_args);
        case 4: return sizeof(dflash_qkv_args);
        case 5: return sizeof(dflash_mlp_args);
        case 6: return sizeof(dflash_ring_args);
        case 7: return sizeof(dflash_head_args);
        case 8: return sizeof(dflash_paths_args);
        default: return 0;
    }
}

int dflash_fuse_workspace_size(const dflash_fuse_args* a, size_t* bytes) {
    const char* fn = "dflash_fuse_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_fuse_sizes(fn, a);
    if (rc) return rc;
    *bytes = a->M == 0 ? 0 : dflash::fuse_plan(*a).ws_bytes;
    return ok();
}

int dflash_attn_workspace_size(const dflash_attn_args* a, size_t* bytes) {
    const char* fn = "dflash_attn_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_attn_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::attn_plan(*a).ws_bytes;
    return ok();
}

int dflash_verify_workspace_size(const dflash_verify_args* a, size_t* bytes) {
    const char* fn = "dflash_verify_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_verify_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::verify_workspace_bytes(a->B, a->V);
    return ok();
}

int dflash_draft_qkv_workspace_size(const dflash_qkv_args* a, size_t* bytes) {
    const char* fn = "dflash_draft_qkv_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_qkv_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::draft_qkv_plan(*a).ws_bytes;
    return ok();
}

int dflash_draft_mlp_workspace_size(const dflash_mlp_args* a, size_t* bytes) {
    const char* fn = "dflash_draft_mlp_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_mlp_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::draft_mlp_plan(*a).ws_bytes;
    return ok();
}

int dflash_draft_head_workspace_size(const dflash_head_args* a, size_t* bytes) {
    const char* fn = "dflash_draft_head_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_head_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::head_workspace_bytes(a->B, a->V);
    return ok();
}

int dflash_draft_paths_workspace_size(const dflash_paths_args* a, size_t* bytes) {
    const char* fn = "dflash_draft_paths_workspace_size";
    if (!bytes) return fail(DFLASH_EINVAL, "%s: null output", fn);
    int rc = validate_paths_sizes(fn, a);
    if (rc) return rc;
    *bytes = dflash::paths_workspace_bytes(a->B, a->V);
    return ok();
}

int dflash_ctx_fuse(const dflash_fuse_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_ctx_fuse";
    int rc = validate_fuse_sizes(fn, a);
    if (rc) return rc;
    if (a->M == 0) return ok();
    for (int i = 0; i < DFLASH_NCAPTURE; ++i)
        if (!a->hs[i] || !aligned16(a->hs[i])) return fail(DFLASH_EINVAL, "%s: hs[%d] null or not 16-byte aligned", fn, i);
    // Row offsets inside a 256-row tile are 32-bit byte offsets: stride <= 2^22.
    if (a->hs_stride < DFLASH_D || a->hs_stride % 8 != 0 || a->hs_stride > (1 << 22))
        return fail(DFLASH_EINVAL, "%s: hs_stride %lld must be in [2560, 2^22] and a multiple of 8", fn,
                    (long long)a->hs_stride);
    REQUIRE_PTR(a->wc);
    REQUIRE_PTR(a->gc);
    REQUIRE_PTR(a->wkv);
    REQUIRE_PTR(a->gk);
    REQUIRE_PTR(a->pos);
    REQUIRE_PTR(a->slot);
    for (int l = 0; l < a->num_layers; ++l)
        if (!a->k_cache[l] || !a->v_cache[l] || !aligned16(a->k_cache[l]) || !aligned16(a->v_cache[l]))
            return fail(DFLASH_EINVAL, "%s: cache pointers of layer %d null or not 16-byte aligned", fn, l);
    if (a->ht_out && !aligned16(a->ht_out)) return fail(DFLASH_EINVAL, "%s: ht_out is not 16-byte aligned", fn);
    if (a->num_pages < 1) return fail(DFLASH_EINVAL, "%s: num_pages must be >= 1", fn);
    if (!(a->eps > 0.f)) return fail(DFLASH_EINVAL, "%s: eps must be > 0", fn);
    if (!(a->rope_theta > 1.f)) return fail(DFLASH_EINVAL, "%s: rope_theta must be > 1", fn);
    const dflash::FusePlan pl = dflash::fuse_plan(*a);
    rc = check_ws(fn, pl.ws_bytes, ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_fuse(*a, pl, ws, static_cast<hipStream_t>(stream)));
}

int dflash_block_attn(const dflash_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_block_attn";
    int rc = validate_attn_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->q);
    REQUIRE_PTR(a->k_blk);
    REQUIRE_PTR(a->v_blk);
    REQUIRE_PTR(a->gq);
    REQUIRE_PTR(a->gk);
    REQUIRE_PTR(a->k_cache);
    REQUIRE_PTR(a->v_cache);
    REQUIRE_PTR(a->block_table);
    REQUIRE_PTR(a->ctx_len);
    REQUIRE_PTR(a->out);
    if (a->lse_out && !aligned16(a->lse_out)) return fail(DFLASH_EINVAL, "%s: lse_out is not 16-byte aligned", fn);
    if (a->num_pages < 1) return fail(DFLASH_EINVAL, "%s: num_pages must be >= 1", fn);
    if (!(a->eps > 0.f)) return fail(DFLASH_EINVAL, "%s: eps must be > 0", fn);
    if (!(a->rope_theta > 1.f)) return fail(DFLASH_EINVAL, "%s: rope_theta must be > 1", fn);
    const dflash::AttnPlan pl = dflash::attn_plan(*a);
    rc = check_ws(fn, pl.ws_bytes, ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_attn(*a, pl, ws, static_cast<hipStream_t>(stream)));
}

int dflash_spec_verify(const dflash_verify_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_spec_verify";
    int rc = validate_verify(fn, a);
    if (rc) return rc;
    const size_t need = dflash::verify_workspace_bytes(a->B, a->V);
    rc = check_ws(fn, need, ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_verify(*a, ws, static_cast<hipStream_t>(stream)));
}

int dflash_spec_verify_noalloc(const dflash_verify_args* a, void* stream) {
    const char* fn = "dflash_spec_verify_noalloc";
    int rc = validate_verify(fn, a);
    if (rc) return rc;
    const size_t need = dflash::verify_workspace_bytes(a->B, a->V);
    if (need > dflash::kVerifyScratchBytes)
        return fail(DFLASH_EWORKSPACE,
                    "%s: B = %d, V = %lld needs %zu bytes of scratch, above the %zu-byte device array of the "
                    "allocation-free entry point (use dflash_spec_verify with a workspace)",
                    fn, a->B, (long long)a->V, need, dflash::kVerifyScratchBytes);
    void* ws = nullptr;
    const hipError_t e = dflash::verify_scratch(&ws);
    if (e != hipSuccess) return fail(DFLASH_EHIP, "%s: scratch address lookup failed: %s", fn, hipGetErrorString(e));
    return launched(fn, dflash::launch_verify(*a, ws, static_cast<hipStream_t>(stream)));
}

int dflash_verify_scratch_bytes(size_t* bytes) {
    if (!bytes) return fail(DFLASH_EINVAL, "dflash_verify_scratch_bytes: null bytes");
    *bytes = dflash::kVerifyScratchBytes;
    return ok();
}

}  // extern "C"

namespace {

int validate_verify(const char* fn, const dflash_verify_args* a) {
    int rc = validate_verify_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->target_logits);
    REQUIRE_PTR(a->draft_logits);
    REQUIRE_PTR(a->draft_tokens);
    REQUIRE_PTR(a->temperature);
    REQUIRE_PTR(a->out_tokens);
    REQUIRE_PTR(a->out_len);
    if (!a->near_ties) return fail(DFLASH_EINVAL, "%s: null pointer near_ties", fn);
    if (a->t_row_stride < a->V || a->d_row_stride < a->V)
        return fail(DFLASH_EINVAL, "%s: row strides must be >= V", fn);
    if (a->t_batch_stride < 0 || a->d_batch_stride < 0)
        return fail(DFLASH_EINVAL, "%s: negative batch stride", fn);
    if ((a->t_row_stride | a->d_row_stride | a->t_batch_stride | a->d_batch_stride) % 8 != 0)
        return fail(DFLASH_EINVAL, "%s: strides must be multiples of 8 elements", fn);
    if (a->draft_stats && !aligned16(a->draft_stats))
        return fail(DFLASH_EINVAL, "%s: draft_stats is not 16-byte aligned", fn);
    return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_draft_embed(const dflash_embed_args* a, void* stream) {
    const char* fn = "dflash_draft_embed";
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    int rc = validate_draft_b(fn, a->dtype, a->B);
    if (rc) return rc;
    if (a->V < 1 || a->V > INT_MAX) return fail(DFLASH_EINVAL, "%s: V %lld outside [1, 2^31)", fn, (long long)a->V);
    if (a->mask_id < 0 || a->mask_id >= a->V)
        return fail(DFLASH_EINVAL, "%s: mask_id %d outside [0, V)", fn, a->mask_id);
    REQUIRE_PTR(a->emb);
    REQUIRE_PTR(a->anchor);
    REQUIRE_PTR(a->x);
    return launched(fn, dflash::launch_embed(*a, static_cast<hipStream_t>(stream)));
}

int dflash_draft_qkv(const dflash_qkv_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_draft_qkv";
    int rc = validate_qkv_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->x);
    REQUIRE_PTR(a->g_in);
    REQUIRE_PTR(a->w_qkv);
    REQUIRE_PTR(a->q);
    REQUIRE_PTR(a->k_blk);
    REQUIRE_PTR(a->v_blk);
    if (!(a->eps > 0.f)) return fail(DFLASH_EINVAL, "%s: eps must be > 0", fn);
    const dflash::DraftQkvPlan pl = dflash::draft_qkv_plan(*a);
    rc = check_ws(fn, pl.ws_bytes, ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_draft_qkv(*a, pl, ws, static_cast<hipStream_t>(stream)));
}

int dflash_draft_mlp(const dflash_mlp_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_draft_mlp";
    int rc = validate_mlp_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->x);
    REQUIRE_PTR(a->o);
    REQUIRE_PTR(a->w_o);
    REQUIRE_PTR(a->g_post);
    REQUIRE_PTR(a->w_gu);
    REQUIRE_PTR(a->w_d);
    REQUIRE_PTR(a->x_out);
    if (a->g_final) {
        if (!aligned16(a->g_final)) return fail(DFLASH_EINVAL, "%s: g_final is not 16-byte aligned", fn);
        REQUIRE_PTR(a->y_out);
    }
    if (a->h_out && !aligned16(a->h_out)) return fail(DFLASH_EINVAL, "%s: h_out is not 16-byte aligned", fn);
    if (a->conv_k < 0 || a->conv_k > 8) return fail(DFLASH_EINVAL, "%s: conv_k %d outside [0, 8]", fn, a->conv_k);
    if (a->conv_k > 0) {
        REQUIRE_PTR(a->w_conv);
        REQUIRE_PTR(a->b_conv);
    }
    if (!(a->eps > 0.f)) return fail(DFLASH_EINVAL, "%s: eps must be > 0", fn);
    const dflash::DraftMlpPlan pl = dflash::draft_mlp_plan(*a);
    rc = check_ws(fn, pl.ws_bytes, ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_draft_mlp(*a, pl, ws, static_cast<hipStream_t>(stream)));
}

int dflash_ring_append(const dflash_ring_args* a, void* stream) {
    const char* fn = "dflash_ring_append";
    if (!a) return fail(DFLASH_EINVAL, "%s: null args", fn);
    if (a->B < 1 || a->B > 65535) return fail(DFLASH_EINVAL, "%s: B %d outside [1, 65535]", fn, a->B);
    if (a->ring_pages < 1) return fail(DFLASH_EINVAL, "%s: ring_pages must be >= 1", fn);
    if (a->rows_per_seq < 1 || a->rows_per_seq > 64)
        return fail(DFLASH_EINVAL, "%s: rows_per_seq %d outside [1, 64]", fn, a->rows_per_seq);
    if (!a->ring || !a->ctx_len || !a->n_new || !a->slot || !a->pos)
        return fail(DFLASH_EINVAL, "%s: null pointer", fn);
    return launched(fn, dflash::launch_ring_append(*a, static_cast<hipStream_t>(stream)));
}

int dflash_draft_head(const dflash_head_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_draft_head";
    int rc = validate_head_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->y);
    REQUIRE_PTR(a->w_head);
    REQUIRE_PTR(a->temperature);
    REQUIRE_PTR(a->logits);
    REQUIRE_PTR(a->draft_tokens);
    if (a->draft_stats && !aligned16(a->draft_stats))
        return fail(DFLASH_EINVAL, "%s: draft_stats is not 16-byte aligned", fn);
    rc = check_ws(fn, dflash::head_workspace_bytes(a->B, a->V), ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_head(*a, ws, static_cast<hipStream_t>(stream)));
}

int dflash_draft_paths(const dflash_paths_args* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "dflash_draft_paths";
    int rc = validate_paths_sizes(fn, a);
    if (rc) return rc;
    REQUIRE_PTR(a->logits);
    if (!a->cand_ids || !a->cand_logp || !a->entropy || !a->paths || !a->scores)
        return fail(DFLASH_EINVAL, "%s: null output pointer", fn);
    rc = check_ws(fn, dflash::paths_workspace_bytes(a->B, a->V), ws, ws_bytes);
    if (rc) return rc;
    return launched(fn, dflash::launch_paths(*a, ws, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- calibration
int dflash_calib_sink_bytes(size_t* bytes) {
    if (!bytes) return fail(DFLASH_EINVAL, "dflash_calib_sink_bytes: null bytes");
    const size_t a = (size_t)dflash::calib_stream_max_grid() * 16, b = (size_t)dflash::calib_mfma_grid() * 256 * 4;
    *bytes = a > b ? a : b;
    return ok();
}

int dflash_calib_stream(const void* src, void* dst, size_t bytes, int grid, void* sink, void* stream) {
    const char* fn = "dflash_calib_stream";
    REQUIRE_PTR(src);
    REQUIRE_PTR(sink);
    if (dst && !aligned16(dst)) return fail(DFLASH_EINVAL, "%s: dst is not 16-byte aligned", fn);
    if (bytes == 0 || bytes % 16 != 0) return fail(DFLASH_EINVAL, "%s: bytes must be a positive multiple of 16", fn);
    if (grid < 0 || grid > dflash::calib_stream_max_grid())
        return fail(DFLASH_EINVAL, "%s: grid %d outside [0, %d]", fn, grid, dflash::calib_stream_max_grid());
    return launched(fn, dflash::launch_calib_stream(src, dst, bytes, grid, sink, static_cast<hipStream_t>(stream)));
}

int dflash_calib_gather(const void* src, size_t bytes, const int32_t* chunk_ids, int64_t nchunks, int chunk_bytes,
                        int grid, void* sink, void* stream) {
    const char* fn = "dflash_calib_gather";
    REQUIRE_PTR(src);
    REQUIRE_PTR(chunk_ids);
    REQUIRE_PTR(sink);
    if (!aligned16(src)) return fail(DFLASH_EINVAL, "%s: src is not 16-byte aligned", fn);
    if (bytes == 0 || bytes % 16 != 0) return fail(DFLASH_EINVAL, "%s: bytes must be a positive multiple of 16", fn);
    if (chunk_bytes < 4096 || chunk_bytes > (1 << 20) || chunk_bytes % 4096 != 0)
        return fail(DFLASH_EINVAL, "%s: chunk_bytes %d must be a multiple of 4096 in [4096, 2^20]", fn, chunk_bytes);
    if (nchunks < 1 || nchunks > ((int64_t)1 << 31) / (chunk_bytes / 4096))
        return fail(DFLASH_EINVAL, "%s: nchunks %lld outside [1, 2^31 / (chunk_bytes / 4096)]", fn, (long long)nchunks);
    if (grid < 0 || grid > dflash::calib_stream_max_grid())
        return fail(DFLASH_EINVAL, "%s: grid %d outside [0, %d]", fn, grid, dflash::calib_stream_max_grid());
    return launched(fn, dflash::launch_calib_gather(src, bytes, chunk_ids, nchunks, chunk_bytes, grid, sink,
                                                    static_cast<hipStream_t>(stream)));
}

int dflash_calib_mfma(int iters, void* sink, double* flops, void* stream) {
    const char* fn = "dflash_calib_mfma";
    REQUIRE_PTR(sink);
    if (iters < 1 || iters > (1 << 24)) return fail(DFLASH_EINVAL, "%s: iters %d outside [1, 2^24]", fn, iters);
    if (flops) *flops = (double)dflash::calib_mfma_grid() * 4 * iters * 8 * (2.0 * 32 * 32 * 16);
    return launched(fn, dflash::launch_calib_mfma(iters, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
