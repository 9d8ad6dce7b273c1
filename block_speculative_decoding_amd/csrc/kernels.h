// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// ---- spec_verify ----
size_t verify_workspace_bytes(int B, int64_t V);
hipError_t launch_verify(const dflash_verify_args& a, void* ws, hipStream_t s);
// Size of the allocation-free entry point's device scratch, and its address
// on the current device (looked up once per device).
constexpr size_t kVerifyScratchBytes = size_t(4) << 20;
hipError_t verify_scratch(void** ptr);

// ---- block_attn ----
struct AttnPlan {
    int split_tokens;  // tokens per split-K chunk (multiple of 128)
    int nsplit;        // chunks per (sequence, kv head) in the grid
    bool balanced;     // equal pieces of all sequences' tiles (DFLASH_SPLIT_BALANCED)
    size_t ws_bytes;
};
AttnPlan attn_plan(const dflash_attn_args& a);
hipError_t launch_attn(const dflash_attn_args& a, const AttnPlan& plan, void* ws, hipStream_t s);

// ---- ctx_fuse ----
struct FusePlan {
    int ks1, ks2;          // split-K factors of the two GEMMs
    bool big;              // 256x256 kernels with the fused K/V epilogue
    bool pair2;            // K/V GEMM on the 128x128 kernel with two k-groups and the K/V epilogue
    int sk_q;              // big first GEMM under stream-K: k-tiles per workgroup (0: off)
    int sk_slots;          // product slots a tile's workgroups write under stream-K (1 otherwise)
    size_t off_part1, off_ht, off_part2, ws_bytes;
};
FusePlan fuse_plan(const dflash_fuse_args& a);
hipError_t launch_fuse(const dflash_fuse_args& a, const FusePlan& plan, void* ws, hipStream_t s);

// ---- draft layer around block attention ----
hipError_t launch_embed(const dflash_embed_args& a, hipStream_t s);
struct DraftQkvPlan {
    int ks;                      // split-K factor of the Q/K/V GEMM
    bool pair;                   // unsplit on two k-groups with the head-layout epilogue (no partials)
    size_t off_a, off_part, ws_bytes;
};
DraftQkvPlan draft_qkv_plan(const dflash_qkv_args& a);
hipError_t launch_draft_qkv(const dflash_qkv_args& a, const DraftQkvPlan& plan, void* ws, hipStream_t s);
struct DraftMlpPlan {
    int ks_o, ks_gu, ks_d;       // split-K factors of the three GEMMs
    size_t off_ao, off_part, off_h, off_c, off_s, ws_bytes;
};
DraftMlpPlan draft_mlp_plan(const dflash_mlp_args& a);
hipError_t launch_draft_mlp(const dflash_mlp_args& a, const DraftMlpPlan& plan, void* ws, hipStream_t s);

// ---- sliding-window cache ----
hipError_t launch_ring_append(const dflash_ring_args& a, hipStream_t s);

// ---- shared LM head and draft proposals ----
size_t head_workspace_bytes(int B, int64_t V);
hipError_t launch_head(const dflash_head_args& a, void* ws, hipStream_t s);

// ---- DFlash2 path selector ----
size_t paths_workspace_bytes(int B, int64_t V);
hipError_t launch_paths(const dflash_paths_args& a, void* ws, hipStream_t s);

// ---- calibration ----
int calib_stream_max_grid();
int calib_mfma_grid();
hipError_t launch_calib_stream(const void* src, void* dst, size_t bytes, int grid, void* sink, hipStream_t s);
hipError_t launch_calib_gather(const void* src, size_t bytes, const int32_t* ids, int64_t nchunks, int chunk_bytes,
                               int grid, void* sink, hipStream_t s);
hipError_t launch_calib_mfma(int iters, void* sink, hipStream_t s);

}  // namespace dflash
