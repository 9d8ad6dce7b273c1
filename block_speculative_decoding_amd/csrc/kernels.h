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

// ---- block_attn ----
struct AttnPlan {
    int split_tokens;  // tokens per split-K chunk (multiple of 128)
    int nsplit;        // chunks per (sequence, kv head) in the grid
    size_t ws_bytes;
};
AttnPlan attn_plan(const dflash_attn_args& a);
hipError_t launch_attn(const dflash_attn_args& a, const AttnPlan& plan, void* ws, hipStream_t s);

// ---- ctx_fuse ----
struct FusePlan {
    int ks1, ks2;          // split-K factors of the two GEMMs
    bool big;              // 256x256 kernels with the fused K/V epilogue
    size_t off_part1, off_ht, off_part2, ws_bytes;
};
FusePlan fuse_plan(const dflash_fuse_args& a);
hipError_t launch_fuse(const dflash_fuse_args& a, const FusePlan& plan, void* ws, hipStream_t s);

}  // namespace dflash
