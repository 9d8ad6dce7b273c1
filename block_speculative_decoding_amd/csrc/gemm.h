// Split-K bf16 GEMM and plain fp32 GEMM (gfx950), shared by the context
// fusion and the draft-layer paths.  Both compute fp32 partial products
//   part[s][m][n] = sum over k in split s of A[m][k] * B[n][k]
// with A given as up to five column segments (columns [s*seg_w, (s+1)*seg_w)
// of A come from aseg[s], rows a_stride elements apart) and B [N][K]
// row-major; the caller sums the ks partials in its epilogue.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace dflash {

constexpr int kGemmXcds = 8;      // XCDs of the part; tiles are laid out contiguously per XCD
constexpr int kGemmGroupM = 8;    // M tiles per group sharing one B panel
constexpr int kGemmMaxKs = 16;    // largest split-K factor (epilogues unroll to it)

struct GemmParams {
    const void* aseg[5];  // A segments: columns [s*seg_w, (s+1)*seg_w) come from aseg[s]
    int64_t a_stride;     // elements between A rows
    int seg_w;
    const void* b;        // [N][K] row-major
    int M, N, K;
    int ks, kt_per_split;
    float* part;          // [ks][M][N]
    uint16_t* out_bf16;   // bf16 path with ks == 1: if set, the product rounded to bf16
                          // goes here ([M][N]) instead of part
    int sk_q;             // 256x256 fp32-partial GEMM only: k-tiles per workgroup run under
                          // stream-K (0: one whole tile per workgroup); see gemm_bf16_big_kernel
    uint16_t* swiglu_out; // bf16 path with ks == 1: if set, B is [gate ; up] (rows [0, N/2) and
                          // [N/2, N)) and silu(gate) * up, from the fp32 products and rounded
                          // to bf16, goes here ([M][N/2]); tile tn multiplies gate rows
                          // 64 tn .. +63 and the same up rows
};

// K/V injection epilogue of the context fusion's second GEMM (N = L * 2048
// columns [K_0 | V_0 | K_1 | ...], 128 per head): k_norm over each K head,
// RoPE with the (cos, sin) table, bf16 store into the paged caches at each
// row's slot (rows whose slot lies outside the cache are skipped).
struct KvEpilogue {
    const float2* cs;      // [M][64] (cos, sin) of pos[row] * inv_freq[i]
    const void* gk;        // [L][128] bf16 k_norm weights
    float eps;
    const int64_t* slot;
    int64_t num_pages;
    void* kc[5];
    void* vc[5];
};

// Head-layout epilogue of the draft layer's Q/K/V projection (N = 6144
// columns [q heads 0..31 | k heads 0..7 | v heads 0..7], 128 per head): row
// m = 8b + j, column 128h + d goes to q[b][h][j][d] (k_blk, v_blk: [b][h][j][d]
// with 8 heads), rounded to bf16.
struct QkvEpilogue {
    uint16_t* q;
    uint16_t* k;
    uint16_t* v;
};

// Tile id for this workgroup: XCD-contiguous ranges, then 8-row M groups.
struct TileId { int tm, tn, ks; bool valid; };
__device__ __forceinline__ TileId tile_id(const GemmParams& p, int tiles_m, int tiles_n) {
    const int total = tiles_m * tiles_n * p.ks;
    const int nblk = gridDim.x;  // padded to a multiple of kGemmXcds
    const int bid = blockIdx.x;
    const int per_xcd = nblk / kGemmXcds;
    const int L = (bid % kGemmXcds) * per_xcd + bid / kGemmXcds;
    TileId t;
    t.valid = L < total;
    const int per_split = tiles_m * tiles_n;
    t.ks = L / per_split;
    const int r = L % per_split;
    const int in_group = kGemmGroupM * tiles_n;
    const int grp = r / in_group;
    const int first_m = grp * kGemmGroupM;
    const int gm = min(tiles_m - first_m, kGemmGroupM);
    const int q = r % in_group;
    t.tm = first_m + q % gm;
    t.tn = q / gm;
    return t;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte LDS read into an MFMA operand register; issued as inline asm so
// that the caller places the lgkmcnt waits (the compiler's own placement
// drains every outstanding read before each matrix instruction).
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
    bf16x8 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Buffer load of 16 bytes per lane written straight to LDS (lane l at the
// M0 base + 16 l), through a raw buffer descriptor: bytes past the
// descriptor's range read as zero.
typedef int i32x4 __attribute__((ext_vector_type(4)));
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) uint32_t* lds,
                                                           int size, int voffset, int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// Raw buffer descriptor: 48-bit base, stride 0, range in bytes.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// Split-K factor for the bf16 kernel: one residency round (two workgroups per
// CU on 256 CUs), at least 4 k-tiles of 64 per split, at most kGemmMaxKs, and
// every split owns at least one k-tile.
int gemm_split(int M, int N, int K);
// The same for the fp32 kernel's 64x64 tiles (at least 2 k-tiles per split).
int gemm_split_f32(int M, int N, int K);
// Sets g.ks and g.kt_per_split (splits own kt_per_split k-tiles of 64).
void gemm_set_split(GemmParams& g, int dtype, int ks);
// bf16: 128x128 tiles, N % 128 == 0, K and seg_w multiples of 64, 16-byte
// aligned rows, a_stride < 2^23; fp32: 64x64 tiles, N % 64 == 0, K and
// seg_w multiples of 16, a_stride a multiple of 4.
hipError_t launch_gemm(const GemmParams& g, int dtype, hipStream_t s);
// bf16 K/V projection with its epilogue (no partials): the same 128x128
// tiles with two 4-wave groups per 512-thread workgroup (one workgroup per
// CU), each group taking half of the tile's k-tiles; the halves are added
// through LDS and the tile goes through the K/V epilogue.  g.ks == 1, N a
// multiple of 2048: each 128-column tile is one head of one layer.
hipError_t launch_gemm_pair(const GemmParams& g, const KvEpilogue& ep, hipStream_t s);
// The same two-group kernel for the Q/K/V projection (g.ks == 1, N == 6144)
// with the head-layout epilogue.
hipError_t launch_gemm_pair_qkv(const GemmParams& g, const QkvEpilogue& qe, hipStream_t s);

}  // namespace dflash
