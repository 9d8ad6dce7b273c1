// Split-K bf16 GEMM and plain fp32 GEMM (gfx950); interface in gemm.h.
//
// The bf16 kernel runs the 32x32x16 bf16 matrix instruction on operands
// staged through LDS by loads that write LDS directly; tiles are laid out
// contiguously per XCD in 8-row groups so that tiles sharing a B panel run on
// the same L2.  Used where the row count is a few hundred to a few thousand
// (context fusion of newly verified rows, the draft layer's projections over
// B x 8 block rows): the weights stream once, split over K so that every CU
// gets a share.
#include "device_common.h"
#include "gemm.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128;

// ---- bf16 GEMM: 128x128 tile, BK = 32, four-stage LDS ring filled by the
// gfx950 direct global->LDS load (global_load_lds_dwordx4: lane l's 16 bytes
// land at the wave's LDS base + 16 l).  A stage holds A and B as [128 rows][4
// chunks of 8 bf16]; chunk c of row r sits at position 4r + (c ^ swz(r)), an
// XOR pattern that keeps the 16-byte operand reads of 8 or 16 consecutive
// rows on distinct banks.  The swizzle is applied to the global address each
// lane fetches, because the LDS position is fixed by the lane index.
constexpr int BKD = 32;                      // k per stage
constexpr int kStages = 4;
constexpr int kStageChunks = 2 * BM * 4;     // A then B, 16-byte chunks
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ void dma16(const void* g, uint4* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(GemmParams p) {
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
    const TileId t = tile_id(p, tiles_m, tiles_n);
    if (!t.valid) return;
    const int nk = p.K / BKD;
    const int kt0 = t.ks * p.kt_per_split;
    const int kt1 = min(nk, kt0 + p.kt_per_split);
    if (kt0 >= kt1) return;
    const int nloc = kt1 - kt0;

    __shared__ __attribute__((aligned(16))) uint4 lds[kStages * kStageChunks];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = t.tm * BM, n0 = t.tn * BN;
    const uint16_t* bmat = static_cast<const uint16_t*>(p.b);

    // Each thread issues 4 DMA chunks per stage at positions P = (j & 1) * 256 +
    // tid of the A half (j = 0, 1) or the B half (j = 2, 3).  Rows past M
    // read row M-1 (valid memory); their results are never stored.
    int src_r[4], src_c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int P = (j & 1) * 256 + tid;
        src_r[j] = P >> 2;
        src_c[j] = (P & 3) ^ swz(P >> 2);
    }
    // The five segment pointers stay in registers: indexing p.aseg with a
    // run-time segment is a scalar memory load whose wait would sit in front
    // of every stage's loads.
    const void *aseg0 = p.aseg[0], *aseg1 = p.aseg[1], *aseg2 = p.aseg[2], *aseg3 = p.aseg[3], *aseg4 = p.aseg[4];
    auto issue = [&](int kt, int slot) {
        const int kg = kt * BKD;
        const int seg = kg / p.seg_w;
        const int kc = kg - seg * p.seg_w;
        const uint16_t* a = static_cast<const uint16_t*>(
            seg == 0 ? aseg0 : seg == 1 ? aseg1 : seg == 2 ? aseg2 : seg == 3 ? aseg3 : aseg4);
        uint4* sbase = lds + slot * kStageChunks;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint16_t* g = j < 2 ? a + (int64_t)min(m0 + src_r[j], p.M - 1) * p.a_stride + kc + 8 * src_c[j]
                                      : bmat + (int64_t)(n0 + src_r[j]) * p.K + kg + 8 * src_c[j];
            // wave-uniform LDS base of this instruction
            dma16(g, sbase + (j >> 1) * (BM * 4) + (j & 1) * 256 + wave * 64);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    const int lr = lane & 31, lh = lane >> 5;

    // Prologue: stages 0..kStages-2 (clamped re-reads past the end are harmless).
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; ++s0) issue(kt0 + min(s0, nloc - 1), s0);

    for (int i = 0; i < nloc; ++i) {
        wait_vm<4 * (kStages - 2)>();  // stage i landed; the two newer ones may be in flight
        // Plain s_barrier: __syncthreads() would also drain every outstanding
        // load.  A wave's reads of stage i-1 completed before its MFMAs ran.
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(kt0 + min(i + kStages - 1, nloc - 1), (i + kStages - 1) % kStages);
        const uint4* sa = lds + (i % kStages) * kStageChunks;
        const uint4* sb = sa + BM * 4;
        bf16x8 af[2][2], bfr[2][2];  // [k-step][block]: all operand reads first
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = 2 * ks + lh;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ra = wr + 32 * q + lr, rb = wc + 32 * q + lr;
                af[ks][q] = __builtin_bit_cast(bf16x8, sa[4 * ra + (ch ^ swz(ra))]);
                bfr[ks][q] = __builtin_bit_cast(bf16x8, sb[4 * rb + (ch ^ swz(rb))]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[q][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][q], bfr[ks][j], acc[q][j], 0, 0, 0);
    }
    wait_vm<0>();  // the clamped trailing loads must land before the workgroup exits

    // Lane holds column lr of each 32x32 block, rows 8*jj + 4*lh + r.
    float* out = p.part + (int64_t)t.ks * p.M * p.N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                const int gn = n0 + wc + 32 * j + lr;
                if (gm < p.M) out[(int64_t)gm * p.N + gn] = acc[i][j][r];
            }
}

// Plain fp32 GEMM for the fp32 path: 64x64 tile, 4x4 outputs per thread.
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p) {
    const int tm = blockIdx.x, tn = blockIdx.y;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    __shared__ float as[16][65], bs[16][65];
    float acc[4][4] = {};
    const float* bmat = static_cast<const float*>(p.b);
    for (int k0 = 0; k0 < p.K; k0 += 16) {
        const int seg = k0 / p.seg_w;
        const int kc = k0 - seg * p.seg_w;
        const float* a = static_cast<const float*>(p.aseg[seg]);
        for (int i = tid; i < 64 * 16; i += kThreads) {
            const int r = i >> 4, kk = i & 15;
            const int gm = tm * 64 + r;
            as[kk][r] = gm < p.M ? a[(int64_t)gm * p.a_stride + kc + kk] : 0.f;
            bs[kk][r] = bmat[(int64_t)(tn * 64 + r) * p.K + k0 + kk];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += as[kk][ty * 4 + i] * bs[kk][tx * 4 + j];
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int gm = tm * 64 + ty * 4 + i;
        if (gm >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) p.part[(int64_t)gm * p.N + tn * 64 + tx * 4 + j] = acc[i][j];
    }
}

}  // namespace

int gemm_split(int M, int N, int K) {
    const int tiles = ((M + BM - 1) / BM) * (N / BN);
    const int nk = K / BKD;
    int ks = 512 / tiles;                 // 2 workgroups per CU on 256 CUs, one round
    if (ks > nk / 8) ks = nk / 8;         // keep >= 8 k-tiles per split
    if (ks > kGemmMaxKs) ks = kGemmMaxKs;
    if (ks < 1) ks = 1;
    // Every split must own at least one k-tile: recount after rounding.
    const int per = (nk + ks - 1) / ks;
    return (nk + per - 1) / per;
}

void gemm_set_split(GemmParams& g, int dtype, int ks) {
    if (dtype != DFLASH_BF16) ks = 1;
    g.ks = ks;
    g.kt_per_split = (g.K / BKD + ks - 1) / ks;
}

hipError_t launch_gemm(const GemmParams& g, int dtype, hipStream_t s) {
    if (dtype == DFLASH_BF16) {
        const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN) * g.ks;
        const int grid = (tiles + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
        gemm_bf16_kernel<<<grid, kThreads, 0, s>>>(g);
    } else {
        gemm_f32_kernel<<<dim3((g.M + 63) / 64, g.N / 64), kThreads, 0, s>>>(g);
    }
    return hipGetLastError();
}

}  // namespace dflash
