// Context fusion + K/V injection (gfx950).
//
// Follows "DFlash & DFlash2: Block-Diffusion LLM-Speedup", section 4.1
// (H_t = RMSNorm(W_c [H1; ...; H5]); every draft layer's K/V cache receives
// W_K H_t / W_V H_t) and "Nemotron 3.5 Bolt E4B", section "Five target states
// become persistent draft context" (five 2560-wide states, 8 KV heads of 128,
// per-head K RMSNorm before RoPE; unquantized K/V projections fused into one
// matrix multiplication).
//
// Launch sequence on one stream (bf16, M below 4096 rows):
//   gemm  (A = the five capture pointers, one K segment each; B = W_c)
//         -> fp32 split-K partials [ks1][M][2560]
//   norm  -> sums the partials, RMSNorm with g_c, stores H_t (dtype); with
//            the K/V epilogue below, also each row's RoPE table
//   gemm  (A = H_t, B = W_KV of all layers at once, N = layers * 2048)
//         while its 128x128 tiles fit one 512-thread workgroup per CU (up to
//         256 tiles, e.g. M <= 384 rows at 5 layers): two 4-wave k-groups per
//         tile added through LDS, then the K/V epilogue (per 128-wide head: K
//         gets k_norm and RoPE, V is copied; both are stored into the paged
//         cache layout); no partials and no kv launch.  Otherwise:
//         -> fp32 split-K partials [ks2][M][N]
//   kv    -> sums the partials and does the same per head.
// From 4096 rows on, both GEMMs use 256x256 tiles without split-K and the
// second one carries the K/V injection in its epilogue (no kv launch); where
// the first GEMM's tiles do not fill whole rounds of one workgroup per CU it
// runs stream-K (equal runs of k-tiles, a few fp32 slots per tile that the
// norm adds).
// fp32 runs the fp32 GEMM with split-K, the norm and the kv launch.
// The bf16 GEMMs run on the 32x32x16 bf16 matrix instruction with operands
// staged through LDS by buffer loads that write LDS directly; tiles are laid
// out contiguously per XCD in 8-row groups so that tiles sharing an operand
// panel run on the same L2.
#include <cmath>

#include "device_common.h"
#include "gemm.h"
#include "head_sample.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = kGemmXcds;

// ---- bf16 GEMM for large M: 256x256 tile, eight waves (two per SIMD) of
// 128x64 (4x2 blocks of the 32x32x16 instruction, 128 fp32 accumulators per
// lane), 64 k per stage in a two-stage LDS ring (2 x 64 KiB), no split-K
// (the fp32-output mode has a stream-K form, below).
//  * Operands reach LDS through buffer loads that write LDS directly (16 B per
//    lane, lane l at the wave's LDS base + 16 l).  The descriptor's range stops
//    at row M, so rows of the last A tile past M read as zero.
//  * A stage row is 128 B = 8 chunks of 16 B; chunk c of row r sits at
//    c ^ ((r >> 1) & 7), which keeps the 16-byte operand reads of 16
//    consecutive rows on distinct banks.
//  * The operand reads of k-substep s+1 are in flight while substep s
//    multiplies (inline-asm ds_read_b128 with explicit lgkmcnt waits: the
//    compiler's own wait placement would drain them), and the next stage's 8
//    loads per thread are issued one by one between the 8 MFMAs of the last
//    substep.
// Column blocks: wave w owns rows 128 (w / 4) .. +128 and, within the 256
// columns, blocks 64 (w % 4) + {0, 32} for the plain GEMM; for the K/V
// projection (KV = true) blocks 128 (w % 4 / 2) + 32 (w % 2) + {0, 64}, so the
// RoPE pair (d, d+64) of a head sits in one lane and a head's 128 columns are
// two waves.  The K/V epilogue does k_norm (row sums over the head, the two
// waves' halves added through LDS), RoPE and the paged-cache store from the
// accumulators; the fp32 product never reaches memory.
constexpr int BMB = 256, BNB = 256;
constexpr int kBigThreads = 512;
constexpr int BKB = 64;                        // k per stage
constexpr int kBigPitch = BKB * 2;             // bytes per LDS row
constexpr int kBigStageBytes = 2 * BMB * kBigPitch;
constexpr int kBigPartsA = BMB * 8 / kBigThreads;  // buffer loads per thread per stage and operand (4)
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Tile t of the stream-K order: groups of kGemmGroupM row tiles, and within
// a group the row tile fastest, so consecutive tiles share a weight panel and
// a group's rows are reused across every column tile.  sk_tile_index is the
// inverse.
__host__ __device__ __forceinline__ void sk_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int in_group = kGemmGroupM * tiles_n;
    const int first_m = t / in_group * kGemmGroupM;
    const int gm = tiles_m - first_m < kGemmGroupM ? tiles_m - first_m : kGemmGroupM;
    const int q = t % in_group;
    tm = first_m + q % gm;
    tn = q / gm;
}
__host__ __device__ __forceinline__ int sk_tile_index(int tm, int tn, int tiles_m, int tiles_n) {
    const int first_m = tm / kGemmGroupM * kGemmGroupM;
    const int gm = tiles_m - first_m < kGemmGroupM ? tiles_m - first_m : kGemmGroupM;
    return first_m * tiles_n + tn * gm + (tm - first_m);
}


// MODE 0: fp32 partials to p.part (the fusion GEMM); 1: the K/V epilogue
// (ep); 2: the shared head's epilogue (hp): bf16 logits stored from
// registers and the draft keys of its rows (persistent over the tiles).
template <int MODE, bool SK = false>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_bf16_big_kernel(GemmParams p, KvEpilogue ep, HeadEpilogue hp) {
    static_assert(!SK || MODE == 0, "stream-K only for the fp32-partial GEMM");
    constexpr bool KV = MODE == 1;
    const int tiles_m = (p.M + BMB - 1) / BMB, tiles_n = p.N / BNB;
    const int nk = p.K / BKB;
    // Stream-K (SK): the tiles' k-tiles are laid end to end in the order of
    // sk_tile and cut into runs of p.sk_q, one per workgroup; the runs are
    // dealt to the XCDs in contiguous ranges.  A run covers the end of one
    // tile and the start of the next, so a tile's k-range is shared by the
    // workgroups whose runs meet it, each writing its products to its own
    // slot (its position minus that of the tile's first workgroup).
    int sk_pos = 0;
    int64_t sk_u = 0, sk_end = 0;
    TileId t = {};
    if (SK) {
        const int per = gridDim.x / kXcds;
        sk_pos = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
        sk_u = (int64_t)sk_pos * p.sk_q;
        sk_end = min((int64_t)tiles_m * tiles_n * nk, sk_u + p.sk_q);
        if (sk_u >= sk_end) return;
    } else if (MODE != 2) {
        t = tile_id(p, tiles_m, tiles_n);
        if (!t.valid) return;
    }

    // Two operand stages; the K epilogue reuses them as a [256][256] bf16
    // staging tile plus 4 KiB of row sums after them.
    __shared__ __attribute__((aligned(16))) uint4 lds[2 * kBigStageBytes / 16 + 256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const void *aseg0 = p.aseg[0], *aseg1 = p.aseg[1], *aseg2 = p.aseg[2], *aseg3 = p.aseg[3], *aseg4 = p.aseg[4];
    // Load j of a thread covers unit P = j * 512 + tid of the A (or B) half:
    // row P >> 3, chunk (P & 7) ^ swz8(row).
    uint32_t voa[kBigPartsA], vob[kBigPartsA];
#pragma unroll
    for (int j = 0; j < kBigPartsA; ++j) {
        const int P = j * kBigThreads + tid, r = P >> 3, c = (P & 7) ^ swz8(r);
        voa[j] = (uint32_t)(r * (int)p.a_stride + 8 * c) * 2u;
        vob[j] = (uint32_t)(r * p.K + 8 * c) * 2u;
    }
    struct StageSrc { i32x4 a, b; };
    // The wave index read as wave-uniform, so that each load's LDS base (M0)
    // is scalar arithmetic.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto load_part = [&](const StageSrc& src, int slot, int part) {
        uint4* sb = lds + slot * (kBigStageBytes / 16) + wave_s * 64;
        if (part < kBigPartsA) {
            llvm_amdgcn_raw_buffer_load_lds(src.a, (__attribute__((address_space(3))) uint32_t*)(sb + part * kBigThreads),
                                            16, (int)voa[part], 0, 0, 0);
        } else {
            const int j = part - kBigPartsA;
            llvm_amdgcn_raw_buffer_load_lds(
                src.b, (__attribute__((address_space(3))) uint32_t*)(sb + BMB * 8 + j * kBigThreads), 16, (int)vob[j], 0, 0, 0);
        }
    };

    f32x16 acc[4][2];
    const int wq = wave & 3;
    const int wr = (wave >> 2) * 128;
    const int wc = KV ? 128 * (wq >> 1) + 32 * (wq & 1) : 64 * wq;  // column of block 0
    constexpr int kBstep = KV ? 64 : 32;                           // columns from block 0 to block 1
    const int lr = lane & 31, lh = lane >> 5;
    // Byte address of this lane's 16-byte operand chunk for k-substep 0 of slot
    // 0; substep s flips chunk bits 1-2 (address ^ 32 s), block q adds 32 rows.
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint4*)lds);
    const uint32_t a_lane = lds0 + kBigPitch * (wr + lr) + 16 * (lh ^ swz8(lr));
    const uint32_t b_lane = lds0 + BMB * kBigPitch + kBigPitch * (wc + lr) + 16 * (lh ^ swz8(lr));
    auto rd = [&](int slot, int ks, bf16x8* a, bf16x8* b) {
        const uint32_t so = (uint32_t)slot * kBigStageBytes, x = 32u * ks;
        const uint32_t aa = (a_lane + so) ^ x, bb = (b_lane + so) ^ x;
        a[0] = lds_read16<0>(aa);
        a[1] = lds_read16<32 * kBigPitch>(aa);
        a[2] = lds_read16<64 * kBigPitch>(aa);
        a[3] = lds_read16<96 * kBigPitch>(aa);
        b[0] = lds_read16<0>(bb);
        b[1] = lds_read16<kBstep * kBigPitch>(bb);
    };
    // The head (mode 2) multiplies with the operands swapped: each 32 x 32
    // block comes out transposed, a lane holding one row of the tile and
    // registers running along its columns, which its epilogue stores directly.
    auto mf = [&](const bf16x8& a, const bf16x8& b, const f32x16& c) {
        return MODE == 2 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    };
    auto mm = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mf(a[i], b[j], acc[i][j]);
    };

    // Prologue and main loop over k-tiles [kb, ke) of the tile at (m0, n0);
    // leaves the tile's products in acc.
    auto run = [&](const int m0, const int n0, const int kb, const int ke) {
        const uint16_t* bmat = static_cast<const uint16_t*>(p.b) + (int64_t)n0 * p.K;
        const uint32_t arows = (uint32_t)min(p.M - m0, BMB);
        // Both operands' buffer descriptors for k-tile kt, computed once per
        // k-tile at the top of the loop: the loads themselves sit between matrix
        // instructions, where a segment select (a division and a five-way pointer
        // choice per load) would hold up the next one.
        auto stage_src = [&](int kt) {
            const int kg = kt * BKB;
            // The K/V projection's A operand (H_t) and the head's (y) are one segment.
            const int seg = MODE != 0 ? 0 : kg / p.seg_w;
            const int kc = kg - seg * p.seg_w;
            const void* av = seg == 0 ? aseg0 : seg == 1 ? aseg1 : seg == 2 ? aseg2 : seg == 3 ? aseg3 : aseg4;
            const uint16_t* a = static_cast<const uint16_t*>(av) + (int64_t)m0 * p.a_stride + kc;
            StageSrc s;
            s.a = buffer_rsrc(a, arows * (uint32_t)p.a_stride * 2u - (uint32_t)kc * 2u);
            s.b = buffer_rsrc(bmat + kg, (uint32_t)BNB * (uint32_t)p.K * 2u - (uint32_t)kg * 2u);
            return s;
        };
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

        bf16x8 fa[2][4], fb[2][2];
#pragma unroll
        for (int s0 = 0; s0 < 2; ++s0) {
            const StageSrc src = stage_src(kb + min(s0, ke - kb - 1));
#pragma unroll
            for (int t2 = 0; t2 < 2 * kBigPartsA; ++t2) load_part(src, s0, t2);
        }
        wait_vm<2 * kBigPartsA>();  // stage 0 landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        rd(0, 0, fa[0], fb[0]);
        for (int i = 0; i < ke - kb; ++i) {
            const int slot = i & 1;
            const StageSrc nsrc = stage_src(kb + min(i + 2, ke - kb - 1));
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                rd(slot, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                wait_lgkm<6>();  // substep s's reads (issued before these 6) are back
                __builtin_amdgcn_sched_barrier(0);
                mm(fa[s & 1], fb[s & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_lgkm<0>();
            wait_vm<0>();                  // stage i+1 landed
            __builtin_amdgcn_s_barrier();  // and every wave is done reading stage i
            asm volatile("" ::: "memory");
            rd(slot ^ 1, 0, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t2 = 0; t2 < 8; ++t2) {
                acc[t2 >> 1][t2 & 1] = mf(fa[1][t2 >> 1], fb[1][t2 & 1], acc[t2 >> 1][t2 & 1]);
                __builtin_amdgcn_sched_barrier(0);
                load_part(nsrc, slot, t2);  // stage i+2 into the slot stage i used
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm<0>();  // the clamped trailing loads must land before the workgroup exits
        wait_lgkm<0>();
    };

    if (SK) {
        // The run's pieces of one or more tiles, each written to this
        // workgroup's slot of its tile.
        while (sk_u < sk_end) {
            const int64_t tile = sk_u / nk;
            const int kb = (int)(sk_u - tile * nk);
            const int ke = (int)min((int64_t)nk, kb + (sk_end - sk_u));
            int tm, tn;
            sk_tile((int)tile, tiles_m, tiles_n, tm, tn);
            const int slot = sk_pos - (int)(tile * nk / p.sk_q);
            run(tm * BMB, tn * BNB, kb, ke);
            float* out = p.part + (int64_t)slot * p.M * p.N;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int gm = tm * BMB + wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int gn = tn * BNB + wc + kBstep * j + lr;
                        if (gm < p.M) out[(int64_t)gm * p.N + gn] = acc[i][j][r];
                    }
            sk_u += ke - kb;
            __syncthreads();  // every wave is done with the stages before the next run's loads
        }
        return;
    }
    auto head_epilogue = [&](const int m0, const int n0, const int tn) {
        // Block (i, j) of a lane holds row wr + 32 i + lr of the tile at columns
        // wc + 32 j + 8 g + 4 lh + s in register 4 g + s.  Rounded to bf16 and
        // traded with the lane 32 away (groups 1, 3 for 0, 2), each lane holds
        // whole 8-column chunks g = lh, lh + 2 of its row: each goes to the
        // logits as a 16-byte store straight from registers, and to LDS
        // ([256 rows][256 columns]; 16-byte chunk c of row r at c ^ (r % 32))
        // for the keys.
        float* s_temp = reinterpret_cast<float*>(lds + 2 * kBigStageBytes / 16);
        if (tid < BMB / 8) {
            const int bq = (m0 >> 3) + tid;
            s_temp[tid] = bq < (p.M >> 3) ? hp.temp[bq] : 0.f;
        }
        __syncthreads();  // every wave is done with the operand stages
        uint16_t* st = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wr + 32 * i + lr;
            const int gm = m0 + row;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t w[4][2];   // group g: bf16 pairs of its 4 columns
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    w[g][0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
                    w[g][1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                }
                // Send the groups the partner completes (lh 0: 1, 3; lh 1: 0, 2).
                uint32_t r[2][2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        r[h][e] = (uint32_t)__shfl_xor((int)(lh ? w[2 * h][e] : w[2 * h + 1][e]), 32);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t o0 = lh ? w[2 * h + 1][0] : w[2 * h][0];   // own half of group 2 h + lh
                    const uint32_t o1 = lh ? w[2 * h + 1][1] : w[2 * h][1];
                    const uint4 c = lh ? make_uint4(r[h][0], r[h][1], o0, o1) : make_uint4(o0, o1, r[h][0], r[h][1]);
                    const int cg = (wc + 32 * j) / 8 + 2 * h + lh;   // chunk of the tile's 32
                    if (gm < p.M) *reinterpret_cast<uint4*>(p.out_bf16 + (int64_t)gm * p.N + n0 + 8 * cg) = c;
                    *reinterpret_cast<uint4*>(st + row * 256 + 8 * (cg ^ (row & 31))) = c;
                }
            }
        }
        __syncthreads();
        // Four threads per row, 64 columns (eight chunks) each; two passes of
        // 128 rows.  The row's four threads are a quad: two DPP swaps reduce it.
        const int q = tid & 3;
        for (int pass = 0; pass < 2; ++pass) {
            const int row = pass * (BMB / 2) + (tid >> 2);
            const int gm = m0 + row;
            const int b = gm >> 3, k = gm & 7;
            const bool active = gm < p.M && k != 0;   // the same for the row's four threads
            const float Tb = s_temp[row >> 3];
            const bool greedy = !(Tb > 0.f);
            const float invT = greedy ? 1.f : 1.0f / Tb;
            const bool stats = active && !greedy && hp.spart != nullptr;   // uniform over the quad
            const StatScale sc = stat_scale(greedy ? 1.f : Tb);
            float best = -INFINITY, sm = -INFINITY, ss = 0.f;
            int bi = 0x7FFFFFFF;
            if (active) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int cg = 8 * q + c;
                    const int64_t i0 = (int64_t)n0 + 8 * cg;
                    const uint4 w = *reinterpret_cast<const uint4*>(st + row * 256 + 8 * (cg ^ (row & 31)));
                    float f[8];
                    f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
                    f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
                    draft_best8(f, i0, greedy, invT, 8ull * (uint64_t)b + (uint64_t)k, hp.seed, hp.offset, best, bi);
                    if (stats) stat_add8(f, sc, sm, ss);
                }
            }
            better_step<kDppXor1>(best, bi);
            better_step<kDppXor2>(best, bi);
            if (stats) {
                stat_merge(sm, ss, dpp_f<kDppXor1>(sm, -INFINITY), dpp_f<kDppXor1>(ss, 0.f), sc);
                stat_merge(sm, ss, dpp_f<kDppXor2>(sm, -INFINITY), dpp_f<kDppXor2>(ss, 0.f), sc);
            }
            if (active && q == 0) {
                const int64_t pi = ((int64_t)b * 7 + k - 1) * hp.nparts + tn;
                hp.part[pi] = {best, bi};
                if (stats) hp.spart[pi] = {sm, ss};
            }
        }
    };
    if (MODE == 2) {
        // Persistent over the tiles: XCD x owns the tile range
        // [x * per, (x + 1) * per) and its K workgroups take every K-th tile of
        // it, so a tile's logit stores drain while the next tile multiplies.
        const int T = tiles_m * tiles_n, per = (T + kXcds - 1) / kXcds, K = gridDim.x / kXcds;
        const int x = blockIdx.x % kXcds;
        for (int loc = blockIdx.x / kXcds; loc < per; loc += K) {
            const int L = x * per + loc;
            if (L >= T) break;
            const int in_group = kGemmGroupM * tiles_n;
            const int first_m = L / in_group * kGemmGroupM;
            const int gm = min(tiles_m - first_m, kGemmGroupM);
            const int q = L % in_group;
            const int tm = first_m + q % gm, tn = q / gm;
            run(tm * BMB, tn * BNB, 0, nk);
            head_epilogue(tm * BMB, tn * BNB, tn);
            __syncthreads();  // every wave is done with the LDS before the next tile's loads
        }
        return;
    }
    const int m0 = t.tm * BMB, n0 = t.tn * BNB;
    run(m0, n0, 0, nk);

    // Lane holds column lr of each 32x32 block, rows 8*(r/4) + 4*lh + (r%4).
    if (!KV) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = m0 + wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int gn = n0 + wc + kBstep * j + lr;
                    if (gm < p.M) p.part[(int64_t)gm * p.N + gn] = acc[i][j][r];
                }
        return;
    }

    // Head of this wave's columns: [layer][K/V][head]; both halves of a head
    // (waves w and w ^ 1) share it.  Dims d0 = 32 (w % 2) + lr and d0 + 64.
    const int hidx = (n0 >> 7) + (wq >> 1);
    const int l = hidx >> 4, isv = (hidx >> 3) & 1, head = hidx & 7;
    const int d0 = 32 * (wq & 1) + lr;
    uint16_t* cache = static_cast<uint16_t*>(isv ? ep.vc[l] : ep.kc[l]);
    const int64_t nslots = ep.num_pages * 16;
    const int rbase = m0 + wr;  // first row of this wave's 128

    if (isv) {
        // V granules hold one dim of 8 tokens (te = 4*(t/8) + t%4, half th =
        // (t/4)%2).  When a 32-row block fills two pages in slot order, the 8
        // values a lane keeps for rows 8*(r/4) + 4*lh + r%4, r = 0..7 (8..15),
        // are exactly the granule of page 0 (page 1) for half lh: one 16-byte
        // store each.  Otherwise every element is stored on its own.
        // The slots every block tests, loaded before the first test.
        int64_t s0v[4], smv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row0 = rbase + 32 * i;
            s0v[i] = row0 < p.M ? ep.slot[row0] : -1;
            smv[i] = row0 + lr < p.M ? ep.slot[row0 + lr] : -1;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row0 = rbase + 32 * i;
            const int64_t s0 = s0v[i], sm = smv[i];
            const bool ok = (s0 & 15) == 0 && s0 >= 0 && s0 + 32 <= nslots && sm == s0 + lr;
            if (__ballot(ok) == ~0ull) {
#pragma unroll
                for (int pg = 0; pg < 2; ++pg) {
                    uint16_t* blk = cache + (((s0 >> 4) + pg) * 8 + head) * 2048;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const f32x16& v = acc[i][j];
                        const int d = d0 + 64 * j;
                        uint4 w;
                        w.x = pack_bf16x2(v[8 * pg + 0], v[8 * pg + 1]);
                        w.y = pack_bf16x2(v[8 * pg + 2], v[8 * pg + 3]);
                        w.z = pack_bf16x2(v[8 * pg + 4], v[8 * pg + 5]);
                        w.w = pack_bf16x2(v[8 * pg + 6], v[8 * pg + 7]);
                        *reinterpret_cast<uint4*>(blk + 512 * (d >> 5) + 256 * lh + 8 * (d & 31)) = w;
                    }
                }
                continue;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = row0 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (gm >= p.M) continue;
                const int64_t slot = ep.slot[gm];
                if (slot < 0 || slot >= nslots) continue;
                uint16_t* blk = cache + ((slot >> 4) * 8 + head) * 2048;
                const int tt = (int)(slot & 15);
                const int te = ((tt >> 3) << 2) | (tt & 3), th = (tt >> 2) & 1;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int d = d0 + 64 * j;
                    blk[512 * (d >> 5) + 256 * th + 8 * (d & 31) + te] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
                }
            }
        }
        return;
    }

    // K: k_norm over the head, RoPE on the pair (d0, d0+64) held by one lane,
    // rounded to bf16 and staged through LDS as [256 rows][256 columns] of
    // this workgroup (16-byte chunk c of row r at c ^ (r % 16) within each
    // 128-column head); then each thread stores 16-byte chunks (8 dims of one
    // token), the K granule of the cache.  16 consecutive threads cover one
    // chunk index of 16 rows: 256 contiguous bytes when those rows fill a page
    // in slot order.
    float g[2];
    {
        const uint16_t* gk = static_cast<const uint16_t*>(ep.gk) + l * 128;
        g[0] = bf16_bits_to_f32(gk[d0]);
        g[1] = bf16_bits_to_f32(gk[d0 + 64]);
    }
    // Per-row partial sums of squares of this wave's 64 columns: each half
    // wave (the 32 columns lr of one row set) is reduced with DPP (pairs,
    // quads, half-row and row mirrors give every lane its 16-lane row sum,
    // then row_bcast:15 adds row 0's into row 1 and row 2's into row 3) and
    // read back from lane 31 (lanes 0-31) or 63 (lanes 32-63).
    float ssp[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float ss = acc[i][0][r] * acc[i][0][r] + acc[i][1][r] * acc[i][1][r];
            ss += dpp_f<kDppXor1>(ss, 0.f);
            ss += dpp_f<kDppXor2>(ss, 0.f);
            ss += dpp_f<kDppHalfMirror>(ss, 0.f);
            ss += dpp_f<kDppMirror>(ss, 0.f);
            ss += dpp_f<kDppBcast15, 0xA>(ss, 0.f);
            const int bits = __builtin_bit_cast(int, ss);
            const int lo = __builtin_amdgcn_readlane(bits, 31), hi = __builtin_amdgcn_readlane(bits, 63);
            ssp[i][r] = __builtin_bit_cast(float, lh ? hi : lo);
        }
    __syncthreads();  // every wave is done with the operand stages in LDS
    float* sums = reinterpret_cast<float*>(lds + 2 * kBigStageBytes / 16);  // [8 waves][128 rows]
    if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) sums[wave * 128 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3)] = ssp[i][r];
    }
    __syncthreads();
    uint16_t* st16 = reinterpret_cast<uint16_t*>(lds);  // [256 rows][256 columns] bf16
    const int cb = 128 * (wq >> 1);                      // this head's first column in the stage
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);  // row within the wave's 128
            const float ss = ssp[i][r] + sums[(wave ^ 1) * 128 + rl];
            const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + ep.eps);
            const int row = wr + rl;
            const int gm = min(m0 + row, p.M - 1);
            const float2 cs = ep.cs[(int64_t)gm * 64 + d0];
            const float a = acc[i][0][r] * (rinv * g[0]), bb = acc[i][1][r] * (rinv * g[1]);
            const int d1 = d0 + 64;
            st16[row * 256 + cb + 8 * ((d0 >> 3) ^ (row & 15)) + (d0 & 7)] = (uint16_t)f32_to_bf16_bits(a * cs.x - bb * cs.y);
            st16[row * 256 + cb + 8 * ((d1 >> 3) ^ (row & 15)) + (d1 & 7)] = (uint16_t)f32_to_bf16_bits(bb * cs.x + a * cs.y);
        }
    }
    __syncthreads();
    // 256 rows x 2 heads x 16 chunks = 8192 chunks, 16 per thread: rows
    // 16 it + (tid % 16), it = 0..15, chunk (tid / 16) % 16.  The 16 slots are
    // loaded before any store depends on them.
    const int hs = tid >> 8;                       // head of the pair this thread stores
    const int headst = ((n0 >> 7) + hs) & 7;
    const int tk = tid & 15, c = (tid >> 4) & 15;
    int64_t slots[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int gm = m0 + 16 * it + tk;
        slots[it] = gm < p.M ? ep.slot[gm] : -1;
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int row = 16 * it + tk;
        const int64_t slot = slots[it];
        if (slot < 0 || slot >= nslots) continue;
        const uint4 w = *reinterpret_cast<const uint4*>(st16 + row * 256 + 128 * hs + 8 * (c ^ (row & 15)));
        uint16_t* blk = cache + ((slot >> 4) * 8 + headst) * 2048;
        *reinterpret_cast<uint4*>(blk + 256 * (c & 7) + 8 * ((int)(slot & 15) + 16 * (c >> 3))) = w;
    }
}

// (cos, sin) of pos[m] * inv_freq[i] for every fused row: fp64 angle and
// range reduction, fp32 sincos.
struct RopeTabParams { const int32_t* pos; float2* cs; int M; double inv_freq[64]; };
__device__ __forceinline__ void rope_entry(const RopeTabParams& p, int m, int i) {
    double ang = (double)p.pos[m] * p.inv_freq[i];
    const double two_pi = 6.283185307179586;
    ang -= rint(ang * (1.0 / two_pi)) * two_pi;
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    p.cs[m * 64 + i] = make_float2(cs, sn);
}
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTabParams p) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.M * 64) return;
    rope_entry(p, idx >> 6, idx & 63);
}

// Sum split-K partials of one row, RMSNorm with g_c, store H_t.  The split
// loop is unrolled to kMaxKs so all partial loads of a row are in flight at once.
constexpr int kMaxKs = kGemmMaxKs;

// Split-K path (ks partials): 640 threads x 4 consecutive columns = one
// 2560-wide row per workgroup, all ks partial loads of a thread in flight.
constexpr int kNormThreads = DFLASH_D / 4;

// Four consecutive values (c0 a multiple of 4) in one store: ht lies in the
// 256-byte aligned workspace and ht_out is 16-byte aligned by the contract.
__device__ __forceinline__ void store4(float* p, const float* h) {
    *reinterpret_cast<float4*>(p) = make_float4(h[0], h[1], h[2], h[3]);
}
__device__ __forceinline__ void store4(uint16_t* p, const float* h) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
}
template <typename T>
__device__ __forceinline__ void norm_store(const float* y, float rinv, const T* gc, int64_t base, int c0, T* ht,
                                           T* ht_out) {
    float h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = Elem<T>::load(gc, c0 + e) * (y[e] * rinv);
    store4(ht + base + c0, h);
    if (ht_out) store4(ht_out + base + c0, h);
}

// With rp.cs set, the workgroup of row m also writes row m's RoPE table.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void fuse_norm_kernel(const float* part, int ks, int M, const T* gc,
                                                                float eps, T* ht, T* ht_out, RopeTabParams rp) {
    constexpr int D = DFLASH_D;
    const int m = blockIdx.x, tid = threadIdx.x;
    if (rp.cs && tid < 64) rope_entry(rp, m, tid);
    float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxKs; ++s) {
        if (s < ks) {
            const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)s * M + m) * D + 4 * tid);
            y[0] += v.x; y[1] += v.y; y[2] += v.z; y[3] += v.w;
        }
    }
    float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    ss = wave_sum(ss);
    __shared__ float red[kNormThreads / 64];
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / 64; ++i) tot += red[i];
    const float rinv = 1.0f / sqrtf(tot * (1.0f / D) + eps);
    norm_store(y, rinv, gc, (int64_t)m * D, 4 * tid, ht, ht_out);
}

// Single-partial path (large M): one wave per row, 4 rows per workgroup, ten
// 16-byte loads per lane in flight, a wave-only reduction.  Under stream-K
// (sk_q > 0) float4 i of a lane lies in column tile i (256 columns), whose
// products sit in the slots of the workgroups whose runs met that tile; they
// are added in slot order.
constexpr int kMaxSkSlots = 4;
template <typename T>
__global__ __launch_bounds__(kThreads) void fuse_norm_rows_kernel(const float* part, int M, const T* gc, float eps,
                                                                 T* ht, T* ht_out, int sk_q, int nk) {
    constexpr int D = DFLASH_D, PER = D / (64 * 4);  // 10 float4 per lane
    static_assert(PER * 256 == D, "one float4 of a lane per 256-column tile");
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (m >= M) return;
    const float4* row = reinterpret_cast<const float4*>(part + (int64_t)m * D);
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = row[64 * i + lane];
    if (sk_q > 0) {
        // Every slot load in flight before the first add.  The workgroup's
        // four rows share a row tile, so the slot counts are scalar work
        // (tile index times 200 stays below 2^31).
        const int tiles_m = (M + BMB - 1) / BMB, tm = blockIdx.x / (BMB / 4);
        const int64_t slot_stride = (int64_t)M * D / 4;
        int n[PER];
        float4 w[kMaxSkSlots - 1][PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const unsigned t = (unsigned)sk_tile_index(tm, i, tiles_m, PER), q = (unsigned)sk_q, k = (unsigned)nk;
            n[i] = (int)(((t + 1) * k - 1) / q - t * k / q) + 1;
        }
#pragma unroll
        for (int sl = 1; sl < kMaxSkSlots; ++sl)
#pragma unroll
            for (int i = 0; i < PER; ++i)
                w[sl - 1][i] = sl < n[i] ? row[sl * slot_stride + 64 * i + lane] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sl = 1; sl < kMaxSkSlots; ++sl)
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (sl < n[i]) {
                    v[i].x += w[sl - 1][i].x; v[i].y += w[sl - 1][i].y;
                    v[i].z += w[sl - 1][i].z; v[i].w += w[sl - 1][i].w;
                }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float y[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        norm_store(y, rinv, gc, (int64_t)m * D, 4 * (64 * i + lane), ht, ht_out);
    }
}

struct KvParams {
    const float* part; int ks; int M; int N;
    const void* gk; float eps;
    const int32_t* pos; const int64_t* slot;
    void* kc[5]; void* vc[5]; int64_t num_pages;
    double inv_freq[64];  // theta^(-i/64), computed on the host in fp64
};

// One wave per (row, 128-wide head of the [K_0 | V_0 | K_1 | ...] output).
template <typename T>
__global__ __launch_bounds__(kThreads) void fuse_kv_kernel(KvParams p) {
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int hidx = blockIdx.y * 4 + (threadIdx.x >> 6);  // [layer][K/V][head]
    const int l = hidx >> 4, kv = (hidx >> 3) & 1, head = hidx & 7;
    const int64_t slot = p.slot[m];
    if (slot < 0 || slot >= p.num_pages * 16) return;
    const int64_t page = slot >> 4;
    const int t = (int)(slot & 15);
    const int n0 = hidx * 128;
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxKs; ++s) {
        if (s < p.ks) {
            const float* row = p.part + ((int64_t)s * p.M + m) * p.N + n0;
            x0 += row[lane];
            x1 += row[lane + 64];
        }
    }
    const int d0 = lane, d1 = lane + 64;
    if (kv == 0) {
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + p.eps);
        const T* gk = static_cast<const T*>(p.gk) + l * 128;
        const float a = Elem<T>::load(gk, d0) * (x0 * rinv);
        const float b = Elem<T>::load(gk, d1) * (x1 * rinv);
        double ang = (double)p.pos[m] * p.inv_freq[lane];
        const double two_pi = 6.283185307179586;
        ang -= rint(ang * (1.0 / two_pi)) * two_pi;
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        T* kc = static_cast<T*>(p.kc[l]) + (page * 8 + head) * 2048;
        const int o0 = 256 * ((d0 & 63) >> 3) + 8 * (t + 16 * (d0 >> 6)) + (d0 & 7);
        const int o1 = 256 * ((d1 & 63) >> 3) + 8 * (t + 16 * (d1 >> 6)) + (d1 & 7);
        Elem<T>::store(kc, o0, a * cs - b * sn);
        Elem<T>::store(kc, o1, b * cs + a * sn);
    } else {
        T* vc = static_cast<T*>(p.vc[l]) + (page * 8 + head) * 2048;
        const int te = ((t >> 3) << 2) | (t & 3), th = (t >> 2) & 1;
        const int o0 = 512 * (d0 >> 5) + 256 * th + 8 * (d0 & 31) + te;
        const int o1 = 512 * (d1 >> 5) + 256 * th + 8 * (d1 & 31) + te;
        Elem<T>::store(vc, o0, x0);
        Elem<T>::store(vc, o1, x1);
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Large fused row counts use the 256x256 kernel (no split-K, fused K/V
// epilogue); small ones the 128x128 split-K kernel.
constexpr int kBigM = 4096;   // from here the 256x256 kernel (no split-K) beats the split-K one
constexpr int kPairTiles = 256;  // K/V GEMM tiles that one 512-thread workgroup per CU covers in one round
constexpr int kSkWorkgroups = 256;  // stream-K runs of the big first GEMM: one 8-wave workgroup per CU

FusePlan fuse_plan(const dflash_fuse_args& a) {
    FusePlan pl;
    const int M = (int)a.M;
    const int N2 = a.num_layers * 2048;
    const bool bf = a.dtype == DFLASH_BF16;
    pl.big = bf && M >= kBigM;
    pl.ks1 = pl.big ? 1 : bf ? gemm_split(M, DFLASH_D, DFLASH_NCAPTURE * DFLASH_D)
                             : gemm_split_f32(M, DFLASH_D, DFLASH_NCAPTURE * DFLASH_D);
    pl.ks2 = pl.big ? 1 : bf ? gemm_split(M, N2, DFLASH_D) : gemm_split_f32(M, N2, DFLASH_D);
    // bf16 below kBigM: where the K/V GEMM's tiles fit one 512-thread
    // workgroup per CU, it runs unsplit on two k-groups with the K/V epilogue
    // (no partials, no K/V kernel).  The first GEMM keeps its split-K
    // partials: on two k-groups with half the splits it measured slower
    // (31.9 against 28.9 us at M = 302) than the norm kernel gains from
    // reading half the partials (5.6 against 6.9 us).
    pl.pair2 = bf && !pl.big && ((M + 127) / 128) * (N2 / 128) <= kPairTiles;
    if (pl.pair2) pl.ks2 = 1;
    // Stream-K for the big first GEMM where its tiles do not fill whole
    // rounds of one workgroup per CU (M = 4096: 160 tiles on 256 CUs): the
    // k-tiles of all tiles are cut into kSkWorkgroups equal runs.
    pl.sk_q = 0;
    pl.sk_slots = 1;
    if (pl.big) {
        const int tiles_m = (M + BMB - 1) / BMB, tiles = tiles_m * (DFLASH_D / BNB);
        const int64_t nk = DFLASH_NCAPTURE * DFLASH_D / BKB;
        if (tiles % kSkWorkgroups != 0 && (int64_t)tiles * nk < ((int64_t)1 << 31)) {
            const int64_t units = (int64_t)tiles * nk;
            pl.sk_q = (int)((units + kSkWorkgroups - 1) / kSkWorkgroups);
            for (int64_t t = 0; t < tiles; ++t) {
                const int n = (int)(((t + 1) * nk - 1) / pl.sk_q - t * nk / pl.sk_q) + 1;
                if (n > pl.sk_slots) pl.sk_slots = n;
            }
            if (pl.sk_slots > kMaxSkSlots) { pl.sk_q = 0; pl.sk_slots = 1; }
        }
    }
    const size_t es = bf ? 2 : 4;
    pl.off_part1 = 0;
    pl.off_ht = align256((size_t)pl.ks1 * pl.sk_slots * M * DFLASH_D * 4);
    pl.off_part2 = pl.off_ht + align256((size_t)M * DFLASH_D * es);
    // The big and pair K/V paths need no second partial buffer, only the RoPE table.
    pl.ws_bytes = pl.off_part2 + (pl.big || pl.pair2 ? align256((size_t)M * 64 * sizeof(float2))
                                                     : align256((size_t)pl.ks2 * M * N2 * 4));
    return pl;
}

hipError_t launch_gemm_big_head(const GemmParams& g, const HeadEpilogue& hp, hipStream_t s) {
    const int tiles = ((g.M + BMB - 1) / BMB) * (g.N / BNB);
    const int grid = std::min((tiles + kXcds - 1) / kXcds * kXcds, kSkWorkgroups);
    gemm_bf16_big_kernel<2><<<grid, kBigThreads, 0, s>>>(g, KvEpilogue{}, hp);
    return hipGetLastError();
}

hipError_t launch_fuse(const dflash_fuse_args& a, const FusePlan& pl, void* ws, hipStream_t s) {
    const int M = (int)a.M;
    if (M == 0) return hipSuccess;
    char* w = static_cast<char*>(ws);
    float* part1 = reinterpret_cast<float*>(w + pl.off_part1);
    void* ht = w + pl.off_ht;
    float* part2 = reinterpret_cast<float*>(w + pl.off_part2);
    const int N2 = a.num_layers * 2048;
    const bool bf = a.dtype == DFLASH_BF16;
    double inv_freq[64];
    for (int i = 0; i < 64; ++i) inv_freq[i] = std::pow((double)a.rope_theta, -(double)i / 64.0);

    GemmParams g1 = {};
    for (int i = 0; i < 5; ++i) g1.aseg[i] = a.hs[i];
    g1.a_stride = a.hs_stride; g1.seg_w = DFLASH_D;
    g1.b = a.wc; g1.M = M; g1.N = DFLASH_D; g1.K = DFLASH_NCAPTURE * DFLASH_D;
    gemm_set_split(g1, a.dtype, pl.ks1);
    g1.part = part1;
    KvEpilogue ep = {};
    if (pl.big && pl.sk_q > 0) {
        g1.sk_q = pl.sk_q;
        gemm_bf16_big_kernel<0, true><<<kSkWorkgroups, kBigThreads, 0, s>>>(g1, ep, HeadEpilogue{});
    } else if (pl.big) {
        const int tiles = ((M + BMB - 1) / BMB) * (DFLASH_D / BNB);
        gemm_bf16_big_kernel<0><<<(tiles + kXcds - 1) / kXcds * kXcds, kBigThreads, 0, s>>>(g1, ep, HeadEpilogue{});
    } else {
        hipError_t e = launch_gemm(g1, a.dtype, s);
        if (e != hipSuccess) return e;
    }

    // The RoPE table of the K/V epilogues (big and pair paths), after H_t in
    // the workspace: written by the norm kernel where it runs one workgroup
    // per row, else by its own launch.
    RopeTabParams rp = {};
    if (pl.big || pl.pair2) {
        rp.pos = a.pos; rp.cs = reinterpret_cast<float2*>(part2); rp.M = M;
        for (int i = 0; i < 64; ++i) rp.inv_freq[i] = inv_freq[i];
        ep.cs = rp.cs;
        ep.gk = a.gk; ep.eps = a.eps; ep.slot = a.slot; ep.num_pages = a.num_pages;
        for (int i = 0; i < 5; ++i) { ep.kc[i] = a.k_cache[i]; ep.vc[i] = a.v_cache[i]; }
    }
    const bool rope_in_norm = pl.ks1 > 1 && rp.cs != nullptr;
    if (rp.cs && !rope_in_norm) rope_table_kernel<<<(M * 64 + 255) / 256, 256, 0, s>>>(rp);

    if (pl.ks1 == 1) {
        const int nb = (M + 3) / 4;
        if (bf)
            fuse_norm_rows_kernel<uint16_t><<<nb, kThreads, 0, s>>>(part1, M, static_cast<const uint16_t*>(a.gc), a.eps,
                                                                    static_cast<uint16_t*>(ht),
                                                                    static_cast<uint16_t*>(a.ht_out), pl.sk_q,
                                                                    g1.K / BKB);
        else
            fuse_norm_rows_kernel<float><<<nb, kThreads, 0, s>>>(part1, M, static_cast<const float*>(a.gc), a.eps,
                                                                 static_cast<float*>(ht), static_cast<float*>(a.ht_out),
                                                                 0, 1);
    } else if (bf) {
        fuse_norm_kernel<uint16_t><<<M, kNormThreads, 0, s>>>(part1, pl.ks1, M, static_cast<const uint16_t*>(a.gc),
                                                              a.eps, static_cast<uint16_t*>(ht),
                                                              static_cast<uint16_t*>(a.ht_out), rp);
    } else {
        fuse_norm_kernel<float><<<M, kNormThreads, 0, s>>>(part1, pl.ks1, M, static_cast<const float*>(a.gc), a.eps,
                                                           static_cast<float*>(ht), static_cast<float*>(a.ht_out), rp);
    }

    GemmParams g2 = {};
    g2.aseg[0] = ht; g2.a_stride = DFLASH_D; g2.seg_w = DFLASH_D;
    g2.b = a.wkv; g2.M = M; g2.N = N2; g2.K = DFLASH_D;
    gemm_set_split(g2, a.dtype, pl.ks2);
    g2.part = part2;
    if (pl.big) {
        const int tiles = ((M + BMB - 1) / BMB) * (N2 / BNB);
        gemm_bf16_big_kernel<1><<<(tiles + kXcds - 1) / kXcds * kXcds, kBigThreads, 0, s>>>(g2, ep, HeadEpilogue{});
        return hipGetLastError();
    }
    if (pl.pair2) return launch_gemm_pair(g2, ep, s);
    hipError_t e = launch_gemm(g2, a.dtype, s);
    if (e != hipSuccess) return e;

    KvParams kp;
    kp.part = part2; kp.ks = pl.ks2; kp.M = M; kp.N = N2;
    kp.gk = a.gk; kp.eps = a.eps;
    for (int i = 0; i < 64; ++i) kp.inv_freq[i] = inv_freq[i];
    kp.pos = a.pos; kp.slot = a.slot; kp.num_pages = a.num_pages;
    for (int i = 0; i < 5; ++i) { kp.kc[i] = a.k_cache[i]; kp.vc[i] = a.v_cache[i]; }
    const dim3 gkv(M, a.num_layers * 4);
    if (bf) fuse_kv_kernel<uint16_t><<<gkv, kThreads, 0, s>>>(kp);
    else fuse_kv_kernel<float><<<gkv, kThreads, 0, s>>>(kp);
    return hipGetLastError();
}

}  // namespace dflash
