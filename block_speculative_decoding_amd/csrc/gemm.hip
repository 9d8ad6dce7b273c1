// Split-K bf16 GEMM with fused epilogues and plain fp32 GEMM (gfx950);
// interface in gemm.h.
//
// The bf16 kernel runs the 32x32x16 bf16 matrix instruction on operands
// staged through LDS by buffer loads that write LDS directly; tiles are laid out
// contiguously per XCD in 8-row groups so that tiles sharing a B panel run on
// the same L2.  Used where the row count is a few hundred to a few thousand
// (context fusion of newly verified rows, the draft layer's projections over
// B x 8 block rows): the weights stream once, split over K so that every CU
// gets a share.  Epilogues: fp32 split-K partials, bf16 products, SwiGLU of
// [gate ; up] tiles; and, on the two-k-group form (one 512-thread workgroup
// per tile, halves added through LDS), the context fusion's K/V injection or
// the draft Q/K/V head layout, which need no partials.
#include "device_common.h"
#include "gemm.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128;

// ---- bf16 GEMM: 128x128 tile, BK = 64, four waves of 64x64 (2x2 blocks of
// the 32x32x16 instruction), a two-stage LDS ring of 32 KiB stages (two
// workgroups per CU).  A stage holds A then B as [128 rows][8 chunks of 16 B];
// chunk c of row r sits at unit 8r + (c ^ swz8(r)), swz8(r) = (r >> 1) & 7.
// Operands reach LDS through buffer loads that write LDS directly, with fixed
// per-lane offsets; A rows past M read as zero (descriptor range).  The next
// substep's operand reads are in flight while the current one multiplies
// (inline-asm reads with explicit lgkmcnt waits), and the next stage's eight
// loads per thread go out between the four MFMAs of the last substep.
constexpr int BKD = 64;                      // k per stage (and per k-tile)
constexpr int kUnits = 2 * BM * 8;           // A then B, 16-byte units per stage
constexpr int kStageBytes = kUnits * 16;     // 32 KiB
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

constexpr int kFtPitch = 136;   // floats per row of the fp32 [128][.] tile in LDS (conflict-free halves)

// K/V epilogue of one 128x128 tile: rows m0 .. m0 + 127, column tile tn =
// one head of one layer ([layer][K/V][head], 128 columns each), from the
// fp32 tile ft in LDS.  512 threads, four per row: thread q of a row owns
// dims 8q .. 8q+7 and 8q+32 .. 8q+39 and their RoPE partners d + 64.
//   K: k_norm over the head's 128 values (the four threads' sums of squares
//      added by two lane swaps), RoPE on (d, d + 64) with the (cos, sin)
//      table, bf16; each run of 8 dims of one token is one 16-byte granule
//      of the page layout: four stores per thread.
//   V: as projected, bf16; a V granule holds one dim of 8 tokens, so each
//      value is its own 2-byte store.
__device__ __forceinline__ void kv_epilogue(const float* ft, int M, int m0, int tn, const KvEpilogue& ep, int tid) {
    const int row = tid >> 2, q = tid & 3;
    const int l = tn >> 4, isv = (tn >> 3) & 1, head = tn & 7;
    const int gm = m0 + row;
    const int64_t nslots = ep.num_pages * 16;
    const int64_t slot = gm < M ? ep.slot[gm] : -1;
    const bool ok = slot >= 0 && slot < nslots;
    const int tt = (int)(slot & 15);
    const float* fr = ft + row * kFtPitch;
    float x[2][8], y[2][8];   // dims 8q + 32h + e and their partners + 64
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const float4 a = *reinterpret_cast<const float4*>(fr + 8 * q + 32 * h + 4 * v);
            const float4 b = *reinterpret_cast<const float4*>(fr + 64 + 8 * q + 32 * h + 4 * v);
            x[h][4 * v + 0] = a.x; x[h][4 * v + 1] = a.y; x[h][4 * v + 2] = a.z; x[h][4 * v + 3] = a.w;
            y[h][4 * v + 0] = b.x; y[h][4 * v + 1] = b.y; y[h][4 * v + 2] = b.z; y[h][4 * v + 3] = b.w;
        }
    if (!isv) {
        float ss = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[h][e] * x[h][e] + y[h][e] * y[h][e];
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        if (!ok) return;
        const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + ep.eps);
        const uint16_t* gk = static_cast<const uint16_t*>(ep.gk) + l * 128;
        const float2* cs = ep.cs + (int64_t)gm * 64;
        uint16_t* blk = static_cast<uint16_t*>(ep.kc[l]) + ((slot >> 4) * 8 + head) * 2048;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t w1[4], w2[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                float o1[2], o2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int d = 8 * q + 32 * h + e + u;
                    const float a = x[h][e + u] * (rinv * bf16_bits_to_f32(gk[d]));
                    const float b = y[h][e + u] * (rinv * bf16_bits_to_f32(gk[d + 64]));
                    const float2 c = cs[d];
                    o1[u] = a * c.x - b * c.y;
                    o2[u] = b * c.x + a * c.y;
                }
                w1[e >> 1] = pack_bf16x2(o1[0], o1[1]);
                w2[e >> 1] = pack_bf16x2(o2[0], o2[1]);
            }
            *reinterpret_cast<uint4*>(blk + 256 * (q + 4 * h) + 8 * tt) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
            *reinterpret_cast<uint4*>(blk + 256 * (q + 4 * h) + 8 * (tt + 16)) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        }
        return;
    }
    if (!ok) return;
    uint16_t* blk = static_cast<uint16_t*>(ep.vc[l]) + ((slot >> 4) * 8 + head) * 2048;
    const int te = ((tt >> 3) << 2) | (tt & 3), th = (tt >> 2) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * q + 32 * h + e;
            blk[512 * (d >> 5) + 256 * th + 8 * (d & 31) + te] = (uint16_t)f32_to_bf16_bits(x[h][e]);
            blk[512 * ((d + 64) >> 5) + 256 * th + 8 * (d & 31) + te] = (uint16_t)f32_to_bf16_bits(y[h][e]);
        }
}

// Q/K/V head-layout epilogue of one 128x128 tile (column tile tn = one
// head: q heads 0..31, then k and v heads 0..7) from the fp32 tile ft in
// LDS.  512 threads, four per row, 32 dims each: a row's 128 dims are 256
// contiguous bytes of the destination, and a sequence's 8 rows follow each
// other.
__device__ __forceinline__ void qkv_epilogue(const float* ft, int M, int m0, int tn, const QkvEpilogue& qe, int tid) {
    const int row = tid >> 2, q4 = tid & 3;
    const int m = m0 + row;
    if (m >= M) return;
    const int b = m >> 3, j = m & 7;
    uint16_t* dst = tn < 32 ? qe.q + (((int64_t)b * 32 + tn) * 8 + j) * 128
                  : tn < 40 ? qe.k + (((int64_t)b * 8 + (tn - 32)) * 8 + j) * 128
                            : qe.v + (((int64_t)b * 8 + (tn - 40)) * 8 + j) * 128;
    const float* fr = ft + row * kFtPitch + 32 * q4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 a = *reinterpret_cast<const float4*>(fr + 8 * v);
        const float4 c = *reinterpret_cast<const float4*>(fr + 8 * v + 4);
        *reinterpret_cast<uint4*>(dst + 32 * q4 + 8 * v) =
            make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(c.x, c.y), pack_bf16x2(c.z, c.w));
    }
}

constexpr int kEpiNone = 0, kEpiKv = 1, kEpiQkv = 2;

// KG groups of four waves per workgroup (KG = 1: 256 threads, two
// workgroups per CU; KG = 2: 512 threads, one per CU).  Group g runs the
// loop above over its share of the tile's k-tiles with its own two stages;
// both groups take the same number of steps (a group past its share loads a
// clamped k-tile and skips the MFMAs), so the workgroup barriers pair up.
// With KG = 2 group 1 then hands its products to group 0 through LDS, and
// the summed tile goes through the K/V or the Q/K/V head-layout epilogue.

template <int KG, int EPI>
__global__ __launch_bounds__(kThreads * KG, 2 / KG) void gemm_bf16_kernel(GemmParams p, KvEpilogue ep, QkvEpilogue qe) {
    static_assert((KG == 1 && EPI == kEpiNone) || (KG == 2 && EPI != kEpiNone),
                  "one k-group with partials or bf16 out; two with the K/V or Q/K/V epilogue");
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
    const TileId t = tile_id(p, tiles_m, tiles_n);
    if (!t.valid) return;
    const int nk = p.K / BKD;
    const int kt0 = t.ks * p.kt_per_split;
    const int kt1 = min(nk, kt0 + p.kt_per_split);
    if (kt0 >= kt1) return;
    const int nloc = kt1 - kt0;

    __shared__ __attribute__((aligned(1024))) uint4 lds[KG * 2 * kUnits];

    const int tid = threadIdx.x, lane = tid & 63;
    // The group index is read as wave-uniform: every quantity derived from it
    // (k range, descriptors, the padding-step test) is then scalar, so the
    // padding steps skip their MFMAs by a branch (matrix instructions ignore
    // the exec mask) and the buffer descriptors sit in SGPRs.
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / kThreads);
    const int tg = tid % kThreads, wave = tg >> 6;   // thread and wave within the group
    const int nh = (nloc + KG - 1) / KG;              // steps every group runs
    const int g0 = kt0 + grp * nh;
    const int ng = max(0, min(nloc - grp * nh, nh));  // k-tiles this group owns
    auto ktile = [&](int i) { return ng > 0 ? g0 + min(i, ng - 1) : kt0; };
    const int m0 = t.tm * BM, n0 = t.tn * BN;
    // SwiGLU tiles: B rows 0..63 of the tile are gate rows 64 tn .., rows
    // 64..127 the up rows N/2 further on.
    const bool swiglu = EPI == kEpiNone && p.swiglu_out != nullptr;
    const int half = p.N / 2;
    const uint16_t* bmat = static_cast<const uint16_t*>(p.b) + (int64_t)(swiglu ? 64 * t.tn : n0) * p.K;
    const uint32_t brows = swiglu ? (uint32_t)(half + 64) : (uint32_t)BN;   // rows the descriptor spans
    const void *aseg0 = p.aseg[0], *aseg1 = p.aseg[1], *aseg2 = p.aseg[2], *aseg3 = p.aseg[3], *aseg4 = p.aseg[4];
    const uint32_t arows = (uint32_t)min(p.M - m0, BM);

    // Load j (0..3) of a thread covers unit P = j * 256 + tg of the A (or B)
    // half: row P >> 3, chunk (P & 7) ^ swz8(row).
    uint32_t voa[4], vob[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int P = j * kThreads + tg, r = P >> 3, c = (P & 7) ^ swz8(r);
        const int rb = swiglu && r >= 64 ? half - 64 + r : r;
        voa[j] = (uint32_t)(r * (int)p.a_stride + 8 * c) * 2u;
        vob[j] = (uint32_t)(rb * p.K + 8 * c) * 2u;
    }
    // Both operands' buffer descriptors for k-tile kt, computed once per
    // k-tile at the top of the loop: the loads themselves sit between matrix
    // instructions, where a segment select (a division and a five-way pointer
    // choice per load) would hold up the next one.
    struct StageSrc { i32x4 a, b; };
    auto stage_src = [&](int kt) {
        const int kg = kt * BKD;
        const int seg = kg / p.seg_w;
        const int kc = kg - seg * p.seg_w;
        const void* av = seg == 0 ? aseg0 : seg == 1 ? aseg1 : seg == 2 ? aseg2 : seg == 3 ? aseg3 : aseg4;
        const uint16_t* a = static_cast<const uint16_t*>(av) + (int64_t)m0 * p.a_stride + kc;
        StageSrc s;
        s.a = buffer_rsrc(a, arows * (uint32_t)p.a_stride * 2u - (uint32_t)kc * 2u);
        s.b = buffer_rsrc(bmat + kg, brows * (uint32_t)p.K * 2u - (uint32_t)kg * 2u);
        return s;
    };
    // The wave index read as wave-uniform, so that each load's LDS base (M0)
    // is scalar arithmetic.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    uint4* const gl = lds + grp * 2 * kUnits;  // this group's two stages
    auto load_part = [&](const StageSrc& src, int slot, int part) {
        uint4* sb = gl + slot * kUnits + wave_s * 64;
        if (part < 4) {
            llvm_amdgcn_raw_buffer_load_lds(src.a, (__attribute__((address_space(3))) uint32_t*)(sb + part * kThreads),
                                            16, (int)voa[part], 0, 0, 0);
        } else {
            const int j = part - 4;
            llvm_amdgcn_raw_buffer_load_lds(
                src.b, (__attribute__((address_space(3))) uint32_t*)(sb + BM * 8 + j * kThreads), 16, (int)vob[j], 0, 0, 0);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    const int lr = lane & 31, lh = lane >> 5;
    // Rows wr + 32 i + lr (A) and wc + 32 j + lr (B) all have swizzle
    // swz8(lr); substep s flips chunk bits 1-2 (address ^ 32 s), block 1 adds
    // 32 rows (4096 bytes).
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint4*)gl);
    const uint32_t a_lane = lds0 + 128u * (wr + lr) + 16u * (lh ^ swz8(lr));
    const uint32_t b_lane = lds0 + 16u * BM * 8 + 128u * (wc + lr) + 16u * (lh ^ swz8(lr));
    auto rd = [&](int slot, int ks, bf16x8* a, bf16x8* b) {
        const uint32_t so = (uint32_t)slot * kStageBytes, x = 32u * ks;
        const uint32_t aa = (a_lane + so) ^ x, bb = (b_lane + so) ^ x;
        a[0] = lds_read16<0>(aa);
        a[1] = lds_read16<4096>(aa);
        b[0] = lds_read16<0>(bb);
        b[1] = lds_read16<4096>(bb);
    };
    auto mm = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    };

    bf16x8 fa[2][2], fb[2][2];
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
        const StageSrc src = stage_src(ktile(s0));
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2) load_part(src, s0, t2);
    }
    wait_vm<8>();  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    rd(0, 0, fa[0], fb[0]);
    for (int i = 0; i < nh; ++i) {
        const int slot = i & 1;
        const bool own = KG == 1 || i < ng;   // uniform per group: false only on a group's padding steps
        const StageSrc nsrc = stage_src(ktile(i + 2));
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            rd(slot, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            wait_lgkm<4>();  // substep s's reads (issued before these 4) are back
            __builtin_amdgcn_sched_barrier(0);
            if (own) mm(fa[s & 1], fb[s & 1]);
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
            if ((t2 & 1) == 0 && own) {
                const int q = t2 >> 1;
                acc[q >> 1][q & 1] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][q >> 1], fb[1][q & 1], acc[q >> 1][q & 1], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            load_part(nsrc, slot, t2);  // stage i+2 into the slot stage i used
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vm<0>();  // the clamped trailing loads must land before the workgroup exits
    wait_lgkm<0>();

    // Lane holds column lr of each 32x32 block, rows 8*(r/4) + 4*lh + (r%4).
    float* const ft = reinterpret_cast<float*>(lds);  // [128][kFtPitch] fp32 tile (KG == 2)
    auto ft_at = [&](int i, int j, int r) {
        return (wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3)) * kFtPitch + wc + 32 * j + lr;
    };
    if (KG == 2) {
        __syncthreads();  // both groups are done with their stages
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) ft[ft_at(i, j, r)] = acc[i][j][r];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = ft_at(i, j, r);
                        ft[o] += acc[i][j][r];
                    }
        }
        __syncthreads();
        if (EPI == kEpiKv) kv_epilogue(ft, p.M, m0, t.tn, ep, tid);
        else qkv_epilogue(ft, p.M, m0, t.tn, qe, tid);
        return;
    }
    if (swiglu) {
        // The up waves (columns 64..127) hand their products to the gate
        // waves through LDS ([128][68] fp32 over the operand stages); each
        // gate wave then stores silu(gate) * up for its 64 x 64 block.
        __syncthreads();  // every wave is done with the operand stages
        constexpr int kUpPitch = 68;
        float* up = reinterpret_cast<float*>(lds);
        if (wc == 64) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        up[(wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3)) * kUpPitch + 32 * j + lr] = acc[i][j][r];
        }
        __syncthreads();
        if (wc == 64) return;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rl = wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int gm = m0 + rl;
                    const float g = acc[i][j][r], u = up[rl * kUpPitch + 32 * j + lr];
                    if (gm < p.M)
                        p.swiglu_out[(int64_t)gm * half + 64 * t.tn + 32 * j + lr] =
                            (uint16_t)f32_to_bf16_bits(g / (1.0f + expf(-g)) * u);
                }
        return;
    }
    if (p.out_bf16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = m0 + wr + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int gn = n0 + wc + 32 * j + lr;
                    if (gm < p.M) p.out_bf16[(int64_t)gm * p.N + gn] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
                }
        return;
    }
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
// fp32 (small fp32 workloads): 64x64 tiles, 256 threads of 4x4 outputs,
// 16-deep k steps staged in LDS from 16-byte loads, the next step's loads in
// registers while the current one multiplies; split-K over blockIdx.z in
// units of 64 k (kt_per_split), each split to its own partial.
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p) {
    const int tm = blockIdx.x, tn = blockIdx.y, sp = blockIdx.z;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    __shared__ __align__(16) float as[16][68], bs[16][68];
    float acc[4][4] = {};
    const float* bmat = static_cast<const float*>(p.b);
    const int kb = sp * p.kt_per_split * BKD;
    const int ke = min(p.K, kb + p.kt_per_split * BKD);
    // loader: row lr of the tile, k quad lq of the step
    const int lr = tid >> 2, lq = (tid & 3) * 4;
    const int gm = tm * 64 + lr;
    float4 ra = make_float4(0.f, 0.f, 0.f, 0.f), rb = ra;
    auto load = [&](int k0) {
        const int seg = k0 / p.seg_w;            // a 16-wide step never crosses a segment
        const int kc = k0 - seg * p.seg_w;
        const float* a = static_cast<const float*>(p.aseg[seg]);
        ra = gm < p.M ? *reinterpret_cast<const float4*>(a + (int64_t)gm * p.a_stride + kc + lq)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
        rb = *reinterpret_cast<const float4*>(bmat + (int64_t)(tn * 64 + lr) * p.K + k0 + lq);
    };
    if (kb < ke) load(kb);
    for (int k0 = kb; k0 < ke; k0 += 16) {
        __syncthreads();   // the previous step's reads of as / bs are done
        as[lq][lr] = ra.x; as[lq + 1][lr] = ra.y; as[lq + 2][lr] = ra.z; as[lq + 3][lr] = ra.w;
        bs[lq][lr] = rb.x; bs[lq + 1][lr] = rb.y; bs[lq + 2][lr] = rb.z; bs[lq + 3][lr] = rb.w;
        __syncthreads();
        if (k0 + 16 < ke) load(k0 + 16);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const float4 av = *reinterpret_cast<const float4*>(&as[kk][ty * 4]);
            const float4 bv = *reinterpret_cast<const float4*>(&bs[kk][tx * 4]);
            const float a4[4] = {av.x, av.y, av.z, av.w}, b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], b4[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = tm * 64 + ty * 4 + i;
        if (m >= p.M) continue;
        *reinterpret_cast<float4*>(p.part + ((int64_t)sp * p.M + m) * p.N + tn * 64 + tx * 4) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
}

}  // namespace

int gemm_split(int M, int N, int K) {
    const int tiles = ((M + BM - 1) / BM) * (N / BN);
    const int nk = K / BKD;
    int ks = 512 / tiles;                 // 2 workgroups per CU on 256 CUs, one round
    if (ks > nk / 4) ks = nk / 4;         // keep >= 4 k-tiles (256 k) per split
    if (ks > kGemmMaxKs) ks = kGemmMaxKs;
    if (ks < 1) ks = 1;
    // Every split must own at least one k-tile: recount after rounding.
    const int per = (nk + ks - 1) / ks;
    return (nk + per - 1) / per;
}

int gemm_split_f32(int M, int N, int K) {
    const int tiles = ((M + 63) / 64) * (N / 64);
    const int nk = K / BKD;
    int ks = 512 / tiles;
    if (ks > nk / 2) ks = nk / 2;         // keep >= 2 k-tiles (128 k) per split
    if (ks > kGemmMaxKs) ks = kGemmMaxKs;
    if (ks < 1) ks = 1;
    const int per = (nk + ks - 1) / ks;
    return (nk + per - 1) / per;
}

hipError_t launch_gemm_pair(const GemmParams& g, const KvEpilogue& ep, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN) * g.ks;
    const int grid = (tiles + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
    gemm_bf16_kernel<2, kEpiKv><<<grid, 2 * kThreads, 0, s>>>(g, ep, QkvEpilogue{});
    return hipGetLastError();
}

hipError_t launch_gemm_pair_qkv(const GemmParams& g, const QkvEpilogue& qe, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN) * g.ks;
    const int grid = (tiles + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
    gemm_bf16_kernel<2, kEpiQkv><<<grid, 2 * kThreads, 0, s>>>(g, KvEpilogue{}, qe);
    return hipGetLastError();
}

void gemm_set_split(GemmParams& g, int dtype, int ks) {
    (void)dtype;
    g.ks = ks;
    g.kt_per_split = (g.K / BKD + ks - 1) / ks;
}

hipError_t launch_gemm(const GemmParams& g, int dtype, hipStream_t s) {
    if (dtype == DFLASH_BF16) {
        const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN) * g.ks;
        const int grid = (tiles + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
        gemm_bf16_kernel<1, kEpiNone><<<grid, kThreads, 0, s>>>(g, KvEpilogue{}, QkvEpilogue{});
    } else {
        gemm_f32_kernel<<<dim3((g.M + 63) / 64, g.N / 64, g.ks), kThreads, 0, s>>>(g);
    }
    return hipGetLastError();
}

}  // namespace dflash
