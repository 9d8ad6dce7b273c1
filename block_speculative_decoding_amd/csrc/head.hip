// Shared LM head over the block rows and the draft proposals (gfx950).
//
// "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash", sections
// "The parameter count exposes the real cost" (the drafter's output head is a
// copy of the target head, [262144, 2560]) and "The released serving cycle"
// (one forward over the eight block positions proposes all seven future
// tokens); "DFlash & DFlash2", section 4.2 (the target's unembedding head
// maps the output states to vocabulary logits).
//
// Launch sequence (keys: head_sample.h):
//   bf16 with 256 rows or more and V % 256 == 0 (fused):
//     gemm+sample -- the 256 x 256-tile projection; its epilogue rounds the
//                    tile to bf16, stores it as 16-byte chunks and folds the
//                    keys of rows k = 1..7 into one (key, index) per row and
//                    tile
//   otherwise:
//     gemm        -- the 128 x 128 kernel with one split and a direct bf16
//                    output (or the fp32 kernel)
//     sample      -- vocabulary-parallel over rows k = 1..7, one (key, index)
//                    per row and 8192-entry chunk
//   pick          -- one wave per row: the best partial is d_k; with
//                    draft_stats requested, the row's statistics partials
//                    are merged into (m, s) for verification
// Keys and statistics are computed from the stored (rounded) logits, so the
// proposals and q's normaliser are those of the values verification reads.
#include "device_common.h"
#include "gemm.h"
#include "head_sample.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = 8192;       // vocabulary entries per sampling workgroup (separate pass)

struct HeadParams {
    const void* logits;   // [B][8][V]
    const float* temp;    // [B]
    int B;
    int64_t V;
    uint64_t seed, offset;
    int nch;              // partials per proposal row
    KeyIdx* part;         // [B][7][nch]
    RowStat* spart;       // [B][7][nch] statistics partials of sampled rows (when dstats is set)
    int32_t* d;           // [B][7]
    float* dstats;        // optional [B][7][2]: (m, s) per proposal row
};

// Eight consecutive stored logits as fp32 (one 16-byte streaming load for
// bf16, two for fp32); offsets are multiples of 8.
template <typename T> struct Group8;
template <> struct Group8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
        const uint4 w = ld_stream(reinterpret_cast<const uint4*>(p));
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
};
template <> struct Group8<float> {
    static __device__ __forceinline__ void load(const float* p, float* f) {
        const uint4 a = ld_stream(reinterpret_cast<const uint4*>(p)), b = ld_stream(reinterpret_cast<const uint4*>(p + 4));
        f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
        f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
    }
};

// Separate sampling pass (rows below 256, or V not a multiple of 256):
// vocabulary-parallel over rows k = 1..7, one workgroup per 8192-entry chunk.
template <typename T>
__global__ __launch_bounds__(kThreads) void draft_sample_kernel(HeadParams p) {
    const int chunk = blockIdx.x % p.nch;
    const int row = blockIdx.x / p.nch;       // b * 7 + (k - 1)
    const int b = row / 7, k = row % 7 + 1;
    const float Tb = p.temp[b];
    const bool greedy = !(Tb > 0.f);
    const float invT = greedy ? 1.f : 1.0f / Tb;
    const T* z = static_cast<const T*>(p.logits) + ((int64_t)b * 8 + k) * p.V;
    const int64_t c0 = (int64_t)chunk * kChunk, c1 = min(p.V, c0 + kChunk);
    const uint64_t ctr1 = 8ull * (uint64_t)b + (uint64_t)k;
    const bool stats = !greedy && p.dstats != nullptr;
    const StatScale sc = stat_scale(greedy ? 1.f : Tb);
    float best = -INFINITY, sm = -INFINITY, ss = 0.f;
    int bi = 0x7FFFFFFF;
    // Every load of the thread is issued before any is used.
    constexpr int kIt = kChunk / (kThreads * 8);
    float f[kIt][8];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + threadIdx.x) * 8;
        if (i0 < c1) Group8<T>::load(z + i0, f[it]);
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + threadIdx.x) * 8;
        if (i0 < c1) {
            draft_best8(f[it], i0, greedy, invT, ctr1, p.seed, p.offset, best, bi);
            if (stats) stat_add8(f[it], sc, sm, ss);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        better(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
        if (stats) stat_merge(sm, ss, __shfl_xor(sm, o), __shfl_xor(ss, o), sc);
    }
    __shared__ KeyIdx sw[kThreads / 64];
    __shared__ RowStat sst[kThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        sw[threadIdx.x >> 6] = {best, bi};
        sst[threadIdx.x >> 6] = {sm, ss};
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) {
            better(best, bi, sw[w].key, sw[w].idx);
            if (stats) stat_merge(sm, ss, sst[w].m, sst[w].s, sc);
        }
        p.part[(int64_t)row * p.nch + chunk] = {best, bi};
        if (stats) p.spart[(int64_t)row * p.nch + chunk] = {sm, ss};
    }
}

// One wave per (sequence, proposal): the best of the row's partials.
__global__ __launch_bounds__(kThreads) void draft_pick_kernel(HeadParams p) {
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= p.B * 7) return;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = lane; c < p.nch; c += 64) {
        const KeyIdx kp = p.part[(int64_t)row * p.nch + c];
        better(best, bi, kp.key, kp.idx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) better(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
    if (lane == 0) p.d[row] = bi == 0x7FFFFFFF ? -1 : bi;   // no finite key (non-finite logits): -1
    if (!p.dstats) return;
    // Statistics: the row's largest partial maximum, then the partial sums
    // rescaled to it and added in fp64.  Greedy rows need none: (-inf, 0).
    const float Tb = p.temp[row / 7];
    float m = -INFINITY;
    if (Tb > 0.f) {
        for (int c = lane; c < p.nch; c += 64) m = fmaxf(m, p.spart[(int64_t)row * p.nch + c].m);
        m = wave_max(m);
    }
    double sum = 0.0;
    if (m != -INFINITY) {
        const double sc = 1.4426950408889634 / (double)Tb;
        for (int c = lane; c < p.nch; c += 64) {
            const RowStat st = p.spart[(int64_t)row * p.nch + c];
            if (st.m != -INFINITY) sum += (double)st.s * exp2((double)(st.m - m) * sc);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    }
    if (lane == 0) {
        p.dstats[2 * row] = m;
        p.dstats[2 * row + 1] = (float)sum;
    }
}

bool fused_path(const dflash_head_args& a) { return a.dtype == DFLASH_BF16 && 8 * a.B >= 256 && a.V % 256 == 0; }

}  // namespace

size_t head_workspace_bytes(int B, int64_t V) {
    // The fused path keeps one partial per row and 256-column tile, the
    // separate pass one per 8192-entry chunk: size for the larger; then as
    // many statistics partials.
    const int64_t n = (V + 255) / 256;
    return (((size_t)B * 7 * n * sizeof(KeyIdx) + 255) & ~(size_t)255) +
           (((size_t)B * 7 * n * sizeof(RowStat) + 255) & ~(size_t)255);
}

hipError_t launch_head(const dflash_head_args& a, void* ws, hipStream_t s) {
    const int M = 8 * a.B;
    GemmParams g = {};
    g.aseg[0] = a.y;
    g.a_stride = DFLASH_D;
    g.seg_w = DFLASH_D;
    g.b = a.w_head;
    g.M = M; g.N = (int)a.V; g.K = DFLASH_D;
    gemm_set_split(g, a.dtype, 1);
    if (a.dtype == DFLASH_BF16) g.out_bf16 = static_cast<uint16_t*>(a.logits);
    else g.part = static_cast<float*>(a.logits);

    HeadParams p;
    p.logits = a.logits; p.temp = a.temperature; p.B = a.B; p.V = a.V;
    p.seed = a.seed; p.offset = a.offset;
    p.part = static_cast<KeyIdx*>(ws);
    {
        const int64_t n = (a.V + 255) / 256;
        p.spart = reinterpret_cast<RowStat*>(static_cast<char*>(ws) +
                                             (((size_t)a.B * 7 * n * sizeof(KeyIdx) + 255) & ~(size_t)255));
    }
    p.d = a.draft_tokens;
    p.dstats = a.draft_stats;
    const int rows = a.B * 7;
    hipError_t e;
    if (fused_path(a)) {
        // 256 x 256 tiles (half the operand bytes per flop of 128 x 128),
        // keys computed in the epilogue from the rounded logits.
        HeadEpilogue ep;
        ep.temp = a.temperature; ep.seed = a.seed; ep.offset = a.offset;
        ep.part = p.part;
        ep.spart = a.draft_stats ? p.spart : nullptr;
        ep.nparts = (int)(a.V / 256);
        if ((e = launch_gemm_big_head(g, ep, s)) != hipSuccess) return e;
        p.nch = ep.nparts;
    } else {
        if ((e = launch_gemm(g, a.dtype, s)) != hipSuccess) return e;
        p.nch = (int)((a.V + kChunk - 1) / kChunk);
        if (a.dtype == DFLASH_BF16) draft_sample_kernel<uint16_t><<<rows * p.nch, kThreads, 0, s>>>(p);
        else draft_sample_kernel<float><<<rows * p.nch, kThreads, 0, s>>>(p);
    }
    draft_pick_kernel<<<(rows + 3) / 4, kThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
