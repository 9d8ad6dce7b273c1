// Shared LM head over the block rows and the draft proposals (gfx950).
//
// "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash", sections
// "The parameter count exposes the real cost" (the drafter's output head is a
// copy of the target head, [262144, 2560]) and "The released serving cycle"
// (one forward over the eight block positions proposes all seven future
// tokens); "DFlash & DFlash2", section 4.2 (the target's unembedding head
// maps the output states to vocabulary logits).
//
// Launch sequence:
//   gemm    -- logits [8B][V] = y [8B][2560] . W_head^T, written in the
//              storage type (bf16: the 256 x 256-tile kernel from 256 rows
//              on, else the 128 x 128 kernel with one split; both with a
//              direct bf16 output; or the fp32 kernel)
//   sample  -- vocab-parallel over rows k = 1..7 of each sequence: greedy rows
//              keep (max, lowest argmax); sampled rows the Gumbel-max key
//              z / T - ln(-ln u) with u from stream 2 of the uniform layout,
//              one Philox4x64-10 block per 8 entries
//   pick    -- one wave per row: merge the chunk partials into d_k
// Sampling reads the stored logits, so the proposals are those of the values
// verification will read.
#include "device_common.h"
#include "gemm.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = 8192;       // vocabulary entries per sampling workgroup
constexpr uint64_t kDraftStream = 2;   // uniform stream of draft sampling

struct KeyPart { float key; int idx; };

struct HeadParams {
    const void* logits;   // [B][8][V]
    const float* temp;    // [B]
    int B;
    int64_t V;
    uint64_t seed, offset;
    int nch;
    KeyPart* part;        // [B][7][nch]
    int32_t* d;           // [B][7]
};

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float* p, float* f) {
        const float4 w = *reinterpret_cast<const float4*>(p);
        f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w;
    }
};

// Larger key wins; equal keys go to the lower index.
__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void draft_sample_kernel(HeadParams p) {
    const int chunk = blockIdx.x % p.nch;
    const int row = blockIdx.x / p.nch;       // b * 7 + (k - 1)
    const int b = row / 7, k = row % 7 + 1;
    const float Tb = p.temp[b];
    const bool greedy = !(Tb > 0.f);
    const float invT = greedy ? 1.f : 1.0f / Tb;
    const T* z = static_cast<const T*>(p.logits) + ((int64_t)b * 8 + k) * p.V;
    constexpr int N = Vec<T>::N;
    const int64_t c0 = (int64_t)chunk * kChunk, c1 = min(p.V, c0 + kChunk);
    const uint64_t ctr1 = 8ull * (uint64_t)b + (uint64_t)k;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    // Every load of the thread is issued before any is used.
    constexpr int kIt = kChunk / (kThreads * N);
    float f[kIt][N];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + threadIdx.x) * N;
        if (i0 < c1) Vec<T>::load(z + i0, f[it]);
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + threadIdx.x) * N;
        if (i0 >= c1) continue;
        if (greedy) {
#pragma unroll
            for (int e = 0; e < N; ++e) better(best, bi, f[it][e], (int)(i0 + e));
            continue;
        }
        // Entry j of an 8-entry group uses half j % 2 of word j / 2 of the
        // group's Philox block (counter (i / 8, 8b + k, 2, offset)).
        const U64x4 c = {(uint64_t)(i0 >> 3), ctr1, kDraftStream, p.offset};
        const U64x4 r = philox4x64_10(c, p.seed, 0ull);
        const uint64_t words[4] = {r.x0, r.x1, r.x2, r.x3};
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int j = (int)((i0 + e) & 7);
            const uint64_t wd = words[j >> 1];
            const float u = (j & 1) ? word_to_uniform_lo(wd) : word_to_uniform(wd);
            better(best, bi, f[it][e] * invT - fast_ln(-fast_ln(u)), (int)(i0 + e));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) better(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
    __shared__ KeyPart sw[kThreads / 64];
    if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = {best, bi};
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) better(best, bi, sw[w].key, sw[w].idx);
        p.part[(int64_t)row * p.nch + chunk] = {best, bi};
    }
}

// One wave per (sequence, proposal): the chunk partials' best key.
__global__ __launch_bounds__(kThreads) void draft_pick_kernel(HeadParams p) {
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= p.B * 7) return;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = lane; c < p.nch; c += 64) better(best, bi, p.part[(int64_t)row * p.nch + c].key,
                                                     p.part[(int64_t)row * p.nch + c].idx);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) better(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
    if (lane == 0) p.d[row] = bi == 0x7FFFFFFF ? -1 : bi;   // no finite key (non-finite logits): -1
}

}  // namespace

size_t head_workspace_bytes(int B, int64_t V) {
    const int64_t nch = (V + kChunk - 1) / kChunk;
    return ((size_t)B * 7 * nch * sizeof(KeyPart) + 255) & ~(size_t)255;
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
    // 256 x 256 tiles once there are 256 rows: half the operand traffic per
    // flop of the 128 x 128 kernel.
    const bool big = a.dtype == DFLASH_BF16 && M >= 256 && a.V % 256 == 0;
    hipError_t e = big ? launch_gemm_big(g, s) : launch_gemm(g, a.dtype, s);
    if (e != hipSuccess) return e;

    HeadParams p;
    p.logits = a.logits; p.temp = a.temperature; p.B = a.B; p.V = a.V;
    p.seed = a.seed; p.offset = a.offset;
    p.nch = (int)((a.V + kChunk - 1) / kChunk);
    p.part = static_cast<KeyPart*>(ws);
    p.d = a.draft_tokens;
    const int rows = a.B * 7;
    if (a.dtype == DFLASH_BF16) draft_sample_kernel<uint16_t><<<rows * p.nch, kThreads, 0, s>>>(p);
    else draft_sample_kernel<float><<<rows * p.nch, kThreads, 0, s>>>(p);
    draft_pick_kernel<<<(rows + 3) / 4, kThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
