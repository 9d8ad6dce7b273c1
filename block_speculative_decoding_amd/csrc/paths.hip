// DFlash2's top-m candidate path selector over the draft logits (gfx950).
//
// "DFlash & DFlash2: Block-Diffusion LLM-Speedup", section "DFlash2", item 2:
// the head yields the top-m candidates per block position, and a path is
// scored by the sum over positions of log P_draft(candidate) plus lambda
// times the entropy of P_draft there; the best paths go to the target.
// P_draft is softmax(z) of the stored logits of rows 1..7.  The drafter
// proposes the block in one forward, so a path's score separates per
// position and a beam of width P keeps exactly the top-P paths.
//
// Launch sequence:
//   path_stats  -- vocabulary-parallel, one workgroup per 8192-entry chunk of
//                  a row: chunk max M_c, S0 = sum e^(z - M_c),
//                  S1 = sum e^(z - M_c) (z - M_c), and the chunk's top-m
//                  (value, index) in order (larger logit first, ties to the
//                  lower index).  Only entries no later than the m-th best
//                  of the 256 thread maxima can be among them, so each
//                  thread keeps a sorted list of just those
//   path_select -- one workgroup per sequence: wave k merges row k's
//                  partials into M, Z = sum e^(z - M), the entropy
//                  log Z - S1 / Z and the top-m candidates with
//                  log p = z - M - log Z; then the beam over the seven
//                  positions, each step ranking the P x m extensions by
//                  counting (score first, then the candidate ranks as a
//                  base-8 code, first position most significant)
#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16384;           // vocabulary entries per stats workgroup (4096 per wave)
constexpr int kList = 8;                 // candidates kept per thread / chunk (m <= 8)
constexpr int kRows = 7;                 // proposal positions per sequence
constexpr int kSortMax = 512;            // P x m <= 64 x 8 extensions per beam step

struct ChunkPart {
    float mx, s0, s1, pad;
    float val[kList];
    int idx[kList];
};

struct PathParams {
    const void* logits;
    int64_t bstride, rstride, V;
    int B, m, P;
    float lam;
    int nch;
    ChunkPart* part;
    int32_t* cand_ids;
    float* cand_logp;
    float* entropy;
    int32_t* paths;
    float* scores;
};

// (v, i) comes before (v2, i2): larger value, equal values by lower index.
__device__ __forceinline__ bool before(float v, int i, float v2, int i2) {
    return v > v2 || (v == v2 && i < i2);
}

// Insert into a list of kList kept in order; the last entry drops out.
// Unrolled compare-exchange: every register index is static.
__device__ __forceinline__ void list_insert(float* lv, int* li, float v, int i) {
    if (!before(v, i, lv[kList - 1], li[kList - 1])) return;
#pragma unroll
    for (int s = 0; s < kList; ++s) {
        if (before(v, i, lv[s], li[s])) {
            const float tv = lv[s];
            const int ti = li[s];
            lv[s] = v;
            li[s] = i;
            v = tv;
            i = ti;
        }
    }
}

__device__ __forceinline__ void list_pop(float* lv, int* li) {
#pragma unroll
    for (int s = 0; s < kList - 1; ++s) {
        lv[s] = lv[s + 1];
        li[s] = li[s + 1];
    }
    lv[kList - 1] = -INFINITY;
    li[kList - 1] = 0x7FFFFFFF;
}

// Softmax statistics relative to a running maximum: (M, S0, S1) with
// S0 = sum e^(z - M) and S1 = sum e^(z - M) (z - M).
struct Stat { float m, s0, s1; };
__device__ __forceinline__ Stat stat_merge(Stat a, Stat b) {
    if (a.m == -INFINITY) return b;
    if (b.m == -INFINITY) return a;
    const float M = fmaxf(a.m, b.m);
    const float ea = expf(a.m - M), eb = expf(b.m - M);
    Stat r;
    r.m = M;
    r.s0 = a.s0 * ea + b.s0 * eb;
    r.s1 = (a.s1 + (a.m - M) * a.s0) * ea + (b.s1 + (b.m - M) * b.s0) * eb;
    return r;
}

// Wave-wide first entry in (value, index) order; every lane gets it.
__device__ __forceinline__ void wave_first(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o);
        const int i2 = __shfl_xor(i, o);
        if (before(v2, i2, v, i)) { v = v2; i = i2; }
    }
}

__device__ __forceinline__ Stat wave_stat(Stat s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Stat t;
        t.m = __shfl_xor(s.m, o);
        t.s0 = __shfl_xor(s.s0, o);
        t.s1 = __shfl_xor(s.s1, o);
        s = stat_merge(s, t);
    }
    return s;
}

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

template <typename T>
__global__ __launch_bounds__(kThreads) void path_stats_kernel(PathParams p) {
    constexpr int kWaves = kThreads / 64;
    __shared__ float s_v[kWaves][kList];
    __shared__ int s_i[kWaves][kList];
    __shared__ float s_st[kWaves][3];
    const int chunk = blockIdx.x % p.nch;
    const int row = blockIdx.x / p.nch;          // b * 7 + (k - 1)
    const int b = row / kRows, k = row % kRows + 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const T* z = static_cast<const T*>(p.logits) + (int64_t)b * p.bstride + (int64_t)k * p.rstride;
    constexpr int N = Vec<T>::N;
    constexpr int kSub = kChunk / kWaves;        // entries per wave
    constexpr int kIt = kSub / (64 * N);
    // V <= 2^24: entry indices fit in int.
    const int c1 = (int)min(p.V, (int64_t)chunk * kChunk + kChunk);
    const int w0 = chunk * kChunk + wave * kSub;
    float f[kIt][N];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int i0 = w0 + (it * 64 + lane) * N;
        if (i0 < c1) Vec<T>::load(z + i0, f[it]);
        else
#pragma unroll
            for (int e = 0; e < N; ++e) f[it][e] = -INFINITY;
    }
    // Lane maximum, then the threshold: the m-th largest of the 64 lane
    // maxima.  Those m values are entries of the wave's range, so its m best
    // entries all have values >= the threshold (equal values are ordered by
    // index inside the lists).
    float vm[kIt];                           // maximum of each loaded vector
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        vm[it] = f[it][0];
#pragma unroll
        for (int e = 1; e < N; ++e) vm[it] = fmaxf(vm[it], f[it][e]);
        mx = fmaxf(mx, vm[it]);
    }
    float tv = mx;
    {
        float ov = mx;
        int ol = lane;
        for (int r = 0; r < p.m; ++r) {
            float v = ov;
            int l = ol;
            wave_first(v, l);
            tv = v;
            if (l == lane) ov = -INFINITY;   // this lane's maximum is taken
        }
    }
    // Softmax sums relative to the lane maximum on the hardware exp2
    // (differences scaled by log2 e, clamped so that padding and masked
    // logits give exactly 0).
    constexpr float kLog2e = 1.4426950408889634f;
    const float ref = mx == -INFINITY ? 0.f : mx * kLog2e;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int it = 0; it < kIt; ++it)
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float d2 = fmaxf(fmaf(f[it][e], kLog2e, -ref), -200.f);
            const float ex = __builtin_amdgcn_exp2f(d2);
            s0 += ex;
            s1 = fmaf(ex, d2, s1);
        }
    Stat st = {mx, s0, s1 * (1.0f / kLog2e)};
    // Few vectors hold an entry that passes the threshold: re-read those (the
    // row is in L2) and insert their passing entries, so that the insertion
    // code appears N times rather than once per entry.  Padding past V is
    // never admitted.
    uint32_t vmask = 0;
#pragma unroll
    for (int it = 0; it < kIt; ++it)
        if (vm[it] >= tv) vmask |= 1u << it;
    float lv[kList];
    int li[kList];
#pragma unroll
    for (int s = 0; s < kList; ++s) { lv[s] = -INFINITY; li[s] = 0x7FFFFFFF; }
    while (vmask) {
        const int it = __builtin_ctz(vmask);
        vmask &= vmask - 1;
        const int i0 = w0 + (it * 64 + lane) * N;
        if (i0 >= c1) continue;
        float g[N];
        Vec<T>::load(z + i0, g);
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (g[e] >= tv) list_insert(lv, li, g[e], i0 + e);
    }
    st = wave_stat(st);
    for (int r = 0; r < p.m; ++r) {
        float v = lv[0];
        int i = li[0];
        wave_first(v, i);
        if (li[0] == i && lv[0] == v) list_pop(lv, li);
        if (lane == 0) { s_v[wave][r] = v; s_i[wave][r] = i; }
    }
    if (lane == 0) { s_st[wave][0] = st.m; s_st[wave][1] = st.s0; s_st[wave][2] = st.s1; }
    __syncthreads();
    if (wave != 0) return;
    // Wave 0 merges the four waves' lists and statistics.
    float v = -INFINITY;
    int i = 0x7FFFFFFF;
    if (lane < kWaves * p.m) { v = s_v[lane / p.m][lane % p.m]; i = s_i[lane / p.m][lane % p.m]; }
    ChunkPart* out = p.part + (int64_t)row * p.nch + chunk;
    for (int r = 0; r < p.m; ++r) {
        float fv = v;
        int fi = i;
        wave_first(fv, fi);
        if (i == fi && v == fv) { v = -INFINITY; i = 0x7FFFFFFF; }
        if (lane == 0) { out->val[r] = fv; out->idx[r] = fi; }
    }
    if (lane == 0) {
        Stat t = {s_st[0][0], s_st[0][1], s_st[0][2]};
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t = stat_merge(t, Stat{s_st[w][0], s_st[w][1], s_st[w][2]});
        out->mx = t.m;
        out->s0 = t.s0;
        out->s1 = t.s1;
    }
}

constexpr int kSelThreads = 512;   // wave k < 7 merges row k; all take part in the beam

__global__ __launch_bounds__(kSelThreads) void path_select_kernel(PathParams p) {
    __shared__ float s_lp[kRows][kList];
    __shared__ int s_id[kRows][kList];
    __shared__ float s_h[kRows];
    __shared__ float ps[kSortMax];
    __shared__ int pc[kSortMax];
    __shared__ float2 xe[kSortMax];
    __shared__ int rank[kSortMax];
    const int b = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = p.m;
    if (wave < kRows) {
        const int k = wave;
        const ChunkPart* part = p.part + ((int64_t)b * kRows + k) * p.nch;
        Stat st = {-INFINITY, 0.f, 0.f};
        float lv[kList];
        int li[kList];
#pragma unroll
        for (int s = 0; s < kList; ++s) { lv[s] = -INFINITY; li[s] = 0x7FFFFFFF; }
        for (int c = lane; c < p.nch; c += 64) {
            st = stat_merge(st, Stat{part[c].mx, part[c].s0, part[c].s1});
            for (int r = 0; r < m; ++r) list_insert(lv, li, part[c].val[r], part[c].idx[r]);
        }
        st = wave_stat(st);
        const float logz = logf(st.s0);
        for (int r = 0; r < m; ++r) {
            float v = lv[0];
            int i = li[0];
            wave_first(v, i);
            if (li[0] == i && lv[0] == v) list_pop(lv, li);
            if (lane == 0) {
                s_lp[k][r] = v - st.m - logz;
                s_id[k][r] = i;
            }
        }
        if (lane == 0) s_h[k] = logz - st.s1 / st.s0;
    }
    if (threadIdx.x == 0) { ps[0] = 0.f; pc[0] = 0; }
    __syncthreads();
    if (threadIdx.x < kRows * m) {
        const int k = threadIdx.x / m, r = threadIdx.x % m;
        p.cand_ids[((int64_t)b * kRows + k) * m + r] = s_id[k][r];
        p.cand_logp[((int64_t)b * kRows + k) * m + r] = s_lp[k][r];
    }
    if (threadIdx.x < kRows) p.entropy[(int64_t)b * kRows + threadIdx.x] = s_h[threadIdx.x];

    // Beam: the np prefixes live in ps / pc.  Each step builds the np x m
    // extensions in xe (score, code), gives each its rank among them by
    // counting the entries that come first (scores descending, then the rank
    // code ascending; codes are distinct, so ranks are too) -- the count of
    // entry e is split over `parts` threads and summed in LDS -- and keeps
    // ranks < P.
    int np = 1;
    for (int k = 0; k < kRows; ++k) {
        const int n = np * m;                  // <= 512 = kSelThreads
        const int parts = kSelThreads / n;
        if (threadIdx.x < n) {
            const int q = threadIdx.x / m, r = threadIdx.x % m;
            xe[threadIdx.x] = make_float2(ps[q] + s_lp[k][r], __int_as_float((pc[q] << 3) | r));
            rank[threadIdx.x] = 0;
        }
        __syncthreads();
        if (threadIdx.x < parts * n) {
            const int e = threadIdx.x % n, part = threadIdx.x / n;
            const float2 me = xe[e];
            const int mc = __float_as_int(me.y);
            const int q0 = part * n / parts, q1 = (part + 1) * n / parts;
            int cnt = 0;
            for (int q = q0; q < q1; ++q) {
                const float2 o = xe[q];
                cnt += before(o.x, __float_as_int(o.y), me.x, mc) ? 1 : 0;
            }
            atomicAdd(&rank[e], cnt);
        }
        __syncthreads();
        const int np2 = min(p.P, n);
        if (threadIdx.x < n && rank[threadIdx.x] < np2) {
            const float2 me = xe[threadIdx.x];
            ps[rank[threadIdx.x]] = me.x;
            pc[rank[threadIdx.x]] = __float_as_int(me.y);
        }
        np = np2;
        __syncthreads();
    }
    float hsum = 0.f;
#pragma unroll
    for (int k = 0; k < kRows; ++k) hsum += s_h[k];
    for (int e = threadIdx.x; e < p.P; e += kSelThreads) {
        p.scores[(int64_t)b * p.P + e] = ps[e] + p.lam * hsum;
#pragma unroll
        for (int k = 0; k < kRows; ++k)
            p.paths[((int64_t)b * p.P + e) * kRows + k] = s_id[k][(pc[e] >> (3 * (kRows - 1 - k))) & 7];
    }
}

}  // namespace

size_t paths_workspace_bytes(int B, int64_t V) {
    const int64_t nch = (V + kChunk - 1) / kChunk;
    return ((size_t)B * kRows * nch * sizeof(ChunkPart) + 255) & ~(size_t)255;
}

hipError_t launch_paths(const dflash_paths_args& a, void* ws, hipStream_t s) {
    PathParams p;
    p.logits = a.logits;
    p.bstride = a.batch_stride;
    p.rstride = a.row_stride;
    p.V = a.V;
    p.B = a.B; p.m = a.m; p.P = a.P;
    p.lam = a.lambda;
    p.nch = (int)((a.V + kChunk - 1) / kChunk);
    p.part = static_cast<ChunkPart*>(ws);
    p.cand_ids = a.cand_ids;
    p.cand_logp = a.cand_logp;
    p.entropy = a.entropy;
    p.paths = a.paths;
    p.scores = a.scores;
    const int grid = a.B * kRows * p.nch;
    if (a.dtype == DFLASH_BF16) path_stats_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
    else path_stats_kernel<float><<<grid, kThreads, 0, s>>>(p);
    path_select_kernel<<<a.B, kSelThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
