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
//   path_stats  -- vocabulary-parallel, one workgroup per 32768-entry chunk of
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
//                  positions.  log p = z - lse per position, so paths differ
//                  only by the sum of their stored candidate logits: each
//                  step ranks the P x m extensions by counting, on that sum
//                  taken exactly (128-bit fixed point, see PathKey), then
//                  the candidate ranks as a base-8 code, first position most
//                  significant
#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32768;           // vocabulary entries per stats workgroup (8192 per wave; 16384: +4%, 8192: +23%)
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
    int nch;               // stats workgroups per row (kChunk entries each)
    int nsub;              // partials per row (one per wave: kChunk / 4 entries each)
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

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void first_step(float& v, int& i) {
    const float v2 = dpp_f<CTRL, ROWS>(v, -INFINITY);
    const int i2 = dpp_i<CTRL, ROWS>(i, 0x7FFFFFFF);
    if (before(v2, i2, v, i)) { v = v2; i = i2; }
}

// Lists of a compile-time length L, in order: insertion as one
// compare-and-select pass (no branches, so no copies of the list around
// them); an entry that comes after all L drops out.
template <int L>
__device__ __forceinline__ void insert_n(float* lv, int* li, float v, int i) {
#pragma unroll
    for (int s = 0; s < L; ++s) {
        const bool b = before(v, i, lv[s], li[s]);
        const float ov = lv[s];
        const int oi = li[s];
        lv[s] = b ? v : ov;
        li[s] = b ? i : oi;
        v = b ? ov : v;
        i = b ? oi : i;
    }
}

template <int L>
__device__ __forceinline__ void pop_n(float* lv, int* li) {
#pragma unroll
    for (int s = 0; s < L - 1; ++s) {
        lv[s] = lv[s + 1];
        li[s] = li[s + 1];
    }
    lv[L - 1] = -INFINITY;
    li[L - 1] = 0x7FFFFFFF;
}

// Wave-wide first entry in (value, index) order; every lane gets it.
__device__ __forceinline__ void wave_first(float& v, int& i) {
    first_step<kDppXor1>(v, i);
    first_step<kDppXor2>(v, i);
    first_step<kDppHalfMirror>(v, i);
    first_step<kDppMirror>(v, i);
    first_step<kDppBcast15, 0xA>(v, i);
    first_step<kDppBcast31, 0xC>(v, i);
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void stat_step(Stat& s) {
    Stat t;
    t.m = dpp_f<CTRL, ROWS>(s.m, -INFINITY);
    t.s0 = dpp_f<CTRL, ROWS>(s.s0, 0.f);
    t.s1 = dpp_f<CTRL, ROWS>(s.s1, 0.f);
    s = stat_merge(s, t);
}

__device__ __forceinline__ Stat wave_stat(Stat s) {
    stat_step<kDppXor1>(s);
    stat_step<kDppXor2>(s);
    stat_step<kDppHalfMirror>(s);
    stat_step<kDppMirror>(s);
    stat_step<kDppBcast15, 0xA>(s);
    stat_step<kDppBcast31, 0xC>(s);
    s.m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.m), 63));
    s.s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.s0), 63));
    s.s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.s1), 63));
    return s;
}

// Loaded vectors stay in their storage form (bf16: 8 values in 4 registers)
// and are unpacked in each pass: half the registers of fp32 copies, so
// more waves share a SIMD to cover the loads' latency.
// Wave-wide max / sum of one float, uniform result.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float max_step(float x) { return fmaxf(x, dpp_f<CTRL, ROWS>(x, -INFINITY)); }
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float sum_step(float x) { return x + dpp_f<CTRL, ROWS>(x, 0.f); }
__device__ __forceinline__ float wave_max_dpp(float x) {
    x = max_step<kDppXor1>(x); x = max_step<kDppXor2>(x); x = max_step<kDppHalfMirror>(x);
    x = max_step<kDppMirror>(x); x = max_step<kDppBcast15, 0xA>(x); x = max_step<kDppBcast31, 0xC>(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x = sum_step<kDppXor1>(x); x = sum_step<kDppXor2>(x); x = sum_step<kDppHalfMirror>(x);
    x = sum_step<kDppMirror>(x); x = sum_step<kDppBcast15, 0xA>(x); x = sum_step<kDppBcast31, 0xC>(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    using Raw = uint4;
    static __device__ __forceinline__ Raw load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
    static __device__ __forceinline__ Raw neg_inf() { return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
    static __device__ __forceinline__ void unpack(const Raw& w, float* f) {
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    using Raw = float4;
    static __device__ __forceinline__ Raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    static __device__ __forceinline__ Raw neg_inf() { return make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY); }
    static __device__ __forceinline__ void unpack(const Raw& w, float* f) { f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w; }
};

template <typename T, int M>     // M = m, the candidates kept
__global__ __launch_bounds__(kThreads) void path_stats_kernel(PathParams p) {
    // Each wave is independent: it covers kSub entries of a row and writes its
    // own partial (no LDS, no barrier); the select kernel merges them.
    constexpr int kWaves = kThreads / 64;
    const int chunk = blockIdx.x % p.nch;        // p.nch: workgroup chunks per row
    const int row = blockIdx.x / p.nch;          // b * 7 + (k - 1)
    const int b = row / kRows, k = row % kRows + 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const T* z = static_cast<const T*>(p.logits) + (int64_t)b * p.bstride + (int64_t)k * p.rstride;
    constexpr int N = Vec<T>::N;
    constexpr int kSub = kChunk / kWaves;        // entries per wave
    constexpr int kIt = kSub / (64 * N);
    // V <= 2^24: entry indices fit in int.
    const int w0 = chunk * kChunk + wave * kSub;
    if (w0 >= p.V) return;                       // past the row (the last chunk only)
    const int c1 = (int)min(p.V, (int64_t)w0 + kSub);
    typename Vec<T>::Raw raw[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int i0 = w0 + (it * 64 + lane) * N;
        raw[it] = i0 < c1 ? Vec<T>::load(z + i0) : Vec<T>::neg_inf();
    }
    float vm[kIt];                           // maximum of each loaded vector
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        float f[N];
        Vec<T>::unpack(raw[it], f);
        vm[it] = f[0];
#pragma unroll
        for (int e = 1; e < N; ++e) vm[it] = fmaxf(vm[it], f[e]);
        mx = fmaxf(mx, vm[it]);
    }
    // Threshold: after M rounds that each take the largest remaining lane
    // maximum (every lane holding it), tv is at most the M-th largest lane
    // maximum.  At least M entries of the wave's range are >= tv, so its M
    // best entries all are.
    float tv = mx;
    {
        float ov = mx;
#pragma unroll
        for (int r = 0; r < M; ++r) {
            tv = wave_max_dpp(ov);
            if (ov == tv) ov = -INFINITY;
        }
    }
    // Softmax sums relative to the lane maximum on the hardware exp2
    // (differences scaled by log2 e, clamped so that padding and masked
    // logits give exactly 0).
    const float ref = mx == -INFINITY ? 0.f : mx * kLog2e;
    // Opaque to the compiler: the unpacked copies of the maximum pass are not
    // kept alive until here (they would double the registers).
#pragma unroll
    for (int it = 0; it < kIt; ++it)
        asm volatile("" : "+v"(raw[it].x), "+v"(raw[it].y), "+v"(raw[it].z), "+v"(raw[it].w));
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        float f[N];
        Vec<T>::unpack(raw[it], f);
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float d2 = fmaxf(fmaf(f[e], kLog2e, -ref), -200.f);
            const float ex = __builtin_amdgcn_exp2f(d2);
            s0 += ex;
            s1 = fmaf(ex, d2, s1);
        }
    }
    // The wave's statistics: rescale every lane's sums to the wave maximum,
    // then add them up.
    const float wm = wave_max_dpp(mx);
    {
        const float dm = mx == -INFINITY ? 0.f : (mx - wm) * kLog2e;   // <= 0, in log2 units
        const float sc = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(dm);
        s1 = (s1 + dm * s0) * sc;                                       // still in log2 units
        s0 *= sc;
    }
    s0 = wave_sum_dpp(s0);
    s1 = wave_sum_dpp(s1);
    // Few vectors hold an entry that passes the threshold: re-read those (the
    // row is in L2) and insert their passing entries.  Padding past V is
    // never admitted.
    uint32_t vmask = 0;
#pragma unroll
    for (int it = 0; it < kIt; ++it)
        if (vm[it] >= tv) vmask |= 1u << it;
    float lv[M];
    int li[M];
#pragma unroll
    for (int s = 0; s < M; ++s) { lv[s] = -INFINITY; li[s] = 0x7FFFFFFF; }
    while (vmask) {
        const int it = __builtin_ctz(vmask);
        vmask &= vmask - 1;
        const int i0 = w0 + (it * 64 + lane) * N;
        if (i0 >= c1) continue;
        float g[N];
        Vec<T>::unpack(Vec<T>::load(z + i0), g);
#pragma unroll
        for (int e = 0; e < N; ++e) insert_n<M>(lv, li, g[e] >= tv ? g[e] : -INFINITY, g[e] >= tv ? i0 + e : 0x7FFFFFFF);
    }
    ChunkPart* out = p.part + (int64_t)row * p.nsub + chunk * kWaves + wave;
#pragma unroll
    for (int r = 0; r < M; ++r) {
        float v = lv[0];
        int i = li[0];
        wave_first(v, i);
        if (li[0] == i && lv[0] == v) pop_n<M>(lv, li);
        if (lane == 0) { out->val[r] = v; out->idx[r] = i; }
    }
    if (lane == 0) { out->mx = wm; out->s0 = s0; out->s1 = s1 * (1.0f / kLog2e); }
}

constexpr int kSelThreads = 512;   // wave k < 7 merges row k; all take part in the beam

// Exact order of (partial) paths.  A stored logit v = Mv * 2^ev with Mv an
// integer; at a per-sequence unit 2^e0 (the finest lowest set bit among the
// sequence's finite candidates) every candidate is the integer Mv << (ev - e0)
// and a path's sum of candidates is an exact 128-bit integer, as long as the
// candidates span at most 2^123 (largest magnitude over finest unit; beyond
// that e0 is raised and the finest bits are dropped, rounding toward -inf).
// A -inf candidate is counted instead of summed: paths order by fewer -inf
// candidates, then the larger sum, then the smaller rank code -- an order
// that stays additive over positions, so the beam keeps the exact top P.
struct PathKey {
    __int128 sum;
    int ninf;
    int code;
    int pad[2];
};

__device__ __forceinline__ bool key_before(const PathKey& a, const PathKey& b) {
    if (a.ninf != b.ninf) return a.ninf < b.ninf;
    if (a.sum != b.sum) return a.sum > b.sum;
    return a.code < b.code;
}

// |v| = mag * 2^e with mag odd (or 0).  +inf and NaN fall outside the
// supported domain; they decompose to some finite pair (no fault).
__device__ __forceinline__ void split_float(float v, uint32_t& mag, int& e, bool& neg) {
    const uint32_t u = __float_as_uint(v);
    const int ex = (int)((u >> 23) & 0xFFu);
    mag = u & 0x7FFFFFu;
    e = -149;
    if (ex != 0) { mag |= 0x800000u; e = ex - 150; }
    neg = (u >> 31) != 0;
    if (mag != 0) {
        const int tz = __builtin_ctz(mag);
        mag >>= tz;
        e += tz;
    }
}

__device__ __forceinline__ double i128_to_double(__int128 x) {
    const bool neg = x < 0;
    const unsigned __int128 ux = neg ? (unsigned __int128)0 - (unsigned __int128)x : (unsigned __int128)x;
    const double d = (double)(uint64_t)(ux >> 64) * 18446744073709551616.0 + (double)(uint64_t)ux;
    return neg ? -d : d;
}

__global__ __launch_bounds__(kSelThreads) void path_select_kernel(PathParams p) {
    __shared__ float s_lp[kRows][kList];
    __shared__ float s_v[kRows][kList];
    __shared__ int s_id[kRows][kList];
    __shared__ float s_h[kRows];
    __shared__ float s_lse[kRows];
    __shared__ __int128 s_key[kRows][kList];
    __shared__ int s_inf[kRows][kList];
    __shared__ int s_e0;
    __shared__ PathKey ps[64];
    __shared__ PathKey xe[kSortMax];
    __shared__ int rank[kSortMax];
    const int b = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = p.m;
    if (wave < kRows) {
        const int k = wave;
        const ChunkPart* part = p.part + ((int64_t)b * kRows + k) * p.nsub;
        Stat st = {-INFINITY, 0.f, 0.f};
        float lv[kList];
        int li[kList];
#pragma unroll
        for (int s = 0; s < kList; ++s) { lv[s] = -INFINITY; li[s] = 0x7FFFFFFF; }
        for (int c = lane; c < p.nsub; c += 64) {
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
                s_v[k][r] = v;
                s_id[k][r] = i;
            }
        }
        if (lane == 0) {
            s_h[k] = logz - st.s1 / st.s0;
            s_lse[k] = st.m + logz;
        }
    }
    __syncthreads();
    // The sequence's unit: finest lowest set bit, raised if the candidates
    // would need more than 126 bits for a sum of seven.
    if (wave == 0) {
        int lo = 0x7FFFFFFF, hi = -0x7FFFFFFF;
        if (lane < kRows * m) {
            const float v = s_v[lane / m][lane % m];
            uint32_t mag;
            int e;
            bool neg;
            split_float(v, mag, e, neg);
            if (v != -INFINITY && mag != 0) {
                lo = e;
                hi = e + 32 - __builtin_clz(mag);    // 2^hi > |v|
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            lo = min(lo, __shfl_xor(lo, o));
            hi = max(hi, __shfl_xor(hi, o));
        }
        if (lane == 0) s_e0 = hi == -0x7FFFFFFF ? 0 : max(lo, hi + 3 - 126);
    }
    __syncthreads();
    if (threadIdx.x < kRows * m) {
        const int k = threadIdx.x / m, r = threadIdx.x % m;
        const float v = s_v[k][r];
        uint32_t mag;
        int e;
        bool neg;
        split_float(v, mag, e, neg);
        const int sh = e - s_e0;
        __int128 key = 0;
        if (mag != 0) {
            if (sh >= 0) key = (__int128)mag << sh;
            else if (sh > -32) key = (__int128)(mag >> -sh);
            if (neg) key = -key;
            if (neg && sh < 0 && (sh <= -32 || (mag & ((1u << -sh) - 1u)) != 0)) key -= 1;   // toward -inf
        }
        s_key[k][r] = key;
        s_inf[k][r] = v == -INFINITY;
        p.cand_ids[((int64_t)b * kRows + k) * m + r] = s_id[k][r];
        p.cand_logp[((int64_t)b * kRows + k) * m + r] = s_lp[k][r];
    }
    if (threadIdx.x < kRows) p.entropy[(int64_t)b * kRows + threadIdx.x] = s_h[threadIdx.x];
    if (threadIdx.x == 0) {
        PathKey z;
        z.sum = 0; z.ninf = 0; z.code = 0; z.pad[0] = z.pad[1] = 0;
        ps[0] = z;
    }
    __syncthreads();

    // Beam: the np prefixes live in ps.  Each step builds the np x m
    // extensions in xe, gives each its rank among them by counting the
    // entries that come first (codes are distinct, so ranks are too) -- the
    // count of entry e is split over `parts` threads and summed in LDS -- and
    // keeps ranks < P.
    int np = 1;
    for (int k = 0; k < kRows; ++k) {
        const int n = np * m;                  // <= 512 = kSelThreads
        const int parts = kSelThreads / n;
        if (threadIdx.x < n) {
            const int q = threadIdx.x / m, r = threadIdx.x % m;
            PathKey x;
            x.sum = ps[q].sum + s_key[k][r];
            x.ninf = ps[q].ninf + s_inf[k][r];
            x.code = (ps[q].code << 3) | r;
            x.pad[0] = x.pad[1] = 0;
            xe[threadIdx.x] = x;
            rank[threadIdx.x] = 0;
        }
        __syncthreads();
        if (threadIdx.x < parts * n) {
            const int e = threadIdx.x % n, part = threadIdx.x / n;
            const PathKey me = xe[e];
            const int q0 = part * n / parts, q1 = (part + 1) * n / parts;
            int cnt = 0;
            for (int q = q0; q < q1; ++q) cnt += key_before(xe[q], me) ? 1 : 0;
            atomicAdd(&rank[e], cnt);
        }
        __syncthreads();
        const int np2 = min(p.P, n);
        if (threadIdx.x < n && rank[threadIdx.x] < np2) ps[rank[threadIdx.x]] = xe[threadIdx.x];
        np = np2;
        __syncthreads();
    }
    // score = sum of candidates - sum of lse + lambda * sum of entropies
    double shift = 0.0;
    float hsum = 0.f;
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
        shift -= (double)s_lse[k];
        hsum += s_h[k];
    }
    shift += (double)p.lam * (double)hsum;
    for (int e = threadIdx.x; e < p.P; e += kSelThreads) {
        const PathKey x = ps[e];
        p.scores[(int64_t)b * p.P + e] =
            x.ninf ? -INFINITY : (float)(ldexp(i128_to_double(x.sum), s_e0) + shift);
#pragma unroll
        for (int k = 0; k < kRows; ++k)
            p.paths[((int64_t)b * p.P + e) * kRows + k] = s_id[k][(x.code >> (3 * (kRows - 1 - k))) & 7];
    }
}

}  // namespace

constexpr int kSubEntries = kChunk / (kThreads / 64);

size_t paths_workspace_bytes(int B, int64_t V) {
    const int64_t nsub = (V + kSubEntries - 1) / kSubEntries;
    return ((size_t)B * kRows * nsub * sizeof(ChunkPart) + 255) & ~(size_t)255;
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
    p.nsub = (int)((a.V + kSubEntries - 1) / kSubEntries);
    p.part = static_cast<ChunkPart*>(ws);
    p.cand_ids = a.cand_ids;
    p.cand_logp = a.cand_logp;
    p.entropy = a.entropy;
    p.paths = a.paths;
    p.scores = a.scores;
    const int grid = a.B * kRows * p.nch;
    const bool bf = a.dtype == DFLASH_BF16;
    switch (a.m) {
#define DFLASH_PATHS_M(MM)                                                                     \
    case MM:                                                                                   \
        if (bf) path_stats_kernel<uint16_t, MM><<<grid, kThreads, 0, s>>>(p);                  \
        else path_stats_kernel<float, MM><<<grid, kThreads, 0, s>>>(p);                        \
        break;
        DFLASH_PATHS_M(1) DFLASH_PATHS_M(2) DFLASH_PATHS_M(3) DFLASH_PATHS_M(4)
        DFLASH_PATHS_M(5) DFLASH_PATHS_M(6) DFLASH_PATHS_M(7) DFLASH_PATHS_M(8)
#undef DFLASH_PATHS_M
        default: return hipErrorInvalidValue;
    }
    path_select_kernel<<<a.B, kSelThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
