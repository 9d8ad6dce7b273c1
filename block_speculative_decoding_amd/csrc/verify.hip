// Exact speculative verification over logits rows (gfx950).
//
// Follows "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash",
// section "Why exact verification preserves the target" (accept with
// min(1, p/q), else draw from normalize(max(0, p - q)); greedy accepts while
// the proposal is the target argmax) and "DFlash & DFlash2", section 4.4.
//
// The work is HBM-bound streaming over [B, 8, V] target and [B, 7, V] draft
// logits.  Four launches, no host round trip:
//   1. stats     -- vocab-parallel, one pass over every row a sequence needs:
//                   raw max, sum of exp at 1/T, argmax (lowest index on ties).
//   2. decide    -- one wave per sequence: merge the chunk partials (fp64),
//                   run the sequential accept scan on Philox uniforms, emit
//                   accepted proposals (and the greedy correction/bonus).
//   3. sample    -- vocab-parallel Gumbel-max over the one row a sampled
//                   sequence still needs (residual max(0, p-q) or the bonus).
//   4. finalize  -- one wave per sequence: merge the Gumbel-max partials.
#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 15;            // 8 target rows + 7 draft rows per sequence
constexpr int64_t kStatsChunk = 32768;
constexpr int64_t kSampleChunk = 8192;

struct StatPart { float m; float s; int idx; int pad; };
struct SamplePart { float key; int idx; float keyp; int idxp; };
struct Desc { int mode; int k; int nacc; int pad; float mt, inv_st, mq, inv_sq; };

enum { MODE_DONE = 0, MODE_RESIDUAL = 1, MODE_BONUS = 2 };

struct Params {
    const void* target; int64_t tbs, trs;
    const void* draft; int64_t dbs, drs;
    const int32_t* dtok;
    const float* temp;
    int B; int64_t V;
    uint64_t seed, offset;
    int32_t* out_tokens; int32_t* out_len; unsigned long long* near_ties;
    int nch1, nch2;
    StatPart* stats; Desc* desc; SamplePart* samp;
};

// 16 bytes of logits widened to fp32.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float* p, float* f) {
        float4 w = *reinterpret_cast<const float4*>(p);
        f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w;
    }
};

// log2(e) / T split into two floats so that (z - m) * scale keeps ~fp64
// accuracy of the scale: x = fma(dz, hi, dz * lo).
struct Scale { float hi, lo; };
__device__ __forceinline__ Scale make_scale(float T) {
    double s = 1.4426950408889634 / (double)T;
    Scale r;
    r.hi = (float)s;
    r.lo = (float)(s - (double)r.hi);
    return r;
}
// -inf (an empty running max) maps to -inf; the split product alone would give
// -inf + inf = NaN whenever lo < 0.
__device__ __forceinline__ float scaled(float dz, Scale s) {
    return dz == -INFINITY ? -INFINITY : fmaf(dz, s.hi, dz * s.lo);
}

__device__ __forceinline__ bool is_greedy(float T) { return !(T > 0.f); }

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Params& p, int b, int r) {
    return r < 8 ? reinterpret_cast<const T*>(p.target) + b * p.tbs + r * p.trs
                 : reinterpret_cast<const T*>(p.draft) + b * p.dbs + (r - 8) * p.drs;
}

// (m, s) pairs of "sum of 2^((z - m) * scale)" combine.
__device__ __forceinline__ void combine_ms(float& m, float& s, float m2, float s2, Scale sc) {
    float M = fmaxf(m, m2);
    if (M == -INFINITY) { m = M; s = 0.f; return; }
    s = s * __builtin_amdgcn_exp2f(scaled(m - M, sc)) + s2 * __builtin_amdgcn_exp2f(scaled(m2 - M, sc));
    m = M;
}
// (value, index) argmax combine with lowest index on ties.
__device__ __forceinline__ void combine_arg(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// ---------------------------------------------------------------- stats
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_kernel(Params p) {
    const int row = blockIdx.x / p.nch1;
    const int chunk = blockIdx.x % p.nch1;
    const int b = row / kRows, r = row % kRows;
    const float Tb = p.temp[b];
    const bool greedy = is_greedy(Tb);
    if (greedy && r >= 8) return;  // greedy sequences never read draft rows
    const T* src = row_ptr<T>(p, b, r);
    const Scale sc = make_scale(greedy ? 1.f : Tb);
    constexpr int N = Vec<T>::N;
    constexpr int U = 4;  // 16-byte loads in flight per thread per step
    const int64_t c0 = (int64_t)chunk * kStatsChunk;
    const int64_t c1 = min(p.V, c0 + kStatsChunk);
    const int tid = threadIdx.x;

    float m = -INFINITY, s = 0.f;
    int am = 0x7FFFFFFF;
    for (int64_t base = c0; base < c1; base += (int64_t)kThreads * N * U) {
        float f[U][N];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            int64_t i = base + ((int64_t)j * kThreads + tid) * N;
            ok[j] = i < c1;
            if (ok[j]) Vec<T>::load(src + i, f[j]);
        }
        float lm = -INFINITY;
        int li = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (!ok[j]) continue;
            int64_t i = base + ((int64_t)j * kThreads + tid) * N;
#pragma unroll
            for (int e = 0; e < N; ++e)
                if (f[j][e] > lm) { lm = f[j][e]; li = (int)(i + e); }
        }
        if (greedy) {
            combine_arg(m, am, lm, li);
        } else {
            float M = fmaxf(m, lm);
            if (M == -INFINITY) continue;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (!ok[j]) continue;
#pragma unroll
                for (int e = 0; e < N; ++e) acc += __builtin_amdgcn_exp2f(scaled(f[j][e] - M, sc));
            }
            s = s * __builtin_amdgcn_exp2f(scaled(m - M, sc)) + acc;
            m = M;
        }
    }
    // wave reduction
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
        int a2 = __shfl_xor(am, o);
        if (greedy) combine_arg(m, am, m2, a2);
        else combine_ms(m, s, m2, s2, sc);
    }
    __shared__ float sm[kThreads / 64], ss[kThreads / 64];
    __shared__ int sa[kThreads / 64];
    const int w = tid >> 6;
    if ((tid & 63) == 0) { sm[w] = m; ss[w] = s; sa[w] = am; }
    __syncthreads();
    if (tid == 0) {
        for (int i = 1; i < kThreads / 64; ++i) {
            if (greedy) combine_arg(m, am, sm[i], sa[i]);
            else combine_ms(m, s, sm[i], ss[i], sc);
        }
        StatPart out;
        out.m = m; out.s = s; out.idx = am; out.pad = 0;
        p.stats[(int64_t)row * p.nch1 + chunk] = out;
    }
}

// ---------------------------------------------------------------- decide
// Merged row statistics: raw max M, sum S (double) of 2^((z - M) * scale), argmax.
struct RowStat { float m; double s; int idx; };

__device__ RowStat merge_row(const Params& p, int b, int r, double scale_d, bool greedy, int lane) {
    const StatPart* sp = p.stats + ((int64_t)b * kRows + r) * p.nch1;
    float m = -INFINITY;
    int am = 0x7FFFFFFF;
    for (int c = lane; c < p.nch1; c += 64) {
        float v = sp[c].m;
        if (greedy) combine_arg(m, am, v, sp[c].idx);
        else m = fmaxf(m, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o);
        int a2 = __shfl_xor(am, o);
        if (greedy) combine_arg(m, am, m2, a2);
        else m = fmaxf(m, m2);
    }
    double s = 0.0;
    if (!greedy) {
        for (int c = lane; c < p.nch1; c += 64) {
            float mc = sp[c].m;
            if (mc != -INFINITY) s += (double)sp[c].s * exp2((double)(mc - m) * scale_d);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    }
    RowStat rs;
    rs.m = m; rs.s = s; rs.idx = am;
    return rs;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void decide_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const float Tb = p.temp[b];
    const bool greedy = is_greedy(Tb);
    const double scale_d = greedy ? 1.0 : 1.4426950408889634 / (double)Tb;
    const int32_t* d = p.dtok + (int64_t)b * 7;
    int32_t* out = p.out_tokens + (int64_t)b * 8;

    if (greedy) {
        int amax[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) amax[r] = merge_row(p, b, r, 1.0, true, lane).idx;
        if (lane == 0) {
            int n = 0;
            while (n < 7 && d[n] == amax[n]) { out[n] = d[n]; ++n; }
            out[n] = amax[n];
            for (int j = n + 1; j < 8; ++j) out[j] = -1;
            p.out_len[b] = n + 1;
            Desc ds = {};
            ds.mode = MODE_DONE; ds.nacc = n;
            p.desc[b] = ds;
        }
        return;
    }

    RowStat st[8], sq[7];
#pragma unroll
    for (int r = 0; r < 8; ++r) st[r] = merge_row(p, b, r, scale_d, false, lane);
#pragma unroll
    for (int r = 0; r < 7; ++r) sq[r] = merge_row(p, b, 8 + r, scale_d, false, lane);
    if (lane != 0) return;

    const T* tgt = reinterpret_cast<const T*>(p.target) + b * p.tbs;
    const T* drf = reinterpret_cast<const T*>(p.draft) + b * p.dbs;
    int n = 0;
    int mode = MODE_BONUS;
    for (int k = 1; k <= 7; ++k) {
        const int x = d[k - 1];
        double rho = 0.0;
        if (x >= 0 && (int64_t)x < p.V) {
            float zt = Elem<T>::load(tgt + (k - 1) * p.trs, x);
            float zd = Elem<T>::load(drf + (k - 1) * p.drs, x);
            // ln2-free ratio in the log2 domain: p(x)/q(x) = 2^(dt - dq) * Sq / St
            double e = ((double)(zt - st[k - 1].m) - (double)(zd - sq[k - 1].m)) * scale_d;
            rho = exp2(e) * (sq[k - 1].s / st[k - 1].s);
        }
        U64x4 ctr = {0ull, 8ull * (uint64_t)b + (uint64_t)k, 0ull, p.offset};
        const float u = word_to_uniform(philox4x64_10(ctr, p.seed, 0ull).x0);
        if (fabs((double)u - rho) < 1e-6) atomicAdd(p.near_ties, 1ull);
        if ((double)u < rho) {
            out[n] = x;
            ++n;
        } else {
            mode = MODE_RESIDUAL;
            break;
        }
    }
    for (int j = n + 1; j < 8; ++j) out[j] = -1;
    p.out_len[b] = n + 1;
    Desc ds;
    ds.mode = mode;
    ds.nacc = n;
    ds.pad = 0;
    if (mode == MODE_RESIDUAL) {
        ds.k = n + 1;
        ds.mt = st[n].m; ds.inv_st = (float)(1.0 / st[n].s);
        ds.mq = sq[n].m; ds.inv_sq = (float)(1.0 / sq[n].s);
    } else {
        ds.k = 8;
        ds.mt = st[7].m; ds.inv_st = (float)(1.0 / st[7].s);
        ds.mq = 0.f; ds.inv_sq = 0.f;
    }
    p.desc[b] = ds;
}

// ---------------------------------------------------------------- sample
__device__ __forceinline__ float gumbel_from_word(uint64_t w) {
    const float u = word_to_uniform(w);
    return -logf(-logf(u));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sample_kernel(Params p) {
    const int b = blockIdx.x / p.nch2;
    const int chunk = blockIdx.x % p.nch2;
    const Desc ds = p.desc[b];
    if (ds.mode == MODE_DONE) return;
    const float Tb = p.temp[b];
    const Scale sc = make_scale(Tb);
    const int k = ds.k;
    const T* tr = reinterpret_cast<const T*>(p.target) + b * p.tbs + (k - 1) * p.trs;
    const T* dr = reinterpret_cast<const T*>(p.draft) + b * p.dbs + (k - 1) * p.drs;
    const bool resid = ds.mode == MODE_RESIDUAL;
    constexpr int N = Vec<T>::N;
    const int64_t c0 = (int64_t)chunk * kSampleChunk;
    const int64_t c1 = min(p.V, c0 + kSampleChunk);
    const uint64_t ctr1 = 8ull * (uint64_t)b + (uint64_t)k;

    float best = -INFINITY, bestp = -INFINITY;
    int bi = 0x7FFFFFFF, bip = 0x7FFFFFFF;
    for (int64_t i0 = c0 + (int64_t)threadIdx.x * N; i0 < c1; i0 += (int64_t)kThreads * N) {
        float zt[N], zq[N];
        Vec<T>::load(tr + i0, zt);
        if (resid) Vec<T>::load(dr + i0, zq);
        float g[N];
#pragma unroll
        for (int q4 = 0; q4 < N / 4; ++q4) {
            U64x4 c = {(uint64_t)(i0 / 4 + q4), ctr1, 1ull, p.offset};
            U64x4 w = philox4x64_10(c, p.seed, 0ull);
            g[4 * q4 + 0] = gumbel_from_word(w.x0);
            g[4 * q4 + 1] = gumbel_from_word(w.x1);
            g[4 * q4 + 2] = gumbel_from_word(w.x2);
            g[4 * q4 + 3] = gumbel_from_word(w.x3);
        }
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int idx = (int)(i0 + e);
            if (resid) {
                const float xt = scaled(zt[e] - ds.mt, sc);
                const float pv = __builtin_amdgcn_exp2f(xt) * ds.inv_st;
                const float qv = __builtin_amdgcn_exp2f(scaled(zq[e] - ds.mq, sc)) * ds.inv_sq;
                const float rr = pv - qv;
                if (rr > 0.f) combine_arg(best, bi, logf(rr) + g[e], idx);
                combine_arg(bestp, bip, xt * kLn2 + g[e], idx);
            } else {
                combine_arg(best, bi, zt[e] / Tb + g[e], idx);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        combine_arg(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
        combine_arg(bestp, bip, __shfl_xor(bestp, o), __shfl_xor(bip, o));
    }
    __shared__ SamplePart sw[kThreads / 64];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sw[w].key = best; sw[w].idx = bi; sw[w].keyp = bestp; sw[w].idxp = bip; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) {
            combine_arg(best, bi, sw[i].key, sw[i].idx);
            combine_arg(bestp, bip, sw[i].keyp, sw[i].idxp);
        }
        SamplePart o;
        o.key = best; o.idx = bi; o.keyp = bestp; o.idxp = bip;
        p.samp[(int64_t)b * p.nch2 + chunk] = o;
    }
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const Desc ds = p.desc[b];
    if (ds.mode == MODE_DONE) return;
    float best = -INFINITY, bestp = -INFINITY;
    int bi = 0x7FFFFFFF, bip = 0x7FFFFFFF;
    for (int c = lane; c < p.nch2; c += 64) {
        const SamplePart sp = p.samp[(int64_t)b * p.nch2 + c];
        combine_arg(best, bi, sp.key, sp.idx);
        combine_arg(bestp, bip, sp.keyp, sp.idxp);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        combine_arg(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
        combine_arg(bestp, bip, __shfl_xor(bestp, o), __shfl_xor(bip, o));
    }
    if (lane == 0) {
        const int tok = (best > -INFINITY) ? bi : bip;  // zero residual falls back to p
        p.out_tokens[(int64_t)b * 8 + ds.nacc] = tok;
    }
}

}  // namespace

size_t verify_workspace_bytes(int B, int64_t V) {
    const int64_t nch1 = (V + kStatsChunk - 1) / kStatsChunk;
    const int64_t nch2 = (V + kSampleChunk - 1) / kSampleChunk;
    size_t bytes = (size_t)B * kRows * nch1 * sizeof(StatPart);
    bytes = (bytes + 255) & ~(size_t)255;
    bytes += ((size_t)B * sizeof(Desc) + 255) & ~(size_t)255;
    bytes += (size_t)B * nch2 * sizeof(SamplePart);
    return bytes;
}

hipError_t launch_verify(const dflash_verify_args& a, void* ws, hipStream_t s) {
    Params p;
    p.target = a.target_logits; p.tbs = a.t_batch_stride; p.trs = a.t_row_stride;
    p.draft = a.draft_logits; p.dbs = a.d_batch_stride; p.drs = a.d_row_stride;
    p.dtok = a.draft_tokens; p.temp = a.temperature;
    p.B = a.B; p.V = a.V; p.seed = a.seed; p.offset = a.offset;
    p.out_tokens = a.out_tokens; p.out_len = a.out_len; p.near_ties = a.near_ties;
    p.nch1 = (int)((a.V + kStatsChunk - 1) / kStatsChunk);
    p.nch2 = (int)((a.V + kSampleChunk - 1) / kSampleChunk);
    char* w = static_cast<char*>(ws);
    size_t off = 0;
    p.stats = reinterpret_cast<StatPart*>(w + off);
    off += (size_t)a.B * kRows * p.nch1 * sizeof(StatPart);
    off = (off + 255) & ~(size_t)255;
    p.desc = reinterpret_cast<Desc*>(w + off);
    off += ((size_t)a.B * sizeof(Desc) + 255) & ~(size_t)255;
    p.samp = reinterpret_cast<SamplePart*>(w + off);

    const dim3 g1(p.nch1 * a.B * kRows), g2(p.nch2 * a.B), gw((a.B + 3) / 4);
    if (a.dtype == DFLASH_BF16) {
        stats_kernel<uint16_t><<<g1, kThreads, 0, s>>>(p);
        decide_kernel<uint16_t><<<gw, kThreads, 0, s>>>(p);
        sample_kernel<uint16_t><<<g2, kThreads, 0, s>>>(p);
    } else {
        stats_kernel<float><<<g1, kThreads, 0, s>>>(p);
        decide_kernel<float><<<gw, kThreads, 0, s>>>(p);
        sample_kernel<float><<<g2, kThreads, 0, s>>>(p);
    }
    finalize_kernel<<<gw, kThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
