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
//                   raw max, sum of exp at 1/T, argmax (lowest index on ties);
//                   the draft rows' (max, sum) may come precomputed from the
//                   shared head instead (draft_stats), and are then not read.
//   2. decide    -- one wave per sequence: merge the chunk partials (fp64),
//                   run the sequential accept scan on Philox uniforms, emit
//                   accepted proposals (and the greedy correction/bonus).
//   3. sample    -- vocab-parallel Gumbel-max over the one row a sampled
//                   sequence still needs (residual max(0, p-q) or the bonus).
//   4. finalize  -- one wave per sequence: merge the Gumbel-max partials.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 15;            // 8 target rows + 7 draft rows per sequence
constexpr int64_t kStatsChunk = 32768;
constexpr int64_t kSampleChunk = 4096;   // draw chunk: 4096 entries (two Philox blocks per thread) beat 2048 and 8192 at B = 64 and 256

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
    int nrows;            // rows per sequence in the statistics grid: 15, or 8 with draft_stats
    const float* dstats;  // optional [B][7][2] (m, s) of the draft rows
    StatPart* stats; Desc* desc; SamplePart* samp;
};

// 16 bytes of logits widened to fp32 (streamed: nontemporal loads).
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
        const uint4 w = ld_stream(reinterpret_cast<const uint4*>(p));
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float* p, float* f) {
        const uint4 w = ld_stream(reinterpret_cast<const uint4*>(p));
        f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y); f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
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
// One chunk of one row.  Greedy rows keep (max, lowest argmax); sampled rows
// keep (max, sum of 2^((z - m) * scale)) and no argmax.  In the sampled
// loop the exponent is fma(z, hi, c_hi) + c_lo with (c_hi, c_lo) = -M * hi
// split exactly (M * hi has at most 48 significant bits), so the only
// systematic error is hi's own rounding (2^-25 relative, times the exponent).
template <typename T, bool GREEDY>
__device__ __forceinline__ void stats_chunk(const T* src, int64_t c0, int64_t c1, Scale sc, float& m, float& s,
                                            int& am) {
    constexpr int N = Vec<T>::N;
    constexpr int U = 4;  // 16-byte loads in flight per thread per step
    const int tid = threadIdx.x;
    for (int64_t base = c0; base < c1; base += (int64_t)kThreads * N * U) {
        float f[U][N];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t i = base + ((int64_t)j * kThreads + tid) * N;
            if (i < c1) {
                Vec<T>::load(src + i, f[j]);
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) f[j][e] = -INFINITY;
            }
        }
        if (GREEDY) {
            float lm = -INFINITY;
            int li = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int i = (int)(base + ((int64_t)j * kThreads + tid) * N);
#pragma unroll
                for (int e = 0; e < N; ++e)
                    if (f[j][e] > lm) { lm = f[j][e]; li = i + e; }
            }
            combine_arg(m, am, lm, li);
        } else {
            float lm = -INFINITY;
#pragma unroll
            for (int j = 0; j < U; ++j)
#pragma unroll
                for (int e = 0; e < N; ++e) lm = fmaxf(lm, f[j][e]);
            const float M = fmaxf(m, lm);
            if (M == -INFINITY) continue;
            const double cm = -(double)M * (double)sc.hi;
            const float c_hi = (float)cm, c_lo = (float)(cm - (double)c_hi);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < U; ++j)
#pragma unroll
                for (int e = 0; e < N; ++e) acc += __builtin_amdgcn_exp2f(fmaf(f[j][e], sc.hi, c_hi) + c_lo);
            s = s * __builtin_amdgcn_exp2f(scaled(m - M, sc)) + acc;
            m = M;
        }
    }
}

// Rows a sequence needs: greedy, target rows 0..7 (argmax); sampled, target
// rows 0..6 and draft rows 0..6 (the bonus draw at row 7 is a Gumbel-max over
// unnormalised logits and needs no statistics).
// With draft_stats the grid covers target rows only (p.nrows = 8).
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_kernel(Params p) {
    const int row = blockIdx.x / p.nch1;
    const int chunk = blockIdx.x % p.nch1;
    const int b = row / p.nrows, r = row % p.nrows;
    const float Tb = p.temp[b];
    const bool greedy = is_greedy(Tb);
    if (greedy ? r >= 8 : r == 7) return;
    const T* src = row_ptr<T>(p, b, r);
    const Scale sc = make_scale(greedy ? 1.f : Tb);
    const int64_t c0 = (int64_t)chunk * kStatsChunk;
    const int64_t c1 = min(p.V, c0 + kStatsChunk);
    const int tid = threadIdx.x;

    float m = -INFINITY, s = 0.f;
    int am = 0x7FFFFFFF;
    if (greedy) stats_chunk<T, true>(src, c0, c1, sc, m, s, am);
    else stats_chunk<T, false>(src, c0, c1, sc, m, s, am);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
        const int a2 = __shfl_xor(am, o);
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
        p.stats[((int64_t)b * kRows + r) * p.nch1 + chunk] = out;
    }
}

// ---------------------------------------------------------------- decide
// One 256-thread block per sequence.  16 lanes merge the chunk partials of
// each row; lanes k-1 (k = 1..7) evaluate decision k in parallel (ratio in
// fp64 from the merged statistics, Philox uniform); thread 0 takes the
// longest accepted prefix.
template <typename T>
__global__ __launch_bounds__(kThreads) void decide_kernel(Params p) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const float Tb = p.temp[b];
    const bool greedy = is_greedy(Tb);
    const double scale_d = greedy ? 1.0 : 1.4426950408889634 / (double)Tb;
    const int nrows = greedy ? 8 : kRows;

    __shared__ float s_m[16];
    __shared__ double s_s[16];
    __shared__ int s_i[16];
    __shared__ double s_rho[8];
    __shared__ float s_u[8];
    __shared__ int s_acc[8];

    {
        const int r = tid >> 4, c0 = tid & 15;
        float m = -INFINITY;
        int am = 0x7FFFFFFF;
        const StatPart* sp = p.stats + ((int64_t)b * kRows + min(r, kRows - 1)) * p.nch1;
        const bool given = !greedy && r >= 8 && r < kRows && p.dstats != nullptr;   // from draft_stats
        const bool used = r < nrows && (greedy || r != 7) && !given;
        if (used)
            for (int c = c0; c < p.nch1; c += 16) {
                if (greedy) combine_arg(m, am, sp[c].m, sp[c].idx);
                else m = fmaxf(m, sp[c].m);
            }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            const float m2 = __shfl_xor(m, o);
            const int a2 = __shfl_xor(am, o);
            if (greedy) combine_arg(m, am, m2, a2);
            else m = fmaxf(m, m2);
        }
        double sum = 0.0;
        if (!greedy && used)
            for (int c = c0; c < p.nch1; c += 16) {
                const float mc = sp[c].m;
                if (mc != -INFINITY) sum += (double)sp[c].s * exp2((double)(mc - m) * scale_d);
            }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        if (given) {
            m = p.dstats[((int64_t)b * 7 + (r - 8)) * 2];
            sum = (double)p.dstats[((int64_t)b * 7 + (r - 8)) * 2 + 1];
        }
        if (c0 == 0) { s_m[r] = m; s_s[r] = sum; s_i[r] = am; }
    }
    __syncthreads();

    const int32_t* d = p.dtok + (int64_t)b * 7;
    if (tid < 7) {
        const int k = tid + 1;
        const int x = d[k - 1];
        if (greedy) {
            s_acc[tid] = x == s_i[k - 1];
        } else {
            double rho = 0.0;
            if (x >= 0 && (int64_t)x < p.V) {
                const T* tgt = reinterpret_cast<const T*>(p.target) + b * p.tbs + (k - 1) * p.trs;
                const T* drf = reinterpret_cast<const T*>(p.draft) + b * p.dbs + (k - 1) * p.drs;
                const float zt = Elem<T>::load(tgt, x), zd = Elem<T>::load(drf, x);
                // p(x)/q(x) = 2^((zt - Mt) - (zd - Mq)) * scale * Sq / St
                const double e = ((double)(zt - s_m[k - 1]) - (double)(zd - s_m[8 + k - 1])) * scale_d;
                rho = exp2(e) * (s_s[8 + k - 1] / s_s[k - 1]);
            }
            U64x4 ctr = {0ull, 8ull * (uint64_t)b + (uint64_t)k, 0ull, p.offset};
            const float u = word_to_uniform(philox4x64_10(ctr, p.seed, 0ull).x0);
            s_rho[tid] = rho;
            s_u[tid] = u;
            s_acc[tid] = (double)u < rho;
        }
    }
    __syncthreads();
    if (tid != 0) return;

    int32_t* out = p.out_tokens + (int64_t)b * 8;
    int n = 0;
    while (n < 7 && s_acc[n]) { out[n] = d[n]; ++n; }
    for (int j = n + 1; j < 8; ++j) out[j] = -1;
    p.out_len[b] = n + 1;
    Desc ds = {};
    ds.nacc = n;
    if (greedy) {
        out[n] = s_i[n];  // correction (row n) or bonus (row 7): the target argmax
        ds.mode = MODE_DONE;
        p.desc[b] = ds;
        return;
    }
    // Near-ties among the decisions actually taken (k = 1 .. min(n + 1, 7)).
    unsigned long long nt = 0;
    for (int k = 1; k <= min(n + 1, 7); ++k)
        if (fabs((double)s_u[k - 1] - s_rho[k - 1]) < 1e-6) ++nt;
    if (nt) atomicAdd(p.near_ties, nt);
    if (n < 7) {
        ds.mode = MODE_RESIDUAL;
        ds.k = n + 1;
        ds.mt = s_m[n]; ds.inv_st = (float)(1.0 / s_s[n]);
        ds.mq = s_m[8 + n]; ds.inv_sq = (float)(1.0 / s_s[8 + n]);
    } else {
        ds.mode = MODE_BONUS;  // row 7 has no statistics: the draw needs none
        ds.k = 8;
    }
    p.desc[b] = ds;
}

// ---------------------------------------------------------------- sample

// Gumbel noise of the 23-bit uniforms lies in [kGmin, kGmax] (u in
// [2^-24, 1 - 2^-24]); the bounds are widened a little for fp32 rounding.
constexpr float kGmax = 16.75f;   // -ln(-ln(1 - 2^-24)) = 16.636
constexpr float kGmin = -2.85f;   // -ln(-ln(2^-24))     = -2.812

// Gumbel-max over one chunk of the row a sampled sequence still needs.  Pass 1
// (no random numbers) finds the chunk's largest log-weight L; the chunk's
// winner then has key >= L + kGmin, so an entry whose log-weight plus kGmax
// falls below that can never win and its Philox block is skipped.  The
// result is exactly the Gumbel-max argmax; only the work depends on the data.
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
    const float invT = 1.0f / Tb;
    constexpr int N = Vec<T>::N;
    constexpr int IT = kSampleChunk / (kThreads * N);  // vectors per thread
    const int64_t c0 = (int64_t)chunk * kSampleChunk;
    const uint64_t ctr1 = 8ull * (uint64_t)b + (uint64_t)k;
    const int tid = threadIdx.x;

    // Pass 1: log-weights.  w = ln r (residual; -inf where r <= 0), the fallback
    // wp = ln p up to a constant, or z / T for the bonus draw.
    float w[IT][N], wp[IT][N];
    float lmax = -INFINITY, lpmax = -INFINITY;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + tid) * N;
        if (i0 >= p.V) {
#pragma unroll
            for (int e = 0; e < N; ++e) { w[it][e] = -INFINITY; wp[it][e] = -INFINITY; }
            continue;
        }
        float zt[N], zq[N];
        Vec<T>::load(tr + i0, zt);
        if (resid) Vec<T>::load(dr + i0, zq);
#pragma unroll
        for (int e = 0; e < N; ++e) {
            if (resid) {
                const float xt = scaled(zt[e] - ds.mt, sc);
                const float pv = __builtin_amdgcn_exp2f(xt) * ds.inv_st;
                const float qv = __builtin_amdgcn_exp2f(scaled(zq[e] - ds.mq, sc)) * ds.inv_sq;
                const float rr = pv - qv;
                w[it][e] = rr > 0.f ? fast_ln(rr) : -INFINITY;
                wp[it][e] = xt * kLn2;
            } else {
                w[it][e] = zt[e] * invT;
                wp[it][e] = -INFINITY;
            }
            lmax = fmaxf(lmax, w[it][e]);
            lpmax = fmaxf(lpmax, wp[it][e]);
        }
    }
    __shared__ float red[2][kThreads / 64];
    lmax = wave_max(lmax);
    lpmax = wave_max(lpmax);
    if ((tid & 63) == 0) { red[0][tid >> 6] = lmax; red[1][tid >> 6] = lpmax; }
    __syncthreads();
    lmax = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    lpmax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    // A chunk with a positive residual never needs the fallback keys (the
    // row then has one); a chunk without one only needs them.
    const bool use_resid = lmax > -INFINITY;
    const float thr = (use_resid ? lmax : lpmax) + kGmin - kGmax;

    float best = -INFINITY, bestp = -INFINITY;
    int bi = 0x7FFFFFFF, bip = 0x7FFFFFFF;
    // One Philox block holds the uniforms of 8 consecutive entries: entry j of
    // the group uses half j % 2 of word j / 2.  A bf16 vector is one group; an
    // fp32 vector is half of one.
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t i0 = c0 + ((int64_t)it * kThreads + tid) * N;
        bool need = false;
#pragma unroll
        for (int e = 0; e < N; ++e) need |= (use_resid ? w[it][e] : wp[it][e]) >= thr;
        if (!need) continue;
        U64x4 c = {(uint64_t)(i0 >> 3), ctr1, 1ull, p.offset};
        const U64x4 r = philox4x64_10(c, p.seed, 0ull);
        const uint64_t words[4] = {r.x0, r.x1, r.x2, r.x3};
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float wv = use_resid ? w[it][e] : wp[it][e];
            if (wv == -INFINITY) continue;
            const int j = (int)((i0 + e) & 7);
            const uint64_t wd = words[j >> 1];
            const float u = (j & 1) ? word_to_uniform_lo(wd) : word_to_uniform(wd);
            const float key = wv - fast_ln(-fast_ln(u));
            if (use_resid) combine_arg(best, bi, key, (int)(i0 + e));
            else combine_arg(bestp, bip, key, (int)(i0 + e));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        combine_arg(best, bi, __shfl_xor(best, o), __shfl_xor(bi, o));
        combine_arg(bestp, bip, __shfl_xor(bestp, o), __shfl_xor(bip, o));
    }
    __shared__ SamplePart sw[kThreads / 64];
    const int wv = tid >> 6;
    if ((tid & 63) == 0) { sw[wv].key = best; sw[wv].idx = bi; sw[wv].keyp = bestp; sw[wv].idxp = bip; }
    __syncthreads();
    if (tid == 0) {
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

// Scratch of the allocation-free entry point: every GPU the library runs on
// holds its own copy of this array until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// it uses the device address hipGetSymbolAddress returns for the current
// device.  Every allocation-free call on a GPU shares that GPU's copy.
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

}  // namespace

hipError_t verify_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

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
    p.dstats = a.draft_stats;
    p.nrows = a.draft_stats ? 8 : kRows;
    char* w = static_cast<char*>(ws);
    size_t off = 0;
    p.stats = reinterpret_cast<StatPart*>(w + off);
    off += (size_t)a.B * kRows * p.nch1 * sizeof(StatPart);
    off = (off + 255) & ~(size_t)255;
    p.desc = reinterpret_cast<Desc*>(w + off);
    off += ((size_t)a.B * sizeof(Desc) + 255) & ~(size_t)255;
    p.samp = reinterpret_cast<SamplePart*>(w + off);

    const dim3 g1(p.nch1 * a.B * p.nrows), g2(p.nch2 * a.B), gw((a.B + 3) / 4);
    if (a.dtype == DFLASH_BF16) {
        stats_kernel<uint16_t><<<g1, kThreads, 0, s>>>(p);
        decide_kernel<uint16_t><<<a.B, kThreads, 0, s>>>(p);
        sample_kernel<uint16_t><<<g2, kThreads, 0, s>>>(p);
    } else {
        stats_kernel<float><<<g1, kThreads, 0, s>>>(p);
        decide_kernel<float><<<a.B, kThreads, 0, s>>>(p);
        sample_kernel<float><<<g2, kThreads, 0, s>>>(p);
    }
    finalize_kernel<<<gw, kThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
