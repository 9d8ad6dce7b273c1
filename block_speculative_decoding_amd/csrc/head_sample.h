// Draft proposals from the shared head's stored logits: the key of an entry
// and the (key, index) partials, shared by the head's separate sampling pass
// and the sampling epilogue of the 256 x 256 projection kernel, so that both
// paths compute the same keys.
//
// "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash", section
// "The released serving cycle" (one forward proposes all seven positions).
// Proposal k = 1..7 of sequence b comes from logits row 8b + k: greedy
// (T <= 0) keeps the largest stored logit; sampled keeps the largest key
// z / T - ln(-ln u), u = U(2, b, k, i) of the uniform layout (one
// Philox4x64-10 block per 8 entries: entry i uses half i % 2 of word
// (i / 2) % 4 of the block with counter (i / 8, 8b + k, 2, offset)); larger
// key wins, equal keys go to the lower index.
#pragma once

#include "device_common.h"
#include "gemm.h"

namespace dflash {

struct KeyIdx { float key; int idx; };
constexpr uint64_t kDraftStream = 2;   // uniform stream of draft sampling

__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Folds the 8 entries i0 .. i0 + 7 (i0 % 8 == 0, stored values f) of
// proposal row (b, k) into (best, bi).  ctr1 = 8b + k.
__device__ __forceinline__ void draft_best8(const float* f, int64_t i0, bool greedy, float invT, uint64_t ctr1,
                                            uint64_t seed, uint64_t offset, float& best, int& bi) {
    if (greedy) {
#pragma unroll
        for (int e = 0; e < 8; ++e) better(best, bi, f[e], (int)(i0 + e));
        return;
    }
    const U64x4 c = {(uint64_t)(i0 >> 3), ctr1, kDraftStream, offset};
    const U64x4 r = philox4x64_10(c, seed, 0ull);
    const uint64_t words[4] = {r.x0, r.x1, r.x2, r.x3};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint64_t wd = words[e >> 1];
        const float u = (e & 1) ? word_to_uniform_lo(wd) : word_to_uniform(wd);
        better(best, bi, f[e] * invT - fast_ln(-fast_ln(u)), (int)(i0 + e));
    }
}

// (key, index) order reduced over each 32-lane half of the wave: lane 31
// ends with lanes 0..31's result and lane 63 with lanes 32..63's (DPP row
// operations; see the reduction order in device_common.h).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void better_step(float& v, int& i) {
    better(v, i, dpp_f<CTRL, ROWS>(v, -INFINITY), dpp_i<CTRL, ROWS>(i, 0x7FFFFFFF));
}
__device__ __forceinline__ void half_wave_best(float& v, int& i) {
    better_step<kDppXor1>(v, i);
    better_step<kDppXor2>(v, i);
    better_step<kDppHalfMirror>(v, i);
    better_step<kDppMirror>(v, i);
    better_step<kDppBcast15, 0xA>(v, i);
}

// Softmax statistics of a sampled proposal row at its temperature, for
// verification's q normaliser: (m, s) with m the largest stored logit and
// s = sum 2^((z - m) * log2(e) / T) = sum e^((z - m) / T).  The scale
// log2(e) / T is split into hi + lo so that the exponent keeps the double
// scale's accuracy: x = fma(z - m, hi, (z - m) * lo), z - m exact for bf16.
struct RowStat { float m, s; };
struct StatScale { float hi, lo; };
__device__ __forceinline__ StatScale stat_scale(float T) {
    const double sc = 1.4426950408889634 / (double)T;
    StatScale r;
    r.hi = (float)sc;
    r.lo = (float)(sc - (double)r.hi);
    return r;
}
__device__ __forceinline__ float stat_exp(float dz, StatScale sc) {
    return dz == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(dz, sc.hi, dz * sc.lo));
}
// Online update with 8 consecutive stored values.
__device__ __forceinline__ void stat_add8(const float* f, StatScale sc, float& m, float& s) {
    float cm = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
    if (cm > m) {
        s = m == -INFINITY ? 0.f : s * stat_exp(m - cm, sc);
        m = cm;
    }
    if (m == -INFINITY) return;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += stat_exp(f[e] - m, sc);
    s += acc;
}
__device__ __forceinline__ void stat_merge(float& m, float& s, float m2, float s2, StatScale sc) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = (m == -INFINITY ? 0.f : s * stat_exp(m - M, sc)) + (m2 == -INFINITY ? 0.f : s2 * stat_exp(m2 - M, sc));
    m = M;
}

// Sampling epilogue of the 256 x 256 projection kernel: for each row
// 8b + k (k >= 1, row < M) and 256-column tile tn, the tile's best key goes
// to part[(7b + k - 1) * nparts + tn] (nparts = N / 256), and, when spart is
// set, a sampled row's statistics over the tile to spart at the same index.
struct HeadEpilogue {
    const float* temp;     // [B]; <= 0 means greedy
    uint64_t seed, offset;
    KeyIdx* part;
    RowStat* spart;        // optional
    int nparts;
};

// bf16 projection of the head rows with the sampling epilogue: 256 x 256
// tiles (N % 256 == 0, ks = 1), at most one workgroup per CU looping over
// them, logits stored from registers as 16-byte chunks to out_bf16.
// (Defined with the fusion kernels.)
hipError_t launch_gemm_big_head(const GemmParams& g, const HeadEpilogue& ep, hipStream_t s);

}  // namespace dflash
