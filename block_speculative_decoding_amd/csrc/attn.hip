// Non-causal draft block attention over a paged, injected KV cache (gfx950).
//
// Follows "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash",
// section "Five target states become persistent draft context": Q [B,32,8,128],
// K/V [B,8,8,128], four query heads per KV head, per-head Q/K RMSNorm before
// RoPE; the block attends bidirectionally over the cached context followed
// by its own eight keys ("DFlash & DFlash2" 4.1: K = [K_ctx ; K_blk]).
//
// bf16 design.  One workgroup (8 waves) owns (sequence b, KV heads 2h and
// 2h+1, split c); four waves work on each head.  A head's (page, head) K and
// V blocks are 4 KiB each and the two heads' blocks are neighbours, so the
// workgroup reads 8-KiB runs of the shuffled pages.  The 4 query heads x 8
// positions of KV head g form 32 query rows, so each 32-token tile is two
// dense 32x32 products on the matrix cores:
//     S^T[32 tok x 32 rows] = K[32 x 128] . Q^T        (8 x mfma 32x32x16)
//     O^T[128 x 32 rows]   += V^T[128 x 32] . P^T      (8 x mfma 32x32x16)
// The page layouts (see include/dflash.h) put each lane's operand bytes in
// one 16-byte run and make each wave-wide load one contiguous 512 B / 1 KiB
// run, so K and V go from HBM straight into operand registers.  A lane of
// S^T owns one query row and 16 of the 32 tokens, so the softmax row
// reductions need a single cross-half exchange.  Waves take tiles
// round-robin within their head; the block's own 8 keys are one extra
// (masked) tile of the last split.  A head's four waves merge through LDS;
// splits merge with a log-sum-exp kernel.  The (sequence, head pair, split)
// units are dealt to the XCDs in contiguous ranges, so each XCD reads whole
// pages of its sequences.
#include <cmath>

#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;    // waves per head, taking the head's tiles round-robin
constexpr int kHpw = 2;      // KV heads per workgroup
constexpr int kXcds = 8;     // XCDs of the part; workgroups go to them in turn
constexpr int kWgThreads = kThreads * kHpw;
constexpr int kTile = 32;
constexpr int kQStride = 136;    // bf16 per LDS row of q^ / k^blk (padded)
constexpr int kAccStride = 132;  // floats per LDS row in the wave merge
constexpr int kPartFloats = 64 + 32 * 128;  // m[32], l[32], acc[32][128]
constexpr int kMaxSplit = 32768;            // tokens per split (page ids of a split live in LDS)

struct AttnParams {
    const void* q; const void* kb; const void* vb; const void* gq; const void* gk;
    float eps; float theta;
    const void* kc; const void* vc; int64_t num_pages;
    const int32_t* bt; int max_pages;
    const int32_t* ctx_len;
    int B;
    int window; int split; int nsplit;
    void* out; float* lse;
    float* part;
    double inv_freq[64];  // theta^(-i/64), computed on the host in fp64
};

struct SeqRange { int S, t0, a0, nspl; };

// The ranges of a sequence whose ctx_len entry is S.
__device__ __forceinline__ SeqRange seq_range_of(const AttnParams& p, int S) {
    SeqRange r;
    const int cap = p.max_pages * 16;
    S = S < 0 ? 0 : (S > cap ? cap : S);
    r.S = S;
    r.t0 = p.window > 0 ? max(0, S - p.window) : 0;
    r.a0 = r.t0 & ~(kTile - 1);
    const int n = S - r.a0;
    r.nspl = n <= 0 ? 1 : (n + p.split - 1) / p.split;
    return r;
}
__device__ __forceinline__ SeqRange seq_range(const AttnParams& p, int b) { return seq_range_of(p, p.ctx_len[b]); }

// cos/sin of pos * inv_freq[i]: angle and range reduction in fp64, then fp32.
__device__ __forceinline__ void rope_cs(int pos, int i, const double* inv_freq, float& c, float& s) {
    double ang = (double)pos * inv_freq[i];
    const double two_pi = 6.283185307179586;
    ang -= rint(ang * (1.0 / two_pi)) * two_pi;
    sincosf((float)ang, &s, &c);
}

// Normalise + rotate one 128-wide row spread over 8 consecutive lanes; lane
// part p holds dims [8p, 8p+8) in x[0..7] and [64+8p, 64+8p+8) in x[8..15].
__device__ __forceinline__ void norm_rope_16(float* x, const float* g, int part, int pos,
                                             float eps, const double* inv_freq) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = x[e] * rinv * g[e];
        const float bb = x[8 + e] * rinv * g[8 + e];
        float c, s;
        rope_cs(pos, 8 * part + e, inv_freq, c, s);
        x[e] = a * c - bb * s;
        x[8 + e] = bb * c + a * s;
    }
}

// Raw bf16 of dims [8p, 8p+8) and [64+8p, 64+8p+8) of a 128-wide row, and
// their widening to x[0..15] in the order norm_rope_16 takes.
__device__ __forceinline__ void load_raw16(const uint16_t* row, int part, uint4 (&r)[2]) {
    __builtin_memcpy(&r[0], row + 8 * part, 16);
    __builtin_memcpy(&r[1], row + 64 + 8 * part, 16);
}
__device__ __forceinline__ void widen16(const uint4 (&r)[2], float* x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {r[h].x, r[h].y, r[h].z, r[h].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * h + e] = bf16_bits_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
    }
}

// norm_rope_16 with the lane's 8 frequencies inv_freq[8p + e] already in
// registers (the same arithmetic).
__device__ __forceinline__ void norm_rope_16f(float* x, const float* g, const double* fr, int pos, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = x[e] * rinv * g[e];
        const float bb = x[8 + e] * rinv * g[8 + e];
        float c, s;
        rope_cs(pos, e, fr, c, s);
        x[e] = a * c - bb * s;
        x[8 + e] = bb * c + a * s;
    }
}

template <typename T>
__device__ __forceinline__ void load_row16(const T* row, int part, float* x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = Elem<T>::load(row, 8 * part + e);
        x[8 + e] = Elem<T>::load(row, 64 + 8 * part + e);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// ---------------------------------------------------------------- bf16 MFMA kernel
constexpr int kSmemFloats = kHpw * kWaves * (64 + 32 * kAccStride);

// Attention of KV heads kHpw hp .. kHpw hp + kHpw - 1 of sequence b over the
// context tokens [tb, te) (tb a multiple of the tile), plus the block's own
// 8 keys when `last`.  part == nullptr: the result is final and goes to the
// output (and LSE); else each head's partial (m, l, acc) goes to
// part + head * part_stride (head within the workgroup).  Every thread of the
// workgroup calls it with the same arguments; smem is the workgroup's
// kSmemFloats of LDS.
__device__ __forceinline__ void attend(const AttnParams& p, int b, int hp, const SeqRange& sr, int tb, int te,
                                       bool last, float* part, int64_t part_stride, float* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hw = wave >> 2, wl = wave & 3;      // head within the workgroup, wave within the head
    const int g = hp * kHpw + hw;
    const int ntiles = te > tb ? (te - tb + kTile - 1) / kTile : 0;
    uint16_t* qs_all = reinterpret_cast<uint16_t*>(smem);        // [kHpw][32][kQStride]
    uint16_t* kbs_all = qs_all + kHpw * 32 * kQStride;           // [kHpw][8][kQStride]
    uint16_t* vbs_all = kbs_all + kHpw * 8 * kQStride;           // [kHpw][8][128]
    uint16_t* qs = qs_all + hw * 32 * kQStride;
    uint16_t* kbs = kbs_all + hw * 8 * kQStride;
    uint16_t* vbs = vbs_all + hw * 8 * 128;

    const uint16_t* gq = static_cast<const uint16_t*>(p.gq);
    const uint16_t* gk = static_cast<const uint16_t*>(p.gk);

    // ---- prologue.  Every global read it needs (q and block k rows with
    // their norm weights, v_blk, the split's page ids) is issued first; once
    // the page ids are in LDS the first context tile's K/V loads go out, and
    // q^ / k^blk (norm + RoPE) are computed while those are in flight.
    const int rn = tid >> 3, rp = tid & 7;  // q row rn = hw2*32 + hh*8 + j, dims of part rp
    const int hw2 = rn >> 5, hh = (rn >> 3) & 3, j = rn & 7;
    const bool kthr = tid < 64 * kHpw;
    const bool vthr = !kthr && tid < 64 * kHpw + 128 * kHpw;
    uint4 rq[2], rgq[2], rk[2], rgk[2];   // raw bf16 rows and norm weights
    uint4 vcopy = make_uint4(0, 0, 0, 0);
    double fr[8];                         // inv_freq[8 rp + e]
    {
        const int g2 = hp * kHpw + hw2;
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                               ((((int64_t)b * 32 + 4 * g2 + hh) * 8 + j) * 128);
        load_raw16(qrow, rp, rq);
        load_raw16(gq, rp, rgq);
#pragma unroll
        for (int e = 0; e < 8; ++e) fr[e] = p.inv_freq[8 * rp + e];
        if (kthr) {
            const int hk = tid >> 6, jj = (tid >> 3) & 7;
            const uint16_t* krow = static_cast<const uint16_t*>(p.kb) + ((((int64_t)b * 8 + hp * kHpw + hk) * 8 + jj) * 128);
            load_raw16(krow, rp, rk);
            load_raw16(gk, rp, rgk);
        } else if (vthr) {
            const int t2 = tid - 64 * kHpw;  // 128 threads x 16 B = the 2 KiB of v_blk (8 x 128 bf16) per head
            const int hv = t2 >> 7;
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.vb) +
                                                              (((int64_t)b * 8 + hp * kHpw + hv) * 8 * 128));
            vcopy = src[t2 & 127];
        }
    }
    // Physical page ids of this split, staged once in LDS (-1 past the sequence
    // or out of range) so a tile's K/V addresses need no dependent global read.
    int* pages = reinterpret_cast<int*>(vbs_all + kHpw * 8 * 128);  // [split/16 + 2]
    const int pg_first = tb >> 4;
    const int npg = ((te > tb ? te - 1 : tb) >> 4) - pg_first + 2;
    {
        const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
        for (int i = tid; i < npg; i += kWgThreads) {
            const int pg = pg_first + i;
            int ph = -1;
            if (pg * 16 < te) {
                ph = bt[pg];
                if (ph < 0 || (int64_t)ph >= p.num_pages) ph = -1;
            }
            pages[i] = ph;
        }
    }
    __syncthreads();

    const int m32 = lane & 31, hl = lane >> 5;
    const uint16_t* kc = static_cast<const uint16_t*>(p.kc);
    const uint16_t* vc = static_cast<const uint16_t*>(p.vc);
    const uint4 z4 = make_uint4(0, 0, 0, 0);

    // Issue the loads of context tile `it` into kr / vr.  Loads are
    // unconditional: a missing page reads page 0 and is zeroed in process.
    auto load = [&](int it, uint4 (&kr)[8], uint4 (&vr)[2][4]) {
        const int T0 = tb + it * kTile;
        const int li = (T0 >> 4) - pg_first;
        const int ph0 = max(pages[li], 0), ph1 = max(pages[li + 1], 0);
        const int myk = (m32 >> 4) ? ph1 : ph0;
        const uint4* kp = reinterpret_cast<const uint4*>(kc + ((int64_t)myk * 8 + g) * 2048 + 8 * ((m32 & 15) + 16 * hl));
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) kr[kb] = ld_stream(kp + 32 * kb);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int ph = kb2 ? ph1 : ph0;
            const uint4* vp = reinterpret_cast<const uint4*>(vc + ((int64_t)ph * 8 + g) * 2048 + 256 * hl + 8 * m32);
#pragma unroll
            for (int db = 0; db < 4; ++db) vr[kb2][db] = ld_stream(vp + 64 * db);
        }
    };
    // The prologue's own reads were issued before the page ids and have
    // arrived by now; waiting for them here (vmcnt 0 only) keeps the compiler
    // from waiting on the tile loads below to reach them.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    uint4 ka[8], va[2][4];
    if (wl < ntiles) load(wl, ka, va);

    {
        float xq[16], gwq[16];
        widen16(rq, xq);
        widen16(rgq, gwq);
        norm_rope_16f(xq, gwq, fr, sr.S + j, p.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qs_all[rn * kQStride + 8 * rp + e] = (uint16_t)f32_to_bf16_bits(xq[e]);
            qs_all[rn * kQStride + 64 + 8 * rp + e] = (uint16_t)f32_to_bf16_bits(xq[8 + e]);
        }
    }
    if (kthr) {
        const int hk = tid >> 6, jj = (tid >> 3) & 7;
        float xk[16], gwk[16];
        widen16(rk, xk);
        widen16(rgk, gwk);
        norm_rope_16f(xk, gwk, fr, sr.S + jj, p.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kbs_all[(hk * 8 + jj) * kQStride + 8 * rp + e] = (uint16_t)f32_to_bf16_bits(xk[e]);
            kbs_all[(hk * 8 + jj) * kQStride + 64 + 8 * rp + e] = (uint16_t)f32_to_bf16_bits(xk[8 + e]);
        }
    } else if (vthr) {
        const int t2 = tid - 64 * kHpw;
        reinterpret_cast<uint4*>(vbs_all + (t2 >> 7) * 8 * 128)[t2 & 127] = vcopy;
    }
    __syncthreads();

    const uint16_t* qlds = qs + m32 * kQStride + 64 * hl;  // this lane's Q^T operand row
    bf16x8 qreg[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qreg[kb] = *reinterpret_cast<const bf16x8*>(qlds + 8 * kb);
    const float sl2 = kLog2e * 0.08838834764831845f;      // log2(e) / sqrt(128)

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = (f32x16){};
    float m_run = -INFINITY, l_run = 0.f;

    // Scores, online softmax and P.V for one loaded tile.  `blk` marks the
    // block's own 8 keys (rows 0..7 valid).
    auto process = [&](int it, bool blk, uint4 (&kr)[8], uint4 (&vr)[2][4]) {
        const int T0 = tb + it * kTile;
        if (!blk && T0 + kTile > te) {
            // Tokens at or past the split end: their pages may be missing or
            // their slots unwritten, so zero keys and values.
            const int li = (T0 >> 4) - pg_first;
            const bool kmiss = pages[li + (m32 >> 4)] < 0 || T0 + m32 >= te;
            if (kmiss) {
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) kr[kb] = z4;
            }
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const int tbase = T0 + 16 * kb2 + 4 * hl;  // tokens tbase+{0..3}, tbase+8+{0..3}
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    uint4& w = vr[kb2][db];
                    if (tbase + 0 >= te) w.x &= 0xFFFF0000u;
                    if (tbase + 1 >= te) w.x &= 0x0000FFFFu;
                    if (tbase + 2 >= te) w.y &= 0xFFFF0000u;
                    if (tbase + 3 >= te) w.y &= 0x0000FFFFu;
                    if (tbase + 8 >= te) w.z &= 0xFFFF0000u;
                    if (tbase + 9 >= te) w.z &= 0x0000FFFFu;
                    if (tbase + 10 >= te) w.w &= 0xFFFF0000u;
                    if (tbase + 11 >= te) w.w &= 0x0000FFFFu;
                }
            }
        }
        // S^T = K . Q^T  (rows: tokens of the tile, columns: the 32 query rows)
        f32x16 s = {};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const bf16x8 qop = qreg[kb];
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[kb]), qop, s, 0, 0, 0);
        }
        // Lane holds query row m32 and tokens 8*jj + 4*hl + r  (register 4*jj + r).
        float pv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = 8 * (r >> 2) + 4 * hl + (r & 3);
            bool valid;
            if (blk) {
                valid = tok < 8;
            } else {
                const int t = T0 + tok;
                valid = t >= sr.t0 && t < te;
            }
            pv[r] = valid ? s[r] * sl2 : -INFINITY;
            tmax = fmaxf(tmax, pv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        uint32_t pk[8];
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(pv[2 * r] - m_use),
                                           __builtin_amdgcn_exp2f(pv[2 * r + 1] - m_use));
            pk[r] = w;
            rs += lo_bf16(w) + hi_bf16(w);
        }
        rs += __shfl_xor(rs, 32);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
        const bf16x8 pb0 = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
        const bf16x8 pb1 = as_bf16x8(make_uint4(pk[4], pk[5], pk[6], pk[7]));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[0][db]), pb0, acc[db], 0, 0, 0);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[1][db]), pb1, acc[db], 0, 0, 0);
        }
    };

    {
        for (int it = wl; it < ntiles; it += kWaves) {
            if (it != wl) load(it, ka, va);   // tile wl was issued in the prologue
            process(it, false, ka, va);
        }
        // The block's own 8 keys / values: one masked tile for the wave next
        // in the round-robin order, in the last split of the sequence.
        if (last && wl == (ntiles & (kWaves - 1))) {
            if (m32 < 8) {
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    ka[kb] = *reinterpret_cast<const uint4*>(kbs + m32 * kQStride + 64 * hl + 8 * kb);
            } else {
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) ka[kb] = z4;
            }
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const int d = 32 * db + m32;
                uint4 w;
                w.x = (uint32_t)vbs[(4 * hl + 0) * 128 + d] | ((uint32_t)vbs[(4 * hl + 1) * 128 + d] << 16);
                w.y = (uint32_t)vbs[(4 * hl + 2) * 128 + d] | ((uint32_t)vbs[(4 * hl + 3) * 128 + d] << 16);
                w.z = 0;
                w.w = 0;
                va[0][db] = w;
                va[1][db] = z4;
            }
            process(ntiles, true, ka, va);
        }
    }

    // ---- merge the four waves through LDS
    __syncthreads();
    float* wm = smem + wave * (64 + 32 * kAccStride);
    if (hl == 0) { wm[m32] = m_run; wm[32 + m32] = l_run; }
    float* wacc = wm + 64;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            wacc[m32 * kAccStride + 32 * db + 8 * (r >> 2) + 4 * hl + (r & 3)] = acc[db][r];
    __syncthreads();

    // Threads [256 h, 256 h + 256) merge head h's four waves.
    const int hm = tid >> 8, gm = hp * kHpw + hm;
    const int n = (tid & 255) >> 3, d0 = 16 * (tid & 7);
    const float* wbase = smem + hm * kWaves * (64 + 32 * kAccStride);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wbase[w * (64 + 32 * kAccStride) + n]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float* base = wbase + w * (64 + 32 * kAccStride);
        const float f = __builtin_amdgcn_exp2f(base[n] - Mu);
        L += base[32 + n] * f;
        const float4* av = reinterpret_cast<const float4*>(base + 64 + n * kAccStride + d0);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4 v = av[e4];
            o[4 * e4 + 0] += f * v.x; o[4 * e4 + 1] += f * v.y;
            o[4 * e4 + 2] += f * v.z; o[4 * e4 + 3] += f * v.w;
        }
    }
    if (part == nullptr) {
        const float inv = 1.0f / L;
        uint16_t* orow = static_cast<uint16_t*>(p.out) + ((((int64_t)b * 32 + 4 * gm + (n >> 3)) * 8 + (n & 7)) * 128) + d0;
        uint4 w0, w1;
        w0.x = pack_bf16x2(o[0] * inv, o[1] * inv);   w0.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        w0.z = pack_bf16x2(o[4] * inv, o[5] * inv);   w0.w = pack_bf16x2(o[6] * inv, o[7] * inv);
        w1.x = pack_bf16x2(o[8] * inv, o[9] * inv);   w1.y = pack_bf16x2(o[10] * inv, o[11] * inv);
        w1.z = pack_bf16x2(o[12] * inv, o[13] * inv); w1.w = pack_bf16x2(o[14] * inv, o[15] * inv);
        reinterpret_cast<uint4*>(orow)[0] = w0;
        reinterpret_cast<uint4*>(orow)[1] = w1;
        if (p.lse && (tid & 7) == 0)
            p.lse[((int64_t)b * 32 + 4 * gm + (n >> 3)) * 8 + (n & 7)] = (Mu + log2f(L)) * kLn2;
    } else {
        float* pp = part + hm * part_stride;
        if ((tid & 7) == 0) { pp[n] = M; pp[32 + n] = L; }
        float4* dst = reinterpret_cast<float4*>(pp + 64 + n * 128 + d0);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            dst[e4] = make_float4(o[4 * e4], o[4 * e4 + 1], o[4 * e4 + 2], o[4 * e4 + 3]);
    }
}

// Fixed splits: work unit u = c + nsplit (hp + 4 b) (split c, KV-head pair hp,
// sequence b) takes tokens [a0 + c split, a0 + (c + 1) split) of its
// sequence; the last split also takes the block's keys.  With several splits
// each writes its partial.  Workgroups go to the XCDs in turn (workgroup L to
// XCD L mod 8), so unit u is given to workgroup (u / per) + 8 (u mod per):
// each XCD takes a contiguous range of units, i.e. whole sequences with all
// four head pairs.  With the plain order every XCD would read one fixed
// 8-KiB slot of every 32-KiB page and some XCDs ran 8% slower than others.
__global__ __launch_bounds__(kWgThreads, 1) void attn_bf16_kernel(AttnParams p) {
    const int per = gridDim.x / kXcds;
    const int u = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (u >= p.nsplit * (8 / kHpw) * p.B) return;
    const int c = u % p.nsplit, hp = (u / p.nsplit) % (8 / kHpw), b = u / (p.nsplit * (8 / kHpw));
    const SeqRange sr = seq_range(p, b);
    if (c >= sr.nspl) return;
    const int tb = sr.a0 + c * p.split;
    const int te = min(sr.S, tb + p.split);
    __shared__ __attribute__((aligned(16))) float smem[kSmemFloats];
    float* part = sr.nspl == 1 ? nullptr : p.part + (((int64_t)b * 8 + hp * kHpw) * p.nsplit + c) * kPartFloats;
    attend(p, b, hp, sr, tb, te, c == sr.nspl - 1, part, (int64_t)p.nsplit * kPartFloats, smem);
}

// ---------------------------------------------------------------- balanced pieces
// Balanced mode: the context tiles of all sequences, each followed by its
// block tile, are laid end to end and cut into kPieces equal pieces per
// KV-head pair; workgroup (piece, hp) walks the sequence segments of its
// piece.  A segment holding a whole sequence writes the output; a sequence
// cut by a piece boundary leaves one partial per piece it touches, in slot 0
// of a piece whose first sequence it is, else slot 1 (only a piece's last
// segment can be cut and not be its first), and the merge combines them.
// Workgroup (0, 0) also writes the merge table after the partials: entry b =
// P0 | P1 << 8 | slot << 16 (the pieces sequence b touches, and the slot of
// its partial in P0), entry B = the tile total.
constexpr int kPieces = 64;             // pieces per KV-head pair: 4 x 64 workgroups, one per CU
constexpr int kMaxBalancedB = 1024;
constexpr size_t kBalancedPartFloats = (size_t)kPieces * 2 * 8 * kPartFloats;   // merge table after these

// Tiles of a sequence: its context tiles, then the block tile.
__device__ __forceinline__ int seq_tiles(const SeqRange& sr) {
    return (sr.S > sr.a0 ? (sr.S - sr.a0 + kTile - 1) / kTile : 0) + 1;
}

// s_pref[b] = first global tile of sequence b, s_pref[B] = all tiles (the
// return value), s_len[b] = ctx_len[b] (so a segment's range needs no global
// read); every thread of the workgroup takes part.
__device__ int tile_prefix(const AttnParams& p, int* s_pref, int* s_len, int* s_tmp) {
    const int nt = blockDim.x, tid = threadIdx.x;
    const int per = (p.B + nt - 1) / nt;
    const int b0 = tid * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
        if (b0 + i < p.B) {
            const int S = p.ctx_len[b0 + i];
            s_len[b0 + i] = S;
            sum += seq_tiles(seq_range_of(p, S));
        }
    s_tmp[tid] = sum;
    __syncthreads();
    for (int o = 1; o < nt; o <<= 1) {   // inclusive scan over the threads' sums
        const int v = tid >= o ? s_tmp[tid - o] : 0;
        __syncthreads();
        s_tmp[tid] += v;
        __syncthreads();
    }
    int run = s_tmp[tid] - sum;
    for (int i = 0; i < per; ++i)
        if (b0 + i < p.B) {
            s_pref[b0 + i] = run;
            run += seq_tiles(seq_range_of(p, s_len[b0 + i]));
        }
    if (tid == nt - 1) s_pref[p.B] = s_tmp[nt - 1];
    __syncthreads();
    return s_pref[p.B];
}

// Piece p of KV-head pair hp runs as workgroup p + 64 hp, on XCD p mod 8.
// Workgroups on odd XCDs read these random 8-KiB page blocks 5-10% slower
// than those on even XCDs (per-workgroup timings over many launches, on
// several boards), so even pieces take 27 shares of the tiles and odd ones 25.
constexpr int kPieceWEven = 27, kPieceWOdd = 25;
constexpr int kPieceWSum = kPieces / 2 * (kPieceWEven + kPieceWOdd);
__host__ __device__ __forceinline__ int piece_lo(int piece, int TT) {
    const int64_t w = (int64_t)(piece >> 1) * (kPieceWEven + kPieceWOdd) + (piece & 1) * kPieceWEven;
    return (int)(w * TT / kPieceWSum);
}
// The piece holding global tile t: the last one that starts at or before t.
__device__ __forceinline__ int piece_of(int t, int TT) {
    int lo = 0, hi = kPieces - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (piece_lo(mid, TT) <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kWgThreads, 1) void attn_bf16_balanced_kernel(AttnParams p) {
    const int piece = blockIdx.x, hp = blockIdx.y;
    __shared__ __attribute__((aligned(16))) float smem[kSmemFloats];
    __shared__ int s_pref[kMaxBalancedB + 1];
    __shared__ int s_len[kMaxBalancedB];
    __shared__ int s_tmp[kWgThreads];
    const int TT = tile_prefix(p, s_pref, s_len, s_tmp);
    if (piece == 0 && hp == 0) {
        int* table = reinterpret_cast<int*>(p.part + kBalancedPartFloats);
        for (int b = threadIdx.x; b < p.B; b += blockDim.x) {
            const int t0 = s_pref[b], P0 = piece_of(t0, TT), P1 = piece_of(s_pref[b + 1] - 1, TT);
            table[b] = P0 | (P1 << 8) | ((piece_lo(P0, TT) == t0 ? 0 : 1) << 16);
        }
        if (threadIdx.x == 0) table[p.B] = TT;
    }
    const int lo = piece_lo(piece, TT), hi = piece_lo(piece + 1, TT);
    if (lo >= hi) return;
    int first = 0, top = p.B - 1;   // the sequence holding tile lo: last b with s_pref[b] <= lo
    while (first < top) {
        const int mid = (first + top + 1) >> 1;
        if (s_pref[mid] <= lo) first = mid;
        else top = mid - 1;
    }
    for (int b = first; b < p.B && s_pref[b] < hi; ++b) {
        const SeqRange sr = seq_range_of(p, s_len[b]);
        const int nt = seq_tiles(sr) - 1;   // context tiles; the block tile is local tile nt
        const int g0 = max(lo, s_pref[b]) - s_pref[b], g1 = min(hi, s_pref[b + 1]) - s_pref[b];
        const int tb = sr.a0 + kTile * g0;
        const int te = min(sr.S, sr.a0 + kTile * min(g1, nt));
        const bool last = g1 > nt;
        float* part = g0 == 0 && last ? nullptr
                                      : p.part + (((int64_t)piece * 2 + (b == first ? 0 : 1)) * 8 + hp * kHpw) * kPartFloats;
        __syncthreads();   // the previous segment is done with the LDS
        attend(p, b, hp, sr, tb, te, last, part, kPartFloats, smem);
    }
}

// ---------------------------------------------------------------- split merge
// One workgroup per (KV head g, sequence b, quarter of the 32 query rows):
// thread (row n, 4 dims) reads one float4 of each of the count partials
// (at(i), i < count; a null at(i) holds nothing).  They are taken kMergeU at a time with every load of a
// batch issued before any is used, and batches combine online (running
// maximum M in log2 units, sum L and the weighted outputs rescaled when M
// grows).
constexpr int kMergeU = 16;

template <typename T, typename PartAt>
__device__ __forceinline__ void merge_rows(const AttnParams& p, int g, int b, int rq, int count, PartAt at) {
    const int tid = threadIdx.x;
    const int n = 8 * rq + (tid >> 5), d0 = 4 * (tid & 31);
    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < count; c0 += kMergeU) {
        float mc[kMergeU], lc[kMergeU];
        float4 ac[kMergeU];
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
            const float* pc = c0 + u < count ? at(c0 + u) : nullptr;
            if (pc) {
                mc[u] = pc[n];
                lc[u] = pc[32 + n];
                ac[u] = *reinterpret_cast<const float4*>(pc + 64 + n * 128 + d0);
            } else {
                mc[u] = -INFINITY;
                lc[u] = 0.f;
                ac[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) Mn = fmaxf(Mn, mc[u]);
        if (Mn == -INFINITY) continue;
        const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        L *= sc;
        o.x *= sc; o.y *= sc; o.z *= sc; o.w *= sc;
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
            const float f = mc[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc[u] - Mn);
            L += lc[u] * f;
            o.x += f * ac[u].x; o.y += f * ac[u].y; o.z += f * ac[u].z; o.w += f * ac[u].w;
        }
        M = Mn;
    }
    const float Mu = M == -INFINITY ? 0.f : M;
    const float inv = 1.0f / L;
    T* orow = static_cast<T*>(p.out) + ((((int64_t)b * 32 + 4 * g + (n >> 3)) * 8 + (n & 7)) * 128) + d0;
    Elem<T>::store(orow, 0, o.x * inv);
    Elem<T>::store(orow, 1, o.y * inv);
    Elem<T>::store(orow, 2, o.z * inv);
    Elem<T>::store(orow, 3, o.w * inv);
    if (p.lse && (tid & 31) == 0)
        p.lse[((int64_t)b * 32 + 4 * g + (n >> 3)) * 8 + (n & 7)] = (Mu + log2f(L)) * kLn2;
}

// Fixed splits: partial c of (b, g) at ((b * 8 + g) * nsplit + c) * kPartFloats.
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnParams p) {
    const int g = blockIdx.x, b = blockIdx.y, rq = blockIdx.z;
    const SeqRange sr = seq_range(p, b);
    if (sr.nspl <= 1) return;
    const float* base = p.part + ((int64_t)b * 8 + g) * p.nsplit * kPartFloats;
    merge_rows<T>(p, g, b, rq, sr.nspl, [&](int c) { return base + (int64_t)c * kPartFloats; });
}

// Balanced pieces: sequence b's partials in the pieces P0 .. P1 it touches.
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_merge_balanced_kernel(AttnParams p) {
    const int g = blockIdx.x, b = blockIdx.y, rq = blockIdx.z;
    const int* table = reinterpret_cast<const int*>(p.part + kBalancedPartFloats);
    const int e = table[b];
    const int P0 = e & 0xFF, P1 = (e >> 8) & 0xFF, slot0 = e >> 16;
    if (P0 == P1) return;   // whole in one piece: written by the attention kernel
    const int TT = table[p.B];
    // With fewer tiles than pieces, pieces between P0 and P1 can be empty:
    // they wrote no partial.
    merge_rows<T>(p, g, b, rq, P1 - P0 + 1, [&](int i) -> const float* {
        const int piece = P0 + i;
        if (piece_lo(piece, TT) >= piece_lo(piece + 1, TT)) return nullptr;
        return p.part + (((int64_t)piece * 2 + (i == 0 ? slot0 : 0)) * 8 + g) * kPartFloats;
    });
}

// ---------------------------------------------------------------- fp32 VALU kernel
// Plain fp32 path (small fp32 workloads): one workgroup per (b, g), eight lanes
// per query row, scalar loads through the page layout, no split.
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnParams p) {
    const int g = blockIdx.x, b = blockIdx.y;
    const SeqRange sr = seq_range(p, b);
    const int tid = threadIdx.x;
    const int n = tid >> 3, part = tid & 7, hh = n >> 3, j = n & 7;
    __shared__ float kbs[8][128];

    const float* gq = static_cast<const float*>(p.gq);
    const float* gk = static_cast<const float*>(p.gk);
    float x[16], gw[16];
    if (tid < 64) {
        const int jj = tid >> 3;
        const float* krow = static_cast<const float*>(p.kb) + ((((int64_t)b * 8 + g) * 8 + jj) * 128);
        load_row16(krow, part, x);
        load_row16(gk, part, gw);
        norm_rope_16(x, gw, part, sr.S + jj, p.eps, p.inv_freq);
#pragma unroll
        for (int e = 0; e < 8; ++e) { kbs[jj][8 * part + e] = x[e]; kbs[jj][64 + 8 * part + e] = x[8 + e]; }
    }
    const float* qrow = static_cast<const float*>(p.q) + ((((int64_t)b * 32 + 4 * g + hh) * 8 + j) * 128);
    float q[16];
    load_row16(qrow, part, q);
    load_row16(gq, part, gw);
    norm_rope_16(q, gw, part, sr.S + j, p.eps, p.inv_freq);
    __syncthreads();

    const float* kc = static_cast<const float*>(p.kc);
    const float* vc = static_cast<const float*>(p.vc);
    const float* vb = static_cast<const float*>(p.vb) + ((int64_t)b * 8 + g) * 8 * 128;
    const float sl2 = kLog2e * 0.08838834764831845f;
    float m = -INFINITY, l = 0.f, o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;

    // Online-softmax update with up to four tokens (kx / vx rows; sc scaled
    // scores, -inf for an unused slot).
    auto step4 = [&](float (*kx)[16], float (*vx)[16], const bool* use) {
        float sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) dot += q[e] * kx[u][e];
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 4);
            sc[u] = use[u] ? dot * sl2 : -INFINITY;
        }
        float mn = m;
#pragma unroll
        for (int u = 0; u < 4; ++u) mn = fmaxf(mn, sc[u]);
        if (mn == -INFINITY) return;
        const float a = exp2f(m - mn);
        l *= a;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] *= a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float pw = exp2f(sc[u] - mn);
            l += pw;
#pragma unroll
            for (int e = 0; e < 16; ++e) o[e] = fmaf(pw, vx[u][e], o[e]);
        }
        m = mn;
    };

    // Context, one page at a time: the page's K and V blocks of head g (two
    // contiguous 8 KiB runs) are staged in LDS by all threads with 16-byte
    // loads, the next page's loads in registers meanwhile.  Tokens outside
    // [t0, S) of a page take no part; missing pages read as zeros.
    __shared__ __align__(16) float ks[2048], vt[16][132];   // K in the page layout, V as [token][dim]
    const int pg0 = sr.t0 >> 4, pg1 = (sr.S + 15) >> 4;
    float4 rk[2], rv[2];
    auto fetch = [&](int pg) {
        const int ph = p.bt[(int64_t)b * p.max_pages + pg];
        const bool okp = ph >= 0 && (int64_t)ph < p.num_pages;
        const float4* kp = reinterpret_cast<const float4*>(kc + ((int64_t)(okp ? ph : 0) * 8 + g) * 2048);
        const float4* vp = reinterpret_cast<const float4*>(vc + ((int64_t)(okp ? ph : 0) * 8 + g) * 2048);
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            rk[i] = okp ? kp[i * kThreads + tid] : z;
            rv[i] = okp ? vp[i * kThreads + tid] : z;
        }
    };
    if (pg0 < pg1) fetch(pg0);
    for (int pg = pg0; pg < pg1; ++pg) {
        __syncthreads();   // the previous page's reads of ks / vs are done
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            reinterpret_cast<float4*>(ks)[i * kThreads + tid] = rk[i];
            // element f of the V block: dim 32 (f >> 9) + ((f >> 3) & 31), token
            // from bit 8 and the low three bits (the layout's slot order)
            const float v4[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int f = (i * kThreads + tid) * 4 + c;
                const int jj = f & 7;
                const int d = 32 * (f >> 9) + ((f >> 3) & 31);
                const int tt = ((jj >> 2) << 3) | (((f >> 8) & 1) << 2) | (jj & 3);
                vt[tt][d] = v4[c];
            }
        }
        __syncthreads();
        if (pg + 1 < pg1) fetch(pg + 1);
        const int lo = max(sr.t0 - 16 * pg, 0), hi = min(sr.S - 16 * pg, 16);
        for (int t0 = lo; t0 < hi; t0 += 4) {
            float kx[4][16], vx[4][16];
            bool use[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int tt = min(t0 + u, 15);
                use[u] = t0 + u < hi;   // slots outside [t0, S) may hold anything (even NaN): zeroed
                // dims 8 part .. +7 and 64 + 8 part .. +7: contiguous in both
                const float4* k0 = reinterpret_cast<const float4*>(ks + 256 * part + 8 * tt);
                const float4* k1 = reinterpret_cast<const float4*>(ks + 256 * part + 8 * (tt + 16));
                const float4* v0 = reinterpret_cast<const float4*>(&vt[tt][8 * part]);
                const float4* v1 = reinterpret_cast<const float4*>(&vt[tt][64 + 8 * part]);
                const float4 kk[4] = {k0[0], k0[1], k1[0], k1[1]}, vv[4] = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float kf[4] = {kk[c].x, kk[c].y, kk[c].z, kk[c].w};
                    const float vf[4] = {vv[c].x, vv[c].y, vv[c].z, vv[c].w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        kx[u][4 * c + r] = use[u] ? kf[r] : 0.f;
                        vx[u][4 * c + r] = use[u] ? vf[r] : 0.f;
                    }
                }
            }
            step4(kx, vx, use);
        }
    }
    // The block's own 8 keys and values.
    for (int j0 = 0; j0 < 8; j0 += 4) {
        float kx[4][16], vx[4][16];
        bool use[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            use[u] = true;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int d = e < 8 ? 8 * part + e : 64 + 8 * part + (e - 8);
                kx[u][e] = kbs[j0 + u][d];
                vx[u][e] = vb[(j0 + u) * 128 + d];
            }
        }
        step4(kx, vx, use);
    }
    const float inv = 1.0f / l;
    float* orow = static_cast<float*>(p.out) + ((((int64_t)b * 32 + 4 * g + hh) * 8 + j) * 128);
#pragma unroll
    for (int e = 0; e < 8; ++e) { orow[8 * part + e] = o[e] * inv; orow[64 + 8 * part + e] = o[8 + e] * inv; }
    if (p.lse && part == 0) p.lse[((int64_t)b * 32 + 4 * g + hh) * 8 + j] = (m + log2f(l)) * kLn2;
}

}  // namespace

AttnPlan attn_plan(const dflash_attn_args& a) {
    AttnPlan pl;
    int64_t cap = (int64_t)a.max_pages * 16;
    if (a.window > 0 && a.window < cap) cap = a.window;
    cap += kTile;  // alignment slack of the first tile
    if (a.dtype == DFLASH_F32) {
        pl.split_tokens = 0;
        pl.nsplit = 1;
        pl.ws_bytes = 0;
        return pl;
    }
    pl.balanced = false;
    if (a.split_tokens == DFLASH_SPLIT_BALANCED) {
        // Balanced pieces, while every piece fits the page-id staging of one
        // split (a piece spans at most its share of the tiles, plus one).
        const int64_t tiles = (int64_t)a.B * (cap / kTile + 2);
        const int64_t piece_tokens = (tiles * kPieceWEven / kPieceWSum + 2) * kTile;
        if (a.B <= kMaxBalancedB && piece_tokens <= kMaxSplit) {
            pl.balanced = true;
            pl.split_tokens = 0;
            pl.nsplit = 1;
            pl.ws_bytes = kBalancedPartFloats * sizeof(float) + ((size_t)a.B + 1) * sizeof(int);
            return pl;
        }
    }
    int split;
    if (a.split_tokens > 0) {
        split = a.split_tokens;
    } else {
        // One residency round: one 8-wave workgroup per CU on 256 CUs.
        // Fewer, longer splits stream better and leave less to merge.
        const int64_t pairs = (int64_t)a.B * (8 / kHpw);
        const int64_t target = 512 / kHpw;
        int64_t want = (target + pairs - 1) / pairs;
        if (want < 1) want = 1;
        int64_t s = (cap + want - 1) / want;
        s = (s + 127) / 128 * 128;
        if (s < 128) s = 128;
        if (s > kMaxSplit) s = kMaxSplit;
        split = (int)s;
    }
    pl.split_tokens = split;
    pl.nsplit = (int)((cap + split - 1) / split);
    if (pl.nsplit < 1) pl.nsplit = 1;
    pl.ws_bytes = pl.nsplit > 1 ? (size_t)a.B * 8 * pl.nsplit * kPartFloats * sizeof(float) : 0;
    return pl;
}

hipError_t launch_attn(const dflash_attn_args& a, const AttnPlan& pl, void* ws, hipStream_t s) {
    AttnParams p;
    p.q = a.q; p.kb = a.k_blk; p.vb = a.v_blk; p.gq = a.gq; p.gk = a.gk;
    p.eps = a.eps; p.theta = a.rope_theta;
    p.kc = a.k_cache; p.vc = a.v_cache; p.num_pages = a.num_pages;
    p.bt = a.block_table; p.max_pages = a.max_pages; p.ctx_len = a.ctx_len; p.B = a.B;
    p.window = a.window; p.split = pl.split_tokens > 0 ? pl.split_tokens : (1 << 30); p.nsplit = pl.nsplit;
    p.out = a.out; p.lse = a.lse_out;
    p.part = static_cast<float*>(ws);
    for (int i = 0; i < 64; ++i) p.inv_freq[i] = std::pow((double)a.rope_theta, -(double)i / 64.0);
    if (a.dtype == DFLASH_F32) {
        attn_f32_kernel<<<dim3(8, a.B), kThreads, 0, s>>>(p);
        return hipGetLastError();
    }
    if (pl.balanced) {
        attn_bf16_balanced_kernel<<<dim3(kPieces, 8 / kHpw), kWgThreads, 0, s>>>(p);
        attn_merge_balanced_kernel<uint16_t><<<dim3(8, a.B, 4), kThreads, 0, s>>>(p);
        return hipGetLastError();
    }
    const int units = pl.nsplit * (8 / kHpw) * a.B;
    attn_bf16_kernel<<<(units + kXcds - 1) / kXcds * kXcds, kWgThreads, 0, s>>>(p);
    if (pl.nsplit > 1) attn_merge_kernel<uint16_t><<<dim3(8, a.B, 4), kThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace dflash
