// The rest of a draft layer around block attention (gfx950).
//
// Follows "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash",
// sections "The released serving cycle" (an eight-position block: one anchor
// and seven mask tokens, one non-causal five-layer forward) and "Five target
// states become persistent draft context" (Q [B,32,8,128], block K/V
// [B,8,8,128]), and "DFlash & DFlash2", sections 4.1 (Q = W^Q H_d and the H_d
// halves of K/V) and 4.2 (the target's embedding table is shared).  The layer
// around attention is read as the pre-norm decoder layer of the Qwen3 family
// the first page names: input RMSNorm, fused Q/K/V projection; output
// projection and residual; post-attention RMSNorm, SwiGLU MLP and residual;
// a final RMSNorm after the last layer.
//
// Rows are the B x 8 block positions (M = 8B, a few hundred to a few
// thousand), so every projection is a weight-streaming GEMM run by the split-K
// kernel of gemm.h; the small launches here sum its fp32 partials and apply
// the elementwise step that follows (head scatter, residual + norm, SwiGLU).
// Every stored activation is rounded to the storage type once, from fp32.
//
// Launch sequence of dflash_draft_qkv:  norm -> gemm (N = 6144) -> scatter
//   (where the GEMM would run two K splits, it runs unsplit on two k-groups
//   per workgroup and writes the q / k_blk / v_blk layouts itself)
// Launch sequence of dflash_draft_mlp:  transpose -> gemm (N = 2560, K = 4096)
//   -> residual + norm (with DFlash2's block convolution: residual + conv +
//   norm per sequence) -> gemm (N = 10240; unsplit bf16 products go
//   through the GEMM's SwiGLU epilogue, else the partials through swiglu)
//   -> gemm (N = 2560, K = 5120) -> residual (+ final norm)
#include "device_common.h"
#include "gemm.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kD = DFLASH_D;                          // 2560
constexpr int kQkvN = (DFLASH_HQ + 2 * DFLASH_HKV) * DFLASH_HEAD_DIM;  // 6144
constexpr int kQN = DFLASH_HQ * DFLASH_HEAD_DIM;      // 4096
constexpr int kKvN = DFLASH_HKV * DFLASH_HEAD_DIM;    // 1024
constexpr int kInter = DFLASH_INTER;                  // 5120

// The value a float takes once stored as T.
template <typename T> __device__ __forceinline__ float round_as(float v);
template <> __device__ __forceinline__ float round_as<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_as<uint16_t>(float v) {
    return bf16_bits_to_f32(f32_to_bf16_bits(v));
}

// Eight consecutive elements of T as fp32 (one 16-byte access for bf16, two
// for fp32).  Element offsets must be multiples of 8.
template <typename T> struct V8;
template <> struct V8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x); f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
        f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z); f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* f) {
        uint4 w;
        w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
        w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<uint4*>(p) = w;
    }
};
template <> struct V8<float> {
    static __device__ __forceinline__ void load(const float* p, float* f) {
        const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* f) {
        *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
};

// acc[0..7] += sum over the ks split-K partials of the 8 columns at i (all
// partial loads issued before the first add: the loop is unrolled to the
// largest split count).
__device__ __forceinline__ void add_parts8(const float* __restrict__ part, int ks, int64_t stride, int64_t i,
                                           float* acc) {
    float4 v[2 * kGemmMaxKs];
#pragma unroll
    for (int s = 0; s < kGemmMaxKs; ++s) {
        if (s < ks) {
            v[2 * s] = *reinterpret_cast<const float4*>(part + s * stride + i);
            v[2 * s + 1] = *reinterpret_cast<const float4*>(part + s * stride + i + 4);
        }
    }
#pragma unroll
    for (int s = 0; s < kGemmMaxKs; ++s) {
        if (s < ks) {
            acc[0] += v[2 * s].x; acc[1] += v[2 * s].y; acc[2] += v[2 * s].z; acc[3] += v[2 * s].w;
            acc[4] += v[2 * s + 1].x; acc[5] += v[2 * s + 1].y; acc[6] += v[2 * s + 1].z; acc[7] += v[2 * s + 1].w;
        }
    }
}

// Row kernels over 2560 columns: 320 threads, 8 consecutive columns each.
constexpr int kRowThreads = kD / 8;   // 320 = 5 waves

// Sum over the 320 threads of a row workgroup (5 waves through LDS).
__device__ __forceinline__ float row_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3] + red[4];
}

// x[8b + j] = emb[j == 0 ? anchor[b] : mask_id]; an anchor outside [0, V)
// gives a zero row.  One workgroup per block row; the bits are copied.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void embed_kernel(const T* __restrict__ emb, int64_t V,
                                                             const int32_t* __restrict__ anchor, int mask_id,
                                                             T* __restrict__ x) {
    const int row = blockIdx.x;
    const int b = row >> 3, j = row & 7;
    const int64_t id = j == 0 ? (int64_t)anchor[b] : (int64_t)mask_id;
    const bool ok = id >= 0 && id < V;
    const int c = threadIdx.x * 8;
    float f[8] = {};
    if (ok) V8<T>::load(emb + id * kD + c, f);
    V8<T>::store(x + (int64_t)row * kD + c, f);
}

// out = g * x / sqrt(mean(x^2) + eps) over 2560 columns; one workgroup per row.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void norm_rows_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                                 float eps, T* __restrict__ out) {
    __shared__ float red[kRowThreads / 64];
    const int64_t row = (int64_t)blockIdx.x * kD;
    const int c = threadIdx.x * 8;
    float v[8], gv[8];
    V8<T>::load(x + row + c, v);
    V8<T>::load(g + c, gv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    const float rinv = 1.0f / sqrtf(row_sum(ss, red) * (1.0f / kD) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = gv[e] * v[e] * rinv;
    V8<T>::store(out + row + c, v);
}

// Sum the Q/K/V partials of row m = 8b + j and scatter column n to
// q[b][n/128][j][n%128] (n < 4096), k_blk / v_blk likewise for the next two
// 1024-column groups.  A thread owns 8 consecutive columns (one head, 8
// consecutive dims): 768 groups per row, 3 per thread.
template <typename T>
__global__ __launch_bounds__(kThreads) void qkv_scatter_kernel(const float* __restrict__ part, int ks, int M,
                                                                T* __restrict__ q, T* __restrict__ k,
                                                                T* __restrict__ v) {
    const int m = blockIdx.x;
    const int b = m >> 3, j = m & 7;
    const int64_t stride = (int64_t)M * kQkvN;
    constexpr int kPer = kQkvN / 8 / kThreads;  // 3
    float y[kPer][8] = {};
#pragma unroll
    for (int i = 0; i < kPer; ++i) add_parts8(part, ks, stride, (int64_t)m * kQkvN + 8 * (threadIdx.x + kThreads * i), y[i]);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int n = 8 * (threadIdx.x + kThreads * i);
        const int d = n & 127;
        T* dst;
        if (n < kQN) dst = q + (((int64_t)b * DFLASH_HQ + (n >> 7)) * 8 + j) * 128 + d;
        else if (n < kQN + kKvN) dst = k + (((int64_t)b * DFLASH_HKV + ((n - kQN) >> 7)) * 8 + j) * 128 + d;
        else dst = v + (((int64_t)b * DFLASH_HKV + ((n - kQN - kKvN) >> 7)) * 8 + j) * 128 + d;
        V8<T>::store(dst, y[i]);
    }
}

// Attention output [B][32][8][128] -> rows [8B][4096]: row 8b + j, column
// 128 h + d holds o[b][h][j][d] (the input layout of W_O).  512 groups of 8
// columns per row, 2 per thread.
template <typename T>
__global__ __launch_bounds__(kThreads) void heads_to_rows_kernel(const T* __restrict__ o, T* __restrict__ ao) {
    const int m = blockIdx.x;
    const int b = m >> 3, j = m & 7;
    float f[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 8 * (threadIdx.x + kThreads * i);
        V8<T>::load(o + (((int64_t)b * DFLASH_HQ + (c >> 7)) * 8 + j) * 128 + (c & 127), f[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) V8<T>::store(ao + (int64_t)m * kQN + 8 * (threadIdx.x + kThreads * i), f[i]);
}

// out = resid + sum of the partials (stored as T); when g is given, also
// norm_out = g * r / sqrt(mean(r^2) + eps) with r the stored value of out.
// One workgroup per 2560-wide row.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void residual_kernel(const float* __restrict__ part, int ks, int M,
                                                                const T* resid, T* out, const T* __restrict__ g,
                                                                float eps, T* __restrict__ norm_out) {
    __shared__ float red[kRowThreads / 64];
    const int64_t row = (int64_t)blockIdx.x * kD;
    const int c = threadIdx.x * 8;
    float r[8];
    V8<T>::load(resid + row + c, r);
    add_parts8(part, ks, (int64_t)M * kD, row + c, r);
    V8<T>::store(out + row + c, r);
    if (g == nullptr) return;  // uniform over the workgroup
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        r[e] = round_as<T>(r[e]);
        ss += r[e] * r[e];
    }
    float gv[8];
    V8<T>::load(g + c, gv);
    const float rinv = 1.0f / sqrtf(row_sum(ss, red) * (1.0f / kD) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = gv[e] * r[e] * rinv;
    V8<T>::store(norm_out + row + c, r);
}

// DFlash2's block convolution fused with the post-attention residual: one
// workgroup per sequence (8 block rows, 8 columns per thread).
//   h[t]  = x[t] + sum of the W_O partials           (stored as T)
//   h'[t] = h[t] + b + sum_{j < k, t - j >= 0} w[j] * h[t - j]   (from the
//           stored h; stored as T into hc, the feed-forward residual)
//   c[t]  = g * h'[t] / sqrt(mean(h'[t]^2) + eps)     (from the stored h')
// k <= 8 (the block length).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void residual_conv_kernel(const float* __restrict__ part, int ks, int M,
                                                                     const T* __restrict__ x,
                                                                     const T* __restrict__ w_conv, int k,
                                                                     const T* __restrict__ b_conv,
                                                                     T* __restrict__ hc, const T* __restrict__ g,
                                                                     float eps, T* __restrict__ c_out) {
    __shared__ float red[8][kRowThreads / 64];
    const int64_t row0 = (int64_t)blockIdx.x * 8 * kD;
    const int c = threadIdx.x * 8;
    float h[8][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) V8<T>::load(x + row0 + t * kD + c, h[t]);
#pragma unroll
    for (int t = 0; t < 8; ++t) add_parts8(part, ks, (int64_t)M * kD, row0 + t * kD + c, h[t]);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) h[t][e] = round_as<T>(h[t][e]);
    float bv[8];
    V8<T>::load(b_conv + c, bv);
    float y[8][8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) y[t][e] = bv[e];
#pragma unroll
    for (int j = 0; j < 8; ++j) {          // unrolled to the block length: static register indices
        if (j >= k) break;
        float wv[8];
        V8<T>::load(w_conv + (int64_t)j * kD + c, wv);
#pragma unroll
        for (int t = j; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) y[t][e] += wv[e] * h[t - j][e];
    }
    float ss[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        ss[t] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[t][e] = h[t][e] + y[t][e];
        }
        V8<T>::store(hc + row0 + t * kD + c, y[t]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[t][e] = round_as<T>(y[t][e]);
            ss[t] += y[t][e] * y[t][e];
        }
        ss[t] = wave_sum(ss[t]);
    }
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int t = 0; t < 8; ++t) red[t][threadIdx.x >> 6] = ss[t];
    __syncthreads();
    float gv[8];
    V8<T>::load(g + c, gv);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float tot = red[t][0] + red[t][1] + red[t][2] + red[t][3] + red[t][4];
        const float rinv = 1.0f / sqrtf(tot * (1.0f / kD) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[t][e] = gv[e] * y[t][e] * rinv;
        V8<T>::store(c_out + row0 + t * kD + c, y[t]);
    }
}

// s = silu(gate) * up from the [gate | up] partials (5120 + 5120 columns).
// 640 groups of 8 columns per row, 2 per thread.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void swiglu_kernel(const float* __restrict__ part, int ks, int M,
                                                              T* __restrict__ s) {
    const int m = blockIdx.x;
    const int64_t stride = (int64_t)M * 2 * kInter, row = (int64_t)m * 2 * kInter;
    float gate[2][8] = {}, up[2][8] = {};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 8 * (threadIdx.x + kRowThreads * i);
        add_parts8(part, ks, stride, row + c, gate[i]);
        add_parts8(part, ks, stride, row + kInter + c, up[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gate[i][e] = gate[i][e] / (1.0f + expf(-gate[i][e])) * up[i][e];
        V8<T>::store(s + (int64_t)m * kInter + 8 * (threadIdx.x + kRowThreads * i), gate[i]);
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t esize(int dtype) { return dtype == DFLASH_BF16 ? 2 : 4; }

GemmParams gemm_params(const void* a, int a_stride, const void* w, int M, int N, int K, int ks, int dtype,
                       float* part) {
    GemmParams g = {};
    g.aseg[0] = a;
    g.a_stride = a_stride;
    g.seg_w = K;
    g.b = w;
    g.M = M; g.N = N; g.K = K;
    g.part = part;
    gemm_set_split(g, dtype, ks);
    return g;
}

template <typename T>
hipError_t run_qkv(const dflash_qkv_args& a, const DraftQkvPlan& pl, char* ws, hipStream_t s) {
    const int M = 8 * a.B;
    T* an = reinterpret_cast<T*>(ws + pl.off_a);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    norm_rows_kernel<T><<<M, kRowThreads, 0, s>>>(static_cast<const T*>(a.x), static_cast<const T*>(a.g_in), a.eps,
                                                  an);
    const GemmParams g = gemm_params(an, kD, a.w_qkv, M, kQkvN, kD, pl.ks, a.dtype, part);
    if (pl.pair) {
        QkvEpilogue qe;
        qe.q = static_cast<uint16_t*>(a.q);
        qe.k = static_cast<uint16_t*>(a.k_blk);
        qe.v = static_cast<uint16_t*>(a.v_blk);
        return launch_gemm_pair_qkv(g, qe, s);
    }
    hipError_t e = launch_gemm(g, a.dtype, s);
    if (e != hipSuccess) return e;
    qkv_scatter_kernel<T><<<M, kThreads, 0, s>>>(part, g.ks, M, static_cast<T*>(a.q), static_cast<T*>(a.k_blk),
                                                 static_cast<T*>(a.v_blk));
    return hipGetLastError();
}

template <typename T>
hipError_t run_mlp(const dflash_mlp_args& a, const DraftMlpPlan& pl, char* ws, hipStream_t s) {
    const int M = 8 * a.B;
    T* ao = reinterpret_cast<T*>(ws + pl.off_ao);
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    // The feed-forward residual (h, or h' with the convolution) lives in h_out
    // when the caller wants a copy, else in the workspace.
    T* h = a.h_out ? static_cast<T*>(a.h_out) : reinterpret_cast<T*>(ws + pl.off_h);
    T* c = reinterpret_cast<T*>(ws + pl.off_c);
    T* sw = reinterpret_cast<T*>(ws + pl.off_s);
    hipError_t e;

    heads_to_rows_kernel<T><<<M, kThreads, 0, s>>>(static_cast<const T*>(a.o), ao);
    const GemmParams g1 = gemm_params(ao, kQN, a.w_o, M, kD, kQN, pl.ks_o, a.dtype, part);
    if ((e = launch_gemm(g1, a.dtype, s)) != hipSuccess) return e;
    if (a.conv_k > 0)
        residual_conv_kernel<T><<<a.B, kRowThreads, 0, s>>>(part, g1.ks, M, static_cast<const T*>(a.x),
                                                          static_cast<const T*>(a.w_conv), a.conv_k,
                                                          static_cast<const T*>(a.b_conv), h,
                                                          static_cast<const T*>(a.g_post), a.eps, c);
    else
        residual_kernel<T><<<M, kRowThreads, 0, s>>>(part, g1.ks, M, static_cast<const T*>(a.x), h,
                                                   static_cast<const T*>(a.g_post), a.eps, c);

    // gate/up: unsplit bf16 products go straight through the SwiGLU epilogue;
    // split-K (few rows) or fp32 products through the partials and swiglu_kernel.
    GemmParams g2 = gemm_params(c, kD, a.w_gu, M, 2 * kInter, kD, pl.ks_gu, a.dtype, part);
    const bool fused = a.dtype == DFLASH_BF16 && g2.ks == 1;
    if (fused) g2.swiglu_out = reinterpret_cast<uint16_t*>(sw);
    if ((e = launch_gemm(g2, a.dtype, s)) != hipSuccess) return e;
    if (!fused) swiglu_kernel<T><<<M, kRowThreads, 0, s>>>(part, g2.ks, M, sw);

    const GemmParams g3 = gemm_params(sw, kInter, a.w_d, M, kD, kInter, pl.ks_d, a.dtype, part);
    if ((e = launch_gemm(g3, a.dtype, s)) != hipSuccess) return e;
    residual_kernel<T><<<M, kRowThreads, 0, s>>>(part, g3.ks, M, h, static_cast<T*>(a.x_out),
                                               static_cast<const T*>(a.g_final), a.eps, static_cast<T*>(a.y_out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_embed(const dflash_embed_args& a, hipStream_t s) {
    if (a.dtype == DFLASH_BF16)
        embed_kernel<uint16_t><<<8 * a.B, kRowThreads, 0, s>>>(static_cast<const uint16_t*>(a.emb), a.V, a.anchor,
                                                             a.mask_id, static_cast<uint16_t*>(a.x));
    else
        embed_kernel<float><<<8 * a.B, kRowThreads, 0, s>>>(static_cast<const float*>(a.emb), a.V, a.anchor, a.mask_id,
                                                          static_cast<float*>(a.x));
    return hipGetLastError();
}

DraftQkvPlan draft_qkv_plan(const dflash_qkv_args& a) {
    DraftQkvPlan pl;
    const int M = 8 * a.B;
    const bool bf = a.dtype == DFLASH_BF16;
    pl.ks = bf ? gemm_split(M, kQkvN, kD) : 1;
    // Where the split-K kernel would run two splits (one residency round of
    // two 4-wave workgroups per CU), one 8-wave workgroup per tile takes both
    // halves of k and writes the head layout itself: the same sums, no fp32
    // partials and no scatter launch.
    pl.pair = bf && pl.ks == 2 && ((M + 127) / 128) * (kQkvN / 128) <= 256;
    if (pl.pair) pl.ks = 1;
    pl.off_a = 0;
    pl.off_part = align256((size_t)M * kD * esize(a.dtype));
    pl.ws_bytes = pl.off_part + (pl.pair ? 0 : align256((size_t)pl.ks * M * kQkvN * 4));
    return pl;
}

hipError_t launch_draft_qkv(const dflash_qkv_args& a, const DraftQkvPlan& pl, void* ws, hipStream_t s) {
    char* w = static_cast<char*>(ws);
    return a.dtype == DFLASH_BF16 ? run_qkv<uint16_t>(a, pl, w, s) : run_qkv<float>(a, pl, w, s);
}

DraftMlpPlan draft_mlp_plan(const dflash_mlp_args& a) {
    DraftMlpPlan pl;
    const int M = 8 * a.B;
    const bool bf = a.dtype == DFLASH_BF16;
    const size_t es = esize(a.dtype);
    pl.ks_o = bf ? gemm_split(M, kD, kQN) : 1;
    pl.ks_gu = bf ? gemm_split(M, 2 * kInter, kD) : 1;
    pl.ks_d = bf ? gemm_split(M, kD, kInter) : 1;
    size_t part = (size_t)pl.ks_o * M * kD;
    if ((size_t)pl.ks_gu * M * 2 * kInter > part) part = (size_t)pl.ks_gu * M * 2 * kInter;
    if ((size_t)pl.ks_d * M * kD > part) part = (size_t)pl.ks_d * M * kD;
    pl.off_ao = 0;
    pl.off_part = align256((size_t)M * kQN * es);
    pl.off_h = pl.off_part + align256(part * 4);
    pl.off_c = pl.off_h + align256((size_t)M * kD * es);
    pl.off_s = pl.off_c + align256((size_t)M * kD * es);
    pl.ws_bytes = pl.off_s + align256((size_t)M * kInter * es);
    return pl;
}

hipError_t launch_draft_mlp(const dflash_mlp_args& a, const DraftMlpPlan& pl, void* ws, hipStream_t s) {
    char* w = static_cast<char*>(ws);
    return a.dtype == DFLASH_BF16 ? run_mlp<uint16_t>(a, pl, w, s) : run_mlp<float>(a, pl, w, s);
}

}  // namespace dflash
