// Device-side helpers shared by the DFlash kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Natural log through the hardware log2 (v_log_f32, about 1 ulp for normal
// inputs): x must be a positive normal float.
__device__ __forceinline__ float fast_ln(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// bfloat16 is stored as raw uint16 bits; widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even narrowing of a finite fp32 value to bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Low / high bf16 of a 32-bit word widened to fp32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// 16-byte load with the nontemporal hint (global_load_dwordx4 ... nt), for
// data streamed once from HBM (cache pages, logit rows).  On gfx950 such
// loads stream about 13% faster than plain ones (7.1 against 6.25 TB/s for a
// read of 4 GiB, measured by the calibration kernels), and they do not evict
// data that is reused.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Element loads for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {  // bf16 bits
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
        return bf16_bits_to_f32(p[i]);
    }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) {
        p[i] = (uint16_t)f32_to_bf16_bits(v);
    }
};

// ---- Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) ----
struct U64x4 { uint64_t x0, x1, x2, x3; };

// Full 64x64 -> 128-bit product from four 32x32+64 multiply-adds
// (v_mad_u64_u32): x*M = (p3 + hi32(p2))*2^64 + lo32(p2)*2^32 + lo32(p0), the
// partial sums chained so that none overflows 64 bits.
__device__ __forceinline__ void mulhilo64(uint64_t m, uint64_t x, uint64_t& hi, uint64_t& lo) {
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
    const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
    const uint64_t p0 = (uint64_t)xl * ml;
    const uint64_t p1 = (uint64_t)xh * ml + (p0 >> 32);
    const uint64_t p2 = (uint64_t)xl * mh + (uint32_t)p1;
    const uint64_t p3 = (uint64_t)xh * mh + (p1 >> 32);
    hi = p3 + (p2 >> 32);
    lo = (p2 << 32) | (uint32_t)p0;
}

__device__ __forceinline__ U64x4 philox4x64_10(U64x4 c, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c.x0, hi0, lo0);
        mulhilo64(M1, c.x2, hi1, lo1);
        U64x4 n;
        n.x0 = hi1 ^ c.x1 ^ k0;
        n.x1 = lo1;
        n.x2 = hi0 ^ c.x3 ^ k1;
        n.x3 = lo0;
        c = n;
        k0 += W0;
        k1 += W1;
    }
    return c;
}

// u = (bits + 0.5) * 2^-23 of a word's top 23 bits (half 0: bits 41..63) or
// of its low word's top 23 bits (half 1: bits 9..31): exact in fp32,
// strictly inside (0, 1).
__device__ __forceinline__ float word_to_uniform(uint64_t w) {
    return ((float)(uint32_t)(w >> 41) + 0.5f) * 1.1920928955078125e-07f;
}
__device__ __forceinline__ float word_to_uniform_lo(uint64_t w) {
    return ((float)(((uint32_t)w >> 9) & 0x7FFFFFu) + 0.5f) * 1.1920928955078125e-07f;
}

// ---- wave64 reductions ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Cross-lane moves through DPP (no LDS round trip): lanes a row mask leaves
// out, or whose source lane does not exist, receive the identity `id`.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float x, float id) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, x),
                                                                 CTRL, ROWS, 0xf, false));
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_i(int x, int id) {
    return __builtin_amdgcn_update_dpp(id, x, CTRL, ROWS, 0xf, false);
}
// The reduction order: swap within pairs, within quads, mirror within
// half-rows and rows (every lane of a 16-lane row then holds the row's
// result), then row 1 <- lane 15 and row 3 <- lane 47 (row_bcast:15, rows 1
// and 3), row 3 <- lane 31 (row_bcast:31, rows 2 and 3): lane 63 ends with
// the wave's result, read back as a uniform value.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

}  // namespace dflash
