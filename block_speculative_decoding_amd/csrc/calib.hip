// Calibration kernels: the practical ceilings the roofline fractions are read
// against, measured on the part that runs the hot path (gfx950).
//
//   stream_read  -- every byte of a buffer read once with 16-byte
//                   nontemporal loads (the faster form for data read once),
//                   eight in flight per thread, each workgroup reading 32 KiB
//                   contiguous runs (grid given, 2048 by default); a
//                   per-workgroup xor of the data goes to a sink so the
//                   loads are not dead.
//   stream_copy  -- the same loads, each stored to a second buffer.
//   gather_read  -- chunks of a buffer read in the order of a list of chunk
//                   ids (a random permutation gives the page-like pattern of
//                   the paged KV cache), 4-KiB pieces, eight in flight per
//                   thread; ids outside the buffer read nothing.
//   mfma_loop    -- bf16 32x32x16 matrix instructions on register operands
//                   only (no memory in the loop), eight independent
//                   accumulators per wave, two waves per SIMD.
#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalUnroll = 8;
constexpr int kCalMaxGrid = 65536;

// Each workgroup reads runs of kCalUnroll * 4 KiB: load u of a thread is
// 4 KiB past load u - 1, so a wave's loads cover whole contiguous runs.
template <bool COPY>
__global__ __launch_bounds__(kCalThreads) void stream_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             int64_t n16, uint4* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kCalThreads * kCalUnroll;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i = (int64_t)blockIdx.x * kCalThreads * kCalUnroll + threadIdx.x; i < n16; i += stride) {
        uint4 v[kCalUnroll];
#pragma unroll
        for (int u = 0; u < kCalUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kCalThreads;
            v[u] = j < n16 ? ld_stream(src + j) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kCalUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kCalThreads;
            if (COPY && j < n16) dst[j] = v[u];
            x.x ^= v[u].x; x.y ^= v[u].y; x.z ^= v[u].z; x.w ^= v[u].w;
        }
    }
    // xor over the workgroup, one 16-byte result per workgroup
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        x.x ^= __shfl_xor(x.x, o); x.y ^= __shfl_xor(x.y, o);
        x.z ^= __shfl_xor(x.z, o); x.w ^= __shfl_xor(x.w, o);
    }
    __shared__ uint4 red[kCalThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kCalThreads / 64; ++w) {
            x.x ^= red[w].x; x.y ^= red[w].y; x.z ^= red[w].z; x.w ^= red[w].w;
        }
        sink[blockIdx.x] = x;
    }
}

// Piece p (4 KiB) of the list is piece p % ppc of chunk ids[p / ppc]; load u
// of a thread reads 16 bytes of piece p0 + u, so a wave's load is one
// contiguous 1-KiB run and a workgroup's eight loads cover 32 KiB.
__global__ __launch_bounds__(kCalThreads) void gather_kernel(const uint4* __restrict__ src, int64_t n16,
                                                             const int32_t* __restrict__ ids, int64_t nchunks,
                                                             int ppc, uint4* __restrict__ sink) {
    const int64_t npieces = nchunks * ppc;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t p0 = (int64_t)blockIdx.x * kCalUnroll; p0 < npieces; p0 += (int64_t)gridDim.x * kCalUnroll) {
        uint4 v[kCalUnroll];
#pragma unroll
        for (int u = 0; u < kCalUnroll; ++u) {
            const int64_t pc = p0 + u;
            v[u] = make_uint4(0u, 0u, 0u, 0u);
            if (pc < npieces) {
                const int64_t id = ids[pc / ppc];
                const int64_t j = (id * ppc + pc % ppc) * kCalThreads + threadIdx.x;
                if (id >= 0 && j < n16) v[u] = ld_stream(src + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kCalUnroll; ++u) {
            x.x ^= v[u].x; x.y ^= v[u].y; x.z ^= v[u].z; x.w ^= v[u].w;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        x.x ^= __shfl_xor(x.x, o); x.y ^= __shfl_xor(x.y, o);
        x.z ^= __shfl_xor(x.z, o); x.w ^= __shfl_xor(x.w, o);
    }
    __shared__ uint4 red[kCalThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kCalThreads / 64; ++w) {
            x.x ^= red[w].x; x.y ^= red[w].y; x.z ^= red[w].z; x.w ^= red[w].w;
        }
        sink[blockIdx.x] = x;
    }
}

constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kCalThreads) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(int64_t)blockIdx.x * kCalThreads + threadIdx.x] = s;
}

}  // namespace

int calib_stream_max_grid() { return kCalMaxGrid; }
int calib_mfma_grid() { return 256 * 2; }   // 4 waves per workgroup: two per SIMD on 256 CUs

hipError_t launch_calib_stream(const void* src, void* dst, size_t bytes, int grid, void* sink, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (grid <= 0) grid = 2048;
    if (dst)
        stream_kernel<true><<<grid, kCalThreads, 0, s>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16,
                                                         static_cast<uint4*>(sink));
    else
        stream_kernel<false><<<grid, kCalThreads, 0, s>>>(static_cast<const uint4*>(src), nullptr, n16,
                                                          static_cast<uint4*>(sink));
    return hipGetLastError();
}

hipError_t launch_calib_gather(const void* src, size_t bytes, const int32_t* ids, int64_t nchunks, int chunk_bytes,
                               int grid, void* sink, hipStream_t s) {
    if (grid <= 0) grid = 2048;
    gather_kernel<<<grid, kCalThreads, 0, s>>>(static_cast<const uint4*>(src), (int64_t)(bytes / 16), ids, nchunks,
                                               chunk_bytes / 4096, static_cast<uint4*>(sink));
    return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, void* sink, hipStream_t s) {
    mfma_loop_kernel<<<calib_mfma_grid(), kCalThreads, 0, s>>>(iters, static_cast<float*>(sink));
    return hipGetLastError();
}

}  // namespace dflash
