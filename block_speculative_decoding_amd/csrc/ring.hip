// Sliding-window draft cache kept as a ring of pages (gfx950).
//
// "Nemotron 3.5 Bolt E4B: Block-Parallel Speculation with DFlash", sections
// "Five target states become persistent draft context" (the drafter attends to
// the latest 1,024 tokens) and "Cache and latency have separate break-even
// points" (a 20 MiB window payload per sequence).  Logical page p of a
// sequence is physical page ring[p mod R]; with the slot t % 16 kept, the ring
// holds the latest 16 R tokens, so R = ceil(W / 16) pages cover a W-token
// window.  This launch turns the rows a cycle verified into cache slots and
// positions for dflash_ctx_fuse and advances the context lengths, all on the
// device (the row counts come from verification's out_len).
#include "device_common.h"
#include "kernels.h"

namespace dflash {
namespace {

// One wave per sequence: lane j < rows_per_seq describes row rows_per_seq*b + j.
__global__ __launch_bounds__(64) void ring_append_kernel(const int32_t* __restrict__ ring, int R,
                                                         int32_t* ctx_len, const int32_t* __restrict__ n_new,
                                                         int rows_per_seq, int64_t* __restrict__ slot,
                                                         int32_t* __restrict__ pos) {
    const int b = blockIdx.x, j = threadIdx.x;
    const int S = ctx_len[b];
    const int n = min(max(n_new[b], 0), rows_per_seq);
    if (j < rows_per_seq) {
        const int64_t row = (int64_t)b * rows_per_seq + j;
        if (j < n) {
            const int t = S + j;
            slot[row] = (int64_t)ring[(int64_t)b * R + (t >> 4) % R] * 16 + (t & 15);
            pos[row] = t;
        } else {
            slot[row] = -1;
            pos[row] = 0;
        }
    }
    if (j == 0) ctx_len[b] = S + n;  // every lane has read ctx_len[b] above
}

}  // namespace

hipError_t launch_ring_append(const dflash_ring_args& a, hipStream_t s) {
    ring_append_kernel<<<a.B, 64, 0, s>>>(a.ring, a.ring_pages, a.ctx_len, a.n_new, a.rows_per_seq, a.slot, a.pos);
    return hipGetLastError();
}

}  // namespace dflash
