// Gathers the live keys and values of a paged cache into contiguous rows,
// for gfx950.
//
// Method (tutorial "FlexAttention in PyTorch", section "Decoding and paged
// KV caches"): a paged cache holds each sequence's keys in fixed-size pages of
// a shared pool, reached through a block table.  The single-query decoding
// step reads the pages in place; a block of several new queries runs the
// rectangular forward, which takes contiguous K and V, so the first n_keys
// keys of every sequence are first copied out of their pages.
//
// Mapping: one workgroup of 256 lanes per (batch x head, 64-key block); the
// block's rows go out as 16-byte pieces, consecutive lanes on consecutive
// pieces of a row (whole 128-byte lines per 8 lanes), K and V in the same
// pass.  The copy is HBM-bound: 2 x n_keys x D x 2 bytes read and written
// per (batch, head).
#include "bsm_internal.hpp"

namespace bsm {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherRows = 64;

__global__ __launch_bounds__(kGatherThreads) void gather_pages_kernel(GatherLaunch g) {
    const int bh = blockIdx.x, blk = blockIdx.y;
    const int b = bh / g.H, h = bh - b * g.H;
    const int pieces = g.row_bytes / 16;  // 16-byte pieces per row
    const int key0 = blk * kGatherRows;
    const int nrows = min(kGatherRows, g.n_keys - key0);
    // rows key0 .. key0 + 63 lie in one page (page sizes are multiples of 64);
    // an out-of-range table entry is clamped into the pool
    const int pg = min(max(g.table[(int64_t)b * g.table_stride + key0 / g.page_size], 0), g.num_pages - 1);
    const int64_t r0 = key0 % g.page_size;
    const char *ks = g.k_src + pg * g.ks_b + h * g.ks_h + r0 * g.ks_t;
    const char *vs = g.v_src + pg * g.vs_b + h * g.vs_h + r0 * g.vs_t;
    char *kd = g.k_dst + b * g.kd_b + h * g.kd_h + (int64_t)key0 * g.kd_t;
    char *vd = g.v_dst + b * g.vd_b + h * g.vd_h + (int64_t)key0 * g.vd_t;
    for (int i = threadIdx.x; i < nrows * pieces; i += kGatherThreads) {
        const int r = i / pieces, c = (i - r * pieces) * 16;
        const uint4 kv = *reinterpret_cast<const uint4 *>(ks + r * g.ks_t + c);
        const uint4 vv = *reinterpret_cast<const uint4 *>(vs + r * g.vs_t + c);
        *reinterpret_cast<uint4 *>(kd + r * g.kd_t + c) = kv;
        *reinterpret_cast<uint4 *>(vd + r * g.vd_t + c) = vv;
    }
}

}  // namespace

hipError_t launch_gather_pages(const GatherLaunch &g, hipStream_t stream) {
    const dim3 grid(g.B * g.H, (g.n_keys + kGatherRows - 1) / kGatherRows), block(kGatherThreads);
    hipLaunchKernelGGL(gather_pages_kernel, grid, block, 0, stream, g);
    return hipGetLastError();
}

}  // namespace bsm
