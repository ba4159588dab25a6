// Block-mask builder: exact 128x128 tile classification of a mask predicate
// and compaction of the non-empty tiles into per-row and per-column lists.
//
// What is built (speedrun notes "FlexAttention", tile-summary paragraph;
// tutorial "FlexAttention in PyTorch", "The two hooks"): for every row of
// query tiles, the number of tiles that are not fully masked and their
// column indices, split into partial and full tiles; the same per column of
// key tiles for the backward pass.  A tile's class follows from the exact
// count of visible (q, kv) pairs in it.
//
// How it is computed on gfx950:
//  * For non-decreasing document ids (packed documents as the running count of
//    end-of-text flags, speedrun notes code listing) the visible keys of query
//    q form at most two intervals: the main one [lo(q), hi(q)] with
//    lo = max(doc start, q - window + 1) and hi = min(doc end, q or T-1), and
//    a sink interval [doc start, min(sinks - 1, hi)].  A tile's pair count is
//    then a sum of 128 interval overlaps -- exact, O(128) per tile.
//  * Any other document ids take a general path that compares document ids
//    key by key inside the causal/window intervals (still exact).
//  * The document range [start, end] of every position is exported
//    (doc_range) so the attention kernels can mask partial tiles with two
//    interval compares per score; (-1, -1) marks rows without contiguous
//    documents.
//  * One workgroup per query-tile row; one lane per key tile; wave ballots and
//    a cross-wave prefix sum compact the partial and full lists in ascending
//    order.  A per-tile class byte is kept in the workspace and a second
//    kernel compacts it per key-tile column the same way.
#include "bsm_internal.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ inline int64_t overlap(int64_t lo, int64_t hi, int64_t k0, int64_t k1) {
    int64_t a = lo > k0 ? lo : k0;
    int64_t b = hi < k1 ? hi : k1;
    return b >= a ? (b - a + 1) : 0;
}

// First index t in [lo, hi) with doc[t] >= val (doc non-decreasing).
__device__ inline int lower_bound_doc(const int32_t *doc, int lo, int hi, int32_t val) {
    while (lo < hi) {
        int mid = lo + ((hi - lo) >> 1);
        if (doc[mid] < val) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// First index t in [lo, hi) with doc[t] > val (doc non-decreasing).
__device__ inline int upper_bound_doc(const int32_t *doc, int lo, int hi, int32_t val) {
    while (lo < hi) {
        int mid = lo + ((hi - lo) >> 1);
        if (doc[mid] <= val) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// nonmono[b][c] = 1 if doc[t] > doc[t + 1] for some t in chunk c.
__global__ __launch_bounds__(kThreads) void check_monotone_kernel(MaskBuildParams p) {
    const int b = blockIdx.y;
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const int32_t *doc = p.doc_ids + (int64_t)b * p.T;
    int bad = 0;
    if (t + 1 < p.T) bad = doc[t] > doc[t + 1];
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) p.nonmono[(int64_t)b * p.nchunks + blockIdx.x] = bad;
}

// Compacts one chunk of up to 256 class decisions (one per thread, in
// ascending column order across threads) into the partial / full lists.
// `run_p`/`run_f` carry the running counts across chunks.
__device__ inline void compact_chunk(bool is_p, bool is_f, int col, int32_t *idx_p,
                                     int32_t *idx_f, int &run_p, int &run_f,
                                     int *s_wp, int *s_wf) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const unsigned long long bp = __ballot(is_p);
    const unsigned long long bf = __ballot(is_f);
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pp = __popcll(bp & lt);
    const int pf = __popcll(bf & lt);
    if (lane == 0) {
        s_wp[wv] = __popcll(bp);
        s_wf[wv] = __popcll(bf);
    }
    __syncthreads();
    int off_p = run_p, off_f = run_f, tot_p = 0, tot_f = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wv) {
            off_p += s_wp[w];
            off_f += s_wf[w];
        }
        tot_p += s_wp[w];
        tot_f += s_wf[w];
    }
    if (is_p) idx_p[off_p + pp] = col;
    if (is_f) idx_f[off_f + pf] = col;
    run_p += tot_p;
    run_f += tot_f;
    __syncthreads();  // s_wp / s_wf are rewritten by the next chunk
}

__device__ inline void pad_tail(int32_t *idx, int from, int n) {
    for (int s = from + (int)threadIdx.x; s < n; s += kThreads) idx[s] = -1;
}

__global__ __launch_bounds__(kThreads) void rows_kernel(MaskBuildParams p) {
    __shared__ int64_t s_alo[kTile], s_ahi[kTile], s_blo[kTile], s_bhi[kTile];
    __shared__ int32_t s_docq[kTile];
    __shared__ int s_wp[kWaves], s_wf[kWaves];
    __shared__ long long s_amin, s_amax, s_bmin, s_bmax;

    const int i = blockIdx.x;
    const int b = blockIdx.y;
    const int T = p.T;
    const int nt = p.nt;
    const bool causal = p.flags & BSM_MASK_CAUSAL;
    const bool document = p.flags & BSM_MASK_DOCUMENT;
    const bool windowed = p.flags & BSM_MASK_WINDOW;
    const bool sinks_on = windowed && (p.flags & BSM_MASK_SINKS) && p.sinks > 0;
    const int32_t *doc = document ? p.doc_ids + (int64_t)b * T : nullptr;

    bool mono = true;
    if (document) {
        int bad = 0;
        for (int c = threadIdx.x; c < p.nchunks; c += kThreads)
            bad |= p.nonmono[(int64_t)b * p.nchunks + c];
        mono = !__syncthreads_or(bad);
    }
    const bool general = document && !mono;  // per-key document compare
    const int64_t w = windowed ? (int64_t)(*p.window) : 0;

    if (threadIdx.x == 0) {
        s_amin = INT64_MAX; s_amax = INT64_MIN;
        s_bmin = INT64_MAX; s_bmax = INT64_MIN;
    }
    __syncthreads();
    if (threadIdx.x < kTile) {
        const int r = threadIdx.x;
        const int q = i * kTile + r;
        int64_t ds = 0, de = T - 1;
        if (document) {
            const int32_t dq = doc[q];
            s_docq[r] = dq;
            if (mono) {
                ds = lower_bound_doc(doc, 0, q + 1, dq);
                de = upper_bound_doc(doc, q, T, dq) - 1;
            }
        }
        int64_t hi = causal ? (int64_t)q : (int64_t)(T - 1);
        if (de < hi) hi = de;
        int64_t lo = ds;
        if (windowed && q - w + 1 > lo) lo = q - w + 1;
        int64_t blo = 1, bhi = 0;  // empty
        if (sinks_on) {
            blo = ds;
            bhi = (int64_t)p.sinks - 1 < hi ? (int64_t)p.sinks - 1 : hi;
        }
        if (document) {
            int32_t *dr = p.out.doc_range + ((int64_t)b * T + q) * 2;
            dr[0] = mono ? (int32_t)ds : -1;
            dr[1] = mono ? (int32_t)de : -1;
        }
        s_alo[r] = lo; s_ahi[r] = hi;
        s_blo[r] = blo; s_bhi[r] = bhi;
        if (lo <= hi) {
            atomicMin(&s_amin, (long long)lo);
            atomicMax(&s_amax, (long long)hi);
        }
        if (blo <= bhi) {
            atomicMin(&s_bmin, (long long)blo);
            atomicMax(&s_bmax, (long long)bhi);
        }
    }
    __syncthreads();
    const int64_t amin = s_amin, amax = s_amax, bmin = s_bmin, bmax = s_bmax;

    const int64_t row_off = ((int64_t)b * nt + i) * nt;
    int32_t *idx_p = p.out.kv_indices + row_off;
    int32_t *idx_f = p.out.full_kv_indices + row_off;
    uint8_t *cls_row = p.cls + row_off;
    int run_p = 0, run_f = 0;

    for (int jb = 0; jb < nt; jb += kThreads) {
        const int j = jb + threadIdx.x;
        uint8_t c = kEmpty;
        if (j < nt) {
            const int64_t k0 = (int64_t)j * kTile, k1 = k0 + kTile - 1;
            const bool cand = (amin <= k1 && amax >= k0) || (bmin <= k1 && bmax >= k0);
            if (cand) {
                int64_t n = 0;
                if (!general) {
                    for (int r = 0; r < kTile; ++r) {
                        const int64_t alo = s_alo[r], ahi = s_ahi[r];
                        n += overlap(alo, ahi, k0, k1);
                        if (sinks_on) {
                            const int64_t blo = s_blo[r], bhi = s_bhi[r];
                            n += overlap(blo, bhi, k0, k1);
                            n -= overlap(alo > blo ? alo : blo, ahi < bhi ? ahi : bhi, k0, k1);
                        }
                    }
                } else {
                    for (int r = 0; r < kTile; ++r) {
                        const int32_t dq = s_docq[r];
                        const int64_t alo = s_alo[r], ahi = s_ahi[r];
                        const int64_t a0 = alo > k0 ? alo : k0, a1 = ahi < k1 ? ahi : k1;
                        for (int64_t kv = a0; kv <= a1; ++kv) n += (doc[kv] == dq);
                        if (sinks_on) {
                            const int64_t blo = s_blo[r], bhi = s_bhi[r];
                            const int64_t b0 = blo > k0 ? blo : k0, b1 = bhi < k1 ? bhi : k1;
                            for (int64_t kv = b0; kv <= b1; ++kv)
                                if (kv < alo || kv > ahi) n += (doc[kv] == dq);
                        }
                    }
                }
                c = n == 0 ? kEmpty : (n == kTilePairs ? kFull : kPartial);
            }
            cls_row[j] = c;
        }
        compact_chunk(c == kPartial, c == kFull, j, idx_p, idx_f, run_p, run_f, s_wp, s_wf);
    }
    pad_tail(idx_p, run_p, nt);
    pad_tail(idx_f, run_f, nt);
    if (threadIdx.x == 0) {
        p.out.kv_num_blocks[(int64_t)b * nt + i] = run_p;
        p.out.full_kv_num_blocks[(int64_t)b * nt + i] = run_f;
    }
}

__global__ __launch_bounds__(kThreads) void cols_kernel(MaskBuildParams p) {
    __shared__ int s_wp[kWaves], s_wf[kWaves];
    const int j = blockIdx.x;
    const int b = blockIdx.y;
    const int nt = p.nt;
    const uint8_t *cls = p.cls + (int64_t)b * nt * nt;
    const int64_t col_off = ((int64_t)b * nt + j) * nt;
    int32_t *idx_p = p.out.q_indices + col_off;
    int32_t *idx_f = p.out.full_q_indices + col_off;
    int run_p = 0, run_f = 0;
    for (int ib = 0; ib < nt; ib += kThreads) {
        const int i = ib + threadIdx.x;
        const uint8_t c = i < nt ? cls[(int64_t)i * nt + j] : kEmpty;
        compact_chunk(c == kPartial, c == kFull, i, idx_p, idx_f, run_p, run_f, s_wp, s_wf);
    }
    pad_tail(idx_p, run_p, nt);
    pad_tail(idx_f, run_f, nt);
    if (threadIdx.x == 0) {
        p.out.q_num_blocks[(int64_t)b * nt + j] = run_p;
        p.out.full_q_num_blocks[(int64_t)b * nt + j] = run_f;
    }
}

// Work orders: the query-tile rows (block 0) and key-tile columns (block 1)
// of every mask batch in the order the attention kernels take them.  Rows
// are grouped in blocks of kOrderBlock consecutive rows of one mask batch
// (the last block of a batch may be shorter) -- neighbouring rows read
// mostly the same key and value tiles.  Blocks go by decreasing key
// min(visible tiles of the block, kOrderKeys - 1), ties in ascending block
// index, rows inside a block in ascending order: the longest work starts
// first and short blocks fill the end of a launch.  Entry e of kv_order is
// the record (bm * nt + i, full tiles, partial tiles, first listed tile) of
// the e-th row in this order, so a kernel starts a row with one load.
//
// A counting sort of the blocks: histogram of the keys in LDS, exclusive
// scan from the largest key down, one wave places the blocks in index order
// (for each key present in a chunk of 64 blocks, the lanes holding it get
// consecutive slots in lane order), then a scan of the block sizes gives
// each block its first entry.
constexpr int kOrderThreads = 1024;
constexpr int kOrderPer = kOrderKeys / kOrderThreads;

// Exclusive prefix sum of one value per thread over the workgroup; returns
// this thread's prefix and sets total.
__device__ inline int block_exclusive_scan(int v, int *s_wsum, int &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int up = __shfl_up(incl, d);
        if (lane >= d) incl += up;
    }
    __syncthreads();  // s_wsum free from any previous use
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < kOrderThreads / 64; ++w) {
        if (w < wv) before += s_wsum[w];
        total += s_wsum[w];
    }
    return before + incl - v;
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(MaskBuildParams p) {
    __shared__ int s_hist[kOrderKeys];
    __shared__ int s_wsum[kOrderThreads / 64];
    const bool cols = blockIdx.x == 1;
    const int32_t *num = cols ? p.out.q_num_blocks : p.out.kv_num_blocks;
    const int32_t *fnum = cols ? p.out.full_q_num_blocks : p.out.full_kv_num_blocks;
    const int32_t *idx = cols ? p.out.q_indices : p.out.kv_indices;
    const int32_t *fidx = cols ? p.out.full_q_indices : p.out.full_kv_indices;
    int32_t *order = cols ? p.out.q_order : p.out.kv_order;
    int32_t *sorted = p.order_ws + (cols ? p.order_ws_stride : 0);  // block at each sorted position
    const int nt = p.nt;
    const int bpb = (nt + kOrderBlock - 1) / kOrderBlock;  // blocks per mask batch
    const int nb = p.mask_b * bpb;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    auto block_rows = [&](int g, int &r0, int &n) {
        const int bm = g / bpb, j = g - bm * bpb;
        r0 = bm * nt + j * kOrderBlock;
        n = min(kOrderBlock, nt - j * kOrderBlock);
    };
    auto key_of = [&](int g) {
        int r0, n;
        block_rows(g, r0, n);
        int tot = 0;
        for (int r = r0; r < r0 + n; ++r) tot += num[r] + fnum[r];
        return min(tot, kOrderKeys - 1);
    };

    for (int x = tid; x < kOrderKeys; x += kOrderThreads) s_hist[x] = 0;
    __syncthreads();
    for (int g = tid; g < nb; g += kOrderThreads) atomicAdd(&s_hist[key_of(g)], 1);
    __syncthreads();
    // Thread t owns keys kOrderKeys-1-kOrderPer*t down to kOrderKeys-kOrderPer*(t+1).
    int v[kOrderPer], sum = 0;
#pragma unroll
    for (int x = 0; x < kOrderPer; ++x) {
        v[x] = s_hist[kOrderKeys - 1 - (kOrderPer * tid + x)];
        sum += v[x];
    }
    int total;
    int start = block_exclusive_scan(sum, s_wsum, total);
#pragma unroll
    for (int x = 0; x < kOrderPer; ++x) {
        s_hist[kOrderKeys - 1 - (kOrderPer * tid + x)] = start;  // first slot of the key
        start += v[x];
    }
    __syncthreads();
    if (wv == 0) {
        for (int g0 = 0; g0 < nb; g0 += 64) {
            const int g = g0 + lane;
            const int key = g < nb ? key_of(g) : -1;
            unsigned long long todo = __ballot(g < nb);
            while (todo) {
                const int src = __builtin_ctzll(todo);
                const int kk = __shfl(key, src);
                const unsigned long long same = __ballot(key == kk);
                const int base = s_hist[kk];
                if (key == kk) sorted[base + __builtin_popcountll(same & ((1ull << lane) - 1))] = g;
                __builtin_amdgcn_wave_barrier();
                if (lane == src) s_hist[kk] = base + __builtin_popcountll(same);
                __builtin_amdgcn_wave_barrier();
                todo &= ~same;
            }
        }
    }
    __threadfence_block();
    __syncthreads();
    // Entries of the rows of each block, in sorted block order.
    int run = 0;  // entries before the current chunk of sorted positions
    for (int pos0 = 0; pos0 < nb; pos0 += kOrderThreads) {
        const int pos = pos0 + tid;
        int r0 = 0, n = 0;
        if (pos < nb) block_rows(sorted[pos], r0, n);
        int chunk_total;
        const int first = run + block_exclusive_scan(n, s_wsum, chunk_total);
        for (int x = 0; x < n; ++x) {
            const int e = r0 + x;
            const int nf = fnum[e], np = num[e];
            const int ft = nf > 0 ? fidx[(int64_t)e * nt] : (np > 0 ? idx[(int64_t)e * nt] : 0);
            int4 rec;
            rec.x = e;
            rec.y = nf;
            rec.z = np;
            rec.w = ft;
            reinterpret_cast<int4 *>(order)[first + x] = rec;
        }
        run += chunk_total;
    }
}

}  // namespace

hipError_t launch_build_block_mask(const MaskBuildParams &p, hipStream_t stream) {
    if (p.flags & BSM_MASK_DOCUMENT) {
        hipLaunchKernelGGL(check_monotone_kernel, dim3(p.nchunks, p.mask_b), dim3(kThreads), 0,
                           stream, p);
    }
    hipLaunchKernelGGL(rows_kernel, dim3(p.nt, p.mask_b), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(cols_kernel, dim3(p.nt, p.mask_b), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(order_kernel, dim3(2), dim3(kOrderThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace bsm
