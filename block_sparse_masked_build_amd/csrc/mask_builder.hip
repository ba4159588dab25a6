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
//    lo = max(doc start, q - window + 1) and hi = min(doc end, max(q, prefix - 1)
//    or T-1), and
//    a sink interval [doc start, min(sinks - 1, hi)].  Merged when they touch,
//    they are disjoint with a gap, so a tile is fully visible to a query only
//    when one interval covers it and empty only when neither meets it: exact
//    classes from two interval tests per (query, tile).
//  * Document boundaries: one 64-way wave search from the tile's first query
//    back to its document start and one from its last query on to its
//    document end; every other document of the tile starts or ends inside it
//    and is found in LDS.
//  * Any other document ids take a general path that compares document ids
//    key by key inside the causal/window intervals (still exact).
//  * The document range [start, end] of every position is exported
//    (doc_range) so the attention kernels can mask partial tiles with two
//    interval compares per score; (-1, -1) marks rows without contiguous
//    documents.
//  * One workgroup per query-tile row; only the tiles between the row's lowest
//    and highest visible key are classified, 64 at a time; wave ballots merge
//    the four waves' row quarters and compact the partial and full lists in
//    ascending order.  A per-tile class byte is kept in the workspace and a
//    second kernel compacts it per key-tile column.
//  * Queries and keys may differ in number (query i at absolute position
//    q_off + i) and need not fill whole tiles: queries past Q_LEN have no
//    visible key, keys past KV_LEN are never visible, so a cut-short tile is
//    never full.
//  * A composed mask (truth table over the five terms, tutorial, Pattern 3:
//    and_masks / or_masks) has no interval structure in general: each
//    query-tile row evaluates every pair of every key tile
//    (rows_table_kernel), exact by construction.
#include "bsm_internal.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// First t in [lo, hi) with doc[t] > val (ABOVE) or doc[t] >= val (!ABOVE), or
// hi if there is none; doc is non-decreasing on [lo, hi).  All 64 lanes of a
// wave call it with the same arguments.  Each round probes 64 evenly spaced
// positions and keeps the gap in which the predicate turns true, so n
// positions take about log64(n) + 1 rounds of loads rather than log2(n)
// dependent ones.
template <bool ABOVE>
__device__ inline int wave_search_doc(const int32_t *doc, int lo, int hi, int32_t val) {
    const int lane = threadIdx.x & 63;
    while (hi - lo > 64) {
        const int step = (hi - lo + 63) >> 6;  // 64 probes cover [lo, hi)
        const int t = lo + lane * step;
        bool hit = true;                       // probes at or past hi count as hits
        if (t < hi) {
            const int32_t d = doc[t];
            hit = ABOVE ? d > val : d >= val;
        }
        const unsigned long long m = __ballot(hit);
        if (m == 0) {                          // every probe is below hi and misses
            lo += 63 * step + 1;
        } else {
            const int f = __builtin_ctzll(m);
            if (f == 0) return lo;
            const int nhi = lo + f * step;     // a hit, or past hi
            lo += (f - 1) * step + 1;          // probe f - 1 missed
            hi = nhi < hi ? nhi : hi;
        }
    }
    const int t = lo + lane;
    bool hit = true;
    if (t < hi) {
        const int32_t d = doc[t];
        hit = ABOVE ? d > val : d >= val;
    }
    const unsigned long long m = __ballot(hit);
    return m ? lo + __builtin_ctzll(m) : hi;
}

// Same searches over a short array in LDS, one lane at a time.
template <bool ABOVE>
__device__ inline int lds_search_doc(const int32_t *a, int lo, int hi, int32_t val) {
    while (lo < hi) {
        const int mid = lo + ((hi - lo) >> 1);
        if (ABOVE ? a[mid] > val : a[mid] >= val) hi = mid; else lo = mid + 1;
    }
    return lo;
}

// nonmono[b][c] = 1 if doc[t] > doc[t + 1] for some t in chunk c.
__global__ __launch_bounds__(kThreads) void check_monotone_kernel(MaskBuildParams p) {
    const int b = blockIdx.y;
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const int32_t *doc = p.doc_ids + (int64_t)b * p.npos;
    int bad = 0;
    if (t + 1 < p.npos) bad = doc[t] > doc[t + 1];
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) p.nonmono[(int64_t)b * p.nchunks + blockIdx.x] = bad;
}

// Whether batch row b's document ids are non-decreasing (every thread of
// the workgroup gets the answer).
__device__ inline bool row_monotone(const MaskBuildParams &p, int b) {
    int bad = 0;
    for (int c = threadIdx.x; c < p.nchunks; c += kThreads) bad |= p.nonmono[(int64_t)b * p.nchunks + c];
    return !__syncthreads_or(bad);
}

// doc_range of every position of a 256-position chunk: the first and last
// position of the position's document (documents are contiguous runs when
// the ids are non-decreasing), or (-1, -1) for every position of a row whose
// ids are not.  The document start of the chunk's first position and the end
// of its last come from wave searches; every other document of the chunk
// starts or ends inside it and is found in LDS.
__global__ __launch_bounds__(kThreads) void ranges_kernel(MaskBuildParams p) {
    __shared__ int32_t s_doc[kThreads];
    __shared__ int s_ds0, s_deN;
    const int b = blockIdx.y;
    const int c0 = blockIdx.x * kThreads;
    const int n = min(kThreads, p.npos - c0);  // positions in this chunk
    const int t = c0 + (int)threadIdx.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int32_t *doc = p.doc_ids + (int64_t)b * p.npos;
    int32_t *dr = p.out.doc_range + (int64_t)b * p.npos * 2;
    const bool mono = row_monotone(p, b);
    if (!mono) {
        if (t < p.npos) {
            dr[(int64_t)t * 2] = -1;
            dr[(int64_t)t * 2 + 1] = -1;
        }
        return;
    }
    const int32_t d = t < p.npos ? doc[t] : 0;
    if ((int)threadIdx.x < n) s_doc[threadIdx.x] = d;
    __syncthreads();
    if (wv == 0) {
        const int v = wave_search_doc<false>(doc, 0, c0 + 1, s_doc[0]);
        if (lane == 0) s_ds0 = v;
    } else if (wv == 1) {
        const int v = wave_search_doc<true>(doc, c0 + n - 1, p.npos, s_doc[n - 1]) - 1;
        if (lane == 0) s_deN = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < n) {
        const int r = threadIdx.x;
        const int ds = d == s_doc[0] ? s_ds0 : c0 + lds_search_doc<false>(s_doc, 1, r, d);
        const int de = d == s_doc[n - 1] ? s_deN : c0 + lds_search_doc<true>(s_doc, r + 1, n - 1, d) - 1;
        dr[(int64_t)t * 2] = ds;
        dr[(int64_t)t * 2 + 1] = de;
    }
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

constexpr int kNone = 0x7fffffff;       // lower end of an empty interval (upper end -1)
constexpr int kRowsPerWave = kTile / kWaves;  // 32

// One workgroup per query-tile row.  The 128 rows' visible keys are reduced
// to intervals in LDS; the tiles between the lowest and highest visible key
// are then classified 64 at a time, lane = tile, each wave testing a quarter
// of the rows, and wave ballots merge the quarters and compact the lists.
__global__ __launch_bounds__(kThreads) void rows_kernel(MaskBuildParams p) {
    __shared__ i32x4 s_iv[kTile];
    __shared__ int32_t s_docq[kTile];
    __shared__ i32x4 s_ext[kTile / 64];
    __shared__ unsigned long long s_any[2][kWaves], s_all[2][kWaves];

    const int i = blockIdx.x;
    const int b = blockIdx.y;
    const int T = p.T;
    const int nt = p.nkb;   // key blocks of the row lists
    const int kb = p.kb;    // their width
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool causal = p.flags & BSM_MASK_CAUSAL;
    const bool document = p.flags & BSM_MASK_DOCUMENT;
    const bool windowed = p.flags & BSM_MASK_WINDOW;
    const bool sinks_on = windowed && (p.flags & BSM_MASK_SINKS) && p.sinks > 0;
    const int32_t *doc = document ? p.doc_ids + (int64_t)b * p.npos : nullptr;
    const int64_t w = windowed ? (int64_t)(*p.window) : 0;

    const bool mono = document ? row_monotone(p, b) : true;
    const bool general = document && !mono;  // per-key document compare

    if (threadIdx.x < kTile) {
        const int r = threadIdx.x;
        const int qi = i * kTile + r;           // query index
        const bool valid = qi < p.q_len;
        const int qa = p.q_off + (valid ? qi : p.q_len - 1);  // absolute position
        int ds = 0, de = T - 1;
        int32_t dq = 0;
        if (document) {
            dq = doc[qa];
            if (mono) {
                const int32_t *dr = p.out.doc_range + ((int64_t)b * p.npos + qa) * 2;
                ds = dr[0];
                de = dr[1];
            }
        }
        s_docq[r] = dq;
        int hi = causal ? (qa > p.prefix - 1 ? qa : p.prefix - 1) : T - 1;
        if (de < hi) hi = de;
        if (T - 1 < hi) hi = T - 1;
        int64_t lo64 = ds;
        if (windowed && (int64_t)qa - w + 1 > lo64) lo64 = (int64_t)qa - w + 1;
        int lo = lo64 < T ? (int)lo64 : T;
        int blo = kNone, bhi = -1;
        if (sinks_on) {
            blo = ds;
            bhi = p.sinks - 1 < hi ? p.sinks - 1 : hi;
        }
        if (!valid || lo > hi) { lo = kNone; hi = -1; }
        if (!valid || blo > bhi) { blo = kNone; bhi = -1; }
        // Extents of the main and sink intervals over the wave's rows (empty
        // intervals are (kNone, -1) and drop out of both).
        int e0 = lo, e1 = hi, e2 = blo, e3 = bhi;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            e0 = min(e0, __shfl_xor(e0, d));
            e1 = max(e1, __shfl_xor(e1, d));
            e2 = min(e2, __shfl_xor(e2, d));
            e3 = max(e3, __shfl_xor(e3, d));
        }
        if (lane == 0) s_ext[wv] = i32x4{e0, e1, e2, e3};
        // Without per-key document tests a row sees the union of two
        // intervals; overlapping or touching ones are merged so that a tile
        // is covered by the union only when one interval covers it.
        if (!general && lo <= hi && blo <= bhi &&
            (lo > blo ? lo : blo) <= (hi < bhi ? hi : bhi) + 1) {
            lo = lo < blo ? lo : blo;
            hi = hi > bhi ? hi : bhi;
            blo = kNone;
            bhi = -1;
        }
        s_iv[r] = i32x4{lo, hi, blo, bhi};
    }
    __syncthreads();
    const i32x4 x0 = s_ext[0], x1 = s_ext[1];
    const int amin = min(x0.x, x1.x), amax = max(x0.y, x1.y);
    const int bmin = min(x0.z, x1.z), bmax = max(x0.w, x1.w);
    int jlo = nt, jhi = -1;  // tiles that can hold a visible pair
    if (amin <= amax) {
        jlo = amin / kb;
        jhi = amax / kb;
    }
    if (bmin <= bmax) {
        jlo = bmin / kb < jlo ? bmin / kb : jlo;
        jhi = bmax / kb > jhi ? bmax / kb : jhi;
    }

    const int64_t row_off = ((int64_t)b * p.nqt + i) * nt;
    int32_t *idx_p = p.out.kv_indices + row_off;
    int32_t *idx_f = p.out.full_kv_indices + row_off;
    uint8_t *cls_row = p.cls + row_off;
    for (int j = threadIdx.x; j < nt; j += kThreads)
        if (j < jlo || j > jhi) cls_row[j] = kEmpty;

    // Lane = (row group, tile): W tiles per pass and 64 / W groups splitting
    // the wave's rows, W the smallest power of two (>= 8) covering the
    // candidate tiles, at most 64.
    const int hull = jhi - jlo + 1;
    int W = 64;
    while (W > 8 && W / 2 >= hull) W >>= 1;
    const int rows_per = kRowsPerWave * W / 64;
    const int tl = lane & (W - 1);
    const int rb = wv * kRowsPerWave + (lane / W) * rows_per;
    const unsigned long long low = W == 64 ? ~0ull : (1ull << W) - 1;
    int run_p = 0, run_f = 0, buf = 0;
    for (int jc = jlo; jc <= jhi; jc += W, buf ^= 1) {
        const int j = jc + tl;
        const int k0 = j * kb, k1 = k0 + kb - 1;
        bool any = false, all = false;
        if (j <= jhi && ((amin <= k1 && amax >= k0) || (bmin <= k1 && bmax >= k0))) {
            if (!general) {
                // Sign bits: x <= k1 <=> x - k1 - 1 < 0, and so on; the two
                // tests of one interval are ANDed, the intervals ORed.
                int acc_any = 0, acc_all = -1;
#pragma unroll 4
                for (int r = rb; r < rb + rows_per; ++r) {
                    const i32x4 v = s_iv[r];
                    acc_any |= ((v.x - k1 - 1) & (k0 - 1 - v.y)) | ((v.z - k1 - 1) & (k0 - 1 - v.w));
                    acc_all &= ((v.x - k0 - 1) & (k1 - 1 - v.y)) | ((v.z - k0 - 1) & (k1 - 1 - v.w));
                }
                any = acc_any < 0;
                all = acc_all < 0;
            } else {
                all = true;
                for (int r = rb; r < rb + rows_per; ++r) {
                    const i32x4 v = s_iv[r];
                    const int32_t d = s_docq[r];
                    int n = 0;
                    const int a0 = v.x > k0 ? v.x : k0, a1 = v.y < k1 ? v.y : k1;
                    for (int kv = a0; kv <= a1; ++kv) n += doc[kv] == d;
                    const int c0 = v.z > k0 ? v.z : k0, c1 = v.w < k1 ? v.w : k1;
                    for (int kv = c0; kv <= c1; ++kv)
                        if (kv < v.x || kv > v.y) n += doc[kv] == d;
                    any |= n > 0;
                    all &= n == kb;
                }
            }
        }
        unsigned long long ba = __ballot(any), bf = __ballot(all);
        for (int sh = W; sh < 64; sh <<= 1) {  // fold the row groups onto lanes 0..W-1
            ba |= ba >> sh;
            bf &= bf >> sh;
        }
        if (lane == 0) {
            s_any[buf][wv] = ba & low;
            s_all[buf][wv] = bf & low;
        }
        __syncthreads();  // the other buffer is rewritten only after the next barrier
        unsigned long long ma = 0, mf = ~0ull;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
            ma |= s_any[buf][x];
            mf &= s_all[buf][x];
        }
        mf &= low;
        const unsigned long long mp = ma & ~mf;  // some pair visible, not all
        if (wv == 0 && lane < W && j <= jhi) {
            const unsigned long long bit = 1ull << lane, lt = bit - 1;
            if (mp & bit) idx_p[run_p + __popcll(mp & lt)] = j;
            if (mf & bit) idx_f[run_f + __popcll(mf & lt)] = j;
            cls_row[j] = (mf & bit) ? kFull : ((mp & bit) ? kPartial : kEmpty);
        }
        run_p += __popcll(mp);
        run_f += __popcll(mf);
    }
    pad_tail(idx_p, run_p, nt);
    pad_tail(idx_f, run_f, nt);
    if (threadIdx.x == 0) {
        p.out.kv_num_blocks[(int64_t)b * p.nqt + i] = run_p;
        p.out.full_kv_num_blocks[(int64_t)b * p.nqt + i] = run_f;
    }
}

// A composed mask: one workgroup per query-tile row evaluates every (query,
// key) pair of every key block, thread (key kk, row group rb) taking the
// rows rb, rb + groups, ... of the block's key kk, and a workgroup vote
// gives the block's class.  Pairs outside Q_LEN x KV_LEN are never visible.
__global__ __launch_bounds__(kThreads) void rows_table_kernel(MaskBuildParams p) {
    __shared__ int32_t s_docq[kTile];
    const int i = blockIdx.x, b = blockIdx.y;
    const int nt = p.nkb, kb = p.kb;   // key blocks of the row lists and their width
    const int groups = kThreads / kb;  // row groups: 2 (128-key blocks) or 4 (64-key blocks)
    const bool document = p.flags & BSM_MASK_DOCUMENT;
    const bool windowed = p.flags & BSM_MASK_WINDOW;
    const int sinks = (p.flags & BSM_MASK_SINKS) ? p.sinks : 0;
    const int prefix = p.prefix;
    const int64_t w = windowed ? (int64_t)(*p.window) : 0;
    const int32_t *doc = document ? p.doc_ids + (int64_t)b * p.npos : nullptr;
    const int kk = threadIdx.x % kb, rb = threadIdx.x / kb;
    if (threadIdx.x < kTile) {
        const int qi = i * kTile + threadIdx.x;
        s_docq[threadIdx.x] = document ? doc[p.q_off + (qi < p.q_len ? qi : p.q_len - 1)] : 0;
    }
    __syncthreads();
    const int64_t row_off = ((int64_t)b * p.nqt + i) * nt;
    int32_t *idx_p = p.out.kv_indices + row_off;
    int32_t *idx_f = p.out.full_kv_indices + row_off;
    uint8_t *cls_row = p.cls + row_off;
    int run_p = 0, run_f = 0;
    for (int j = 0; j < nt; ++j) {
        const int kv = j * kb + kk;
        const bool kvalid = kv < p.T;
        const int32_t dk = document && kvalid ? doc[kv] : 0;
        int any = 0, all = kvalid;
        for (int m = 0; m < kTile / groups; ++m) {
            const int r = rb + groups * m;
            const int qi = i * kTile + r;
            const int64_t qa = (int64_t)p.q_off + qi;
            const int c = qa >= kv, d = document && s_docq[r] == dk, wt = windowed && qa - kv < w;
            const int st = kv < sinks, pt = kv < prefix;
            const int vis = qi < p.q_len && kvalid && ((p.table >> (c + 2 * d + 4 * wt + 8 * st + 16 * pt)) & 1u);
            any |= vis;
            all &= vis;
        }
        any = __syncthreads_or(any);
        all = __syncthreads_and(all);
        if (threadIdx.x == 0) {
            cls_row[j] = all ? kFull : (any ? kPartial : kEmpty);
            if (all) idx_f[run_f] = j;
            else if (any) idx_p[run_p] = j;
        }
        run_f += all ? 1 : 0;
        run_p += (any && !all) ? 1 : 0;
    }
    pad_tail(idx_p, run_p, nt);
    pad_tail(idx_f, run_f, nt);
    if (threadIdx.x == 0) {
        p.out.kv_num_blocks[(int64_t)b * p.nqt + i] = run_p;
        p.out.full_kv_num_blocks[(int64_t)b * p.nqt + i] = run_f;
    }
}

__global__ __launch_bounds__(kThreads) void cols_kernel(MaskBuildParams p) {
    __shared__ int s_wp[kWaves], s_wf[kWaves];
    const int j = blockIdx.x;
    const int b = blockIdx.y;
    const int nq = p.nqt, nk = p.nkt, nkb = p.nkb;
    const uint8_t *cls = p.cls + (int64_t)b * nq * nkb;
    const int64_t col_off = ((int64_t)b * nk + j) * nq;
    int32_t *idx_p = p.out.q_indices + col_off;
    int32_t *idx_f = p.out.full_q_indices + col_off;
    int run_p = 0, run_f = 0;
    for (int ib = 0; ib < nq; ib += kThreads) {
        const int i = ib + threadIdx.x;
        uint8_t c = kEmpty;
        if (i < nq) {
            const uint8_t *row = cls + (int64_t)i * nkb;
            if (p.kb == kTile) {
                c = row[j];
            } else {
                // a 128 x 128 tile from its two 64-key blocks (the second
                // may lie past KV_LEN): full iff both are, empty iff both are
                const uint8_t c0 = row[2 * j], c1 = 2 * j + 1 < nkb ? row[2 * j + 1] : kEmpty;
                c = (c0 == kFull && c1 == kFull) ? kFull : (c0 == kEmpty && c1 == kEmpty) ? kEmpty : kPartial;
            }
        }
        compact_chunk(c == kPartial, c == kFull, i, idx_p, idx_f, run_p, run_f, s_wp, s_wf);
    }
    pad_tail(idx_p, run_p, nq);
    pad_tail(idx_f, run_f, nq);
    if (threadIdx.x == 0) {
        p.out.q_num_blocks[(int64_t)b * nk + j] = run_p;
        p.out.full_q_num_blocks[(int64_t)b * nk + j] = run_f;
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
// Up to 1024 blocks each thread ranks one block against all keys in LDS.
// Beyond that, a counting sort: histogram of the keys in LDS, exclusive scan
// from the largest key down, one wave places the blocks in index order (for
// each key present in a chunk of 64 blocks, the lanes holding it get
// consecutive slots in lane order).  A scan of the block sizes in sorted
// order then gives each block its first entry.
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
    const int nt = cols ? p.nkt : p.nqt;    // rows (columns) per mask batch
    const int len = cols ? p.nqt : p.nkb;   // list length of a row (column)
    const int bpb = (nt + kOrderBlock - 1) / kOrderBlock;  // blocks per mask batch
    const int nb = p.mask_b * bpb;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    auto block_rows = [&](int g, int &r0, int &n) {
        const int bm = g / bpb, j = g - bm * bpb;
        r0 = bm * nt + j * kOrderBlock;
        n = min(kOrderBlock, nt - j * kOrderBlock);
    };
    // Loads of all rows of a block are independent and issued together
    // (clamped to the block's last row, which every block has).
    auto key_of = [&](int g) {
        int r0, n;
        block_rows(g, r0, n);
        int tot = 0;
#pragma unroll
        for (int x = 0; x < kOrderBlock; ++x) {
            const int e = r0 + (x < n ? x : n - 1);
            const int v = num[e] + fnum[e];
            tot += x < n ? v : 0;
        }
        return min(tot, kOrderKeys - 1);
    };

    const int *srt;  // block at each sorted position
    if (nb <= kOrderThreads) {
        // Few blocks: each takes its rank from one pass over all keys in LDS.
        int *s_key = s_hist, *s_sorted = s_hist + kOrderThreads;
        int key = 0;
        if (tid < nb) {
            key = key_of(tid);
            s_key[tid] = key;
        }
        __syncthreads();
        if (tid < nb) {
            int pos = 0;
#pragma unroll 8
            for (int g = 0; g < nb; ++g) {
                const int kg = s_key[g];
                pos += (kg > key) | ((kg == key) & (g < tid));
            }
            s_sorted[pos] = tid;
        }
        __syncthreads();
        srt = s_sorted;
    } else {
        // Counting sort: histogram of the keys, exclusive scan from the
        // largest key down, one wave places the blocks in index order.
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
        srt = sorted;
    }
    // Entries of the rows of each block, in sorted block order.
    int run = 0;  // entries before the current chunk of sorted positions
    for (int pos0 = 0; pos0 < nb; pos0 += kOrderThreads) {
        const int pos = pos0 + tid;
        int r0 = 0, n = 0;
        if (pos < nb) block_rows(srt[pos], r0, n);
        int chunk_total;
        const int first = run + block_exclusive_scan(n, s_wsum, chunk_total);
        if (n > 0) {
            // Every load of the block before the first store: the record
            // stores could alias the lists as far as the compiler knows.
            int nf[kOrderBlock], np[kOrderBlock], fi[kOrderBlock], pi[kOrderBlock];
#pragma unroll
            for (int x = 0; x < kOrderBlock; ++x) {
                const int e = r0 + (x < n ? x : n - 1);
                nf[x] = fnum[e];
                np[x] = num[e];
                fi[x] = fidx[(int64_t)e * len];
                pi[x] = idx[(int64_t)e * len];
            }
#pragma unroll
            for (int x = 0; x < kOrderBlock; ++x) {
                int4 rec;
                rec.x = r0 + x;
                rec.y = nf[x];
                rec.z = np[x];
                rec.w = nf[x] > 0 ? fi[x] : (np[x] > 0 ? pi[x] : 0);
                if (x < n) reinterpret_cast<int4 *>(order)[first + x] = rec;
            }
        }
        run += chunk_total;
    }
}

}  // namespace

hipError_t launch_build_block_mask(const MaskBuildParams &p, hipStream_t stream) {
    if (p.flags & BSM_MASK_DOCUMENT) {
        hipLaunchKernelGGL(check_monotone_kernel, dim3(p.nchunks, p.mask_b), dim3(kThreads), 0,
                           stream, p);
        hipLaunchKernelGGL(ranges_kernel, dim3(p.nchunks, p.mask_b), dim3(kThreads), 0, stream, p);
    }
    if (p.flags & BSM_MASK_TABLE)
        hipLaunchKernelGGL(rows_table_kernel, dim3(p.nqt, p.mask_b), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(rows_kernel, dim3(p.nqt, p.mask_b), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(cols_kernel, dim3(p.nkt, p.mask_b), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(order_kernel, dim3(2), dim3(kOrderThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace bsm
