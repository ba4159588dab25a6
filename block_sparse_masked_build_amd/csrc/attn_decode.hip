// Block-sparse masked attention for decoding: one query per (batch, head)
// at the last live position of a key/value cache, for gfx950.
//
// Method (tutorial "FlexAttention in PyTorch", section "Decoding and paged
// KV caches"): while generating, a single query attends to a cache whose
// length grows by one per step, so the mask must follow the live length;
// the tutorial buckets the cache allocation (e.g. to multiples of 1024) and
// either rebuilds the block mask against the current length or derives the
// key blocks from an existing one.  Here the allocation ("capacity") is what
// the launch is sized by, and the live length is a device value read by the
// kernels, so one launch configuration serves every step of a bucket.  The
// query of batch element b sits at position p = kv_len[b] - 1 and sees key kv
// when kv < kv_len[b] and the mask predicate holds for (p, kv); its scores go
// through the score modifications in the forward's own formulation
// (mod_apply: ALiBi or a relative-position bias table, then the exp2-based
// tanh soft-cap).
//
// Which keys are read:
//  * with a block mask (built once for the whole capacity, square), the
//    row of query tiles holding p lists every key tile any query of that
//    row can see -- a superset of the query's own -- so only those tiles are
//    read (a document-masked decode reads its document's tiles only); the
//    mask needs no rebuild while the cache grows inside the capacity;
//  * without one, every 1024-key chunk below the live length is read,
//    except chunks wholly before the window that hold no sink.
//
// Mapping to CDNA4: a single query has no matrix-product shape, and K and V
// are streamed once, so the path is HBM-bound and runs on the vector units:
//  * decode_partial_kernel: one workgroup per (batch x head, slot of up to
//    eight 128-key tiles), batch x head fastest so that the busy slots of
//    short caches spread over the XCDs: 8 waves of one tile each for
//    D <= 128, 4 waves of two tiles at D = 256.  A wave takes its tiles in
//    64-key blocks whose list entries and page-table entries are looked up
//    while the query row loads.  For D <= 128 a load instruction
//    covers whole rows (16 bytes per lane, D / 8 lanes per row), K and V of
//    a block are requested together, and the scores' partial dot products
//    are summed across each row's lanes; for D = 256 lane = key for the
//    scores and lane = head dimension for the value sum.  fp32 online
//    softmax in the log2 domain per wave, waves merged through LDS; the
//    slot's (max, sum, unnormalised output) go to the workspace.
//  * decode_combine_kernel: one workgroup per (batch, head) merges the slots
//    through their log-sum-exps and writes out (bf16) and lse (fp32, natural
//    log; -inf and out = 0 when no key is visible).
#include <cmath>

#include "attn_common.hpp"

namespace bsm {
namespace {

typedef elem_t dec_elem8 __attribute__((ext_vector_type(8)));

// threads per decoding workgroup: 8 waves of one tile each for D <= 128, 4
// waves of two tiles at D = 256 (whose registers allow one wave per SIMD)
template <int D>
constexpr int kDecThreadsOf = D == 256 ? 256 : 512;
constexpr int kSlotTiles = kDecodeSlotTiles;       // 128-key tiles per workgroup


struct DecodeParams {
    int32_t B, H, capacity, D, nslot, nt;
    const int32_t *kv_len;       // device: live length(s)
    int32_t kv_len_stride;       // 0: one value for the batch; 1: one per batch element
    uint32_t mask_flags, table;  // table: truth table of a composed mask (BSM_MASK_TABLE)
    int32_t sinks, prefix;
    float scale, softcap;
    const int32_t *doc_ids;      // [mask_b, capacity] or NULL
    const int32_t *window;       // device scalar or NULL
    int32_t mask_b;
    const float *alibi_slopes;   // [H] or NULL
    const float *bias;           // [H, 2 bias_r + 1] relative-position bias table or NULL (then ADD is ALiBi)
    int32_t bias_r;
    // block mask rows (NULL kv_num: no block mask)
    const int32_t *kv_num, *kv_idx, *full_kv_num, *full_kv_idx;
    // paged K/V (NULL block_table: one contiguous cache per (b, h)): key kv of
    // batch element b sits in page block_table[b * table_stride + kv / page_size]
    // at row kv % page_size; k_sb / v_sb are then the page strides
    const int32_t *block_table;
    int32_t table_stride, page_size, num_pages;
    const elem_t *q; int64_t q_sb, q_sh;
    const elem_t *k; int64_t k_sb, k_sh, k_st;
    const elem_t *v; int64_t v_sb, v_sh, v_st;
    elem_t *o; int64_t o_sb, o_sh;
    float *lse;                  // [B, H]
    float *part_o;               // [B*H, nslot, D]
    float *part_ml;              // [B*H, nslot, 2]: running max (log2 domain) and sum
};

// Live length of batch element b, clamped to [0, capacity].
__device__ inline int live_len(const DecodeParams &P, int b) {
    const int L = P.kv_len[P.kv_len_stride ? b : 0];
    return L < 0 ? 0 : (L > P.capacity ? P.capacity : L);
}

// The mask predicate for the query at p and key kv < live length.
__device__ inline bool dec_visible(const DecodeParams &P, int bm, int p, int kv, int window, int docq) {
    if (P.mask_flags & BSM_MASK_TABLE) {
        // composed mask: look the five terms up in its truth table
        const uint32_t f = P.mask_flags;
        uint32_t idx = kv <= p ? 1u : 0u;
        if ((f & BSM_MASK_DOCUMENT) && P.doc_ids[(int64_t)bm * P.capacity + kv] == docq) idx |= 2u;
        if ((f & BSM_MASK_WINDOW) && (int64_t)p - kv < window) idx |= 4u;
        if ((f & BSM_MASK_SINKS) && kv < P.sinks) idx |= 8u;
        if ((f & BSM_MASK_PREFIX) && kv < P.prefix) idx |= 16u;
        return (P.table >> idx) & 1u;
    }
    if ((P.mask_flags & BSM_MASK_CAUSAL) && kv > p && !(kv < P.prefix)) return false;
    if ((P.mask_flags & BSM_MASK_DOCUMENT) && P.doc_ids[(int64_t)bm * P.capacity + kv] != docq) return false;
    if (P.mask_flags & BSM_MASK_WINDOW) {
        const bool in_win = (int64_t)p - kv < window;
        const bool sink = (P.mask_flags & BSM_MASK_SINKS) && kv < P.sinks;
        if (!in_win && !sink) return false;
    }
    return true;
}

template <int D>
__device__ inline void write_empty_slot(const DecodeParams &P, int64_t slot) {
    for (int d = threadIdx.x; d < D; d += (int)blockDim.x) P.part_o[slot * D + d] = 0.0f;
    if (threadIdx.x == 0) {
        P.part_ml[slot * 2] = -INFINITY;
        P.part_ml[slot * 2 + 1] = 0.0f;
    }
}

// lane l's value of a 64-bit integer, for a wave-uniform l
__device__ inline int64_t readlane64(int64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ADD: an additive position term -- the ALiBi slope, or with P.bias the bias
// table (one wave-uniform branch per key block; the decoding step is bound
// by its HBM reads, not by this arithmetic).
template <int D, bool ADD, bool SOFTCAP, bool LISTED>
__global__ __launch_bounds__(kDecThreadsOf<D>) void decode_partial_kernel(DecodeParams P) {
    constexpr int kDecThreads = kDecThreadsOf<D>, kDecWaves = kDecThreads / 64;
    constexpr int kWaveTiles = kSlotTiles / kDecWaves;  // tiles per wave
    constexpr int kDimsPerLane = D / 64;  // output dims per lane: lane * kDimsPerLane + i
    __shared__ float sq[D];               // the query row, fp32
    __shared__ float sp[kDecWaves][64];   // probabilities of a wave's 64 keys
    __shared__ float sm[kDecWaves], sl[kDecWaves];
    __shared__ float so[kDecWaves][D];

    const int slot_i = blockIdx.y, bh = blockIdx.x;
    const int b = bh / P.H, h = bh - b * P.H;
    const int bm = P.mask_b == 1 ? 0 : b;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t slot = (int64_t)bh * P.nslot + slot_i;
    const int L = live_len(P, b);
    const int p = L - 1;
    const int window = (P.mask_flags & BSM_MASK_WINDOW) ? *P.window : 0;

    // Tiles of this slot: entries 8 slot_i .. 8 slot_i + 7 of the block-mask
    // row of p (full tiles first), or the slot's eight consecutive tiles; a
    // slot with none of them below the live length writes an empty partial.
    int row = 0, nfull = 0, nlist = 0;
    if (L == 0) {
        write_empty_slot<D>(P, slot);
        return;
    }
    if (LISTED) {
        row = bm * P.nt + p / kTile;
        // counts clamped to the row length, so indices stay inside the lists
        nfull = min(max(P.full_kv_num[row], 0), P.nt);
        nlist = nfull + min(max(P.kv_num[row], 0), P.nt - nfull);
        if (kSlotTiles * slot_i >= nlist) {
            write_empty_slot<D>(P, slot);
            return;
        }
    } else {
        const int64_t c0 = (int64_t)slot_i * kSlotTiles * kTile;
        const int64_t c1 = min(c0 + kSlotTiles * kTile, (int64_t)L);  // keys [c0, c1)
        bool skip = c0 >= L;
        // wholly before the window and holding no sink (the standard
        // combination only: a composed mask may OR the window with more)
        if (!skip && (P.mask_flags & BSM_MASK_WINDOW) && !(P.mask_flags & BSM_MASK_TABLE))
            skip = (int64_t)p - (c1 - 1) >= window && !((P.mask_flags & BSM_MASK_SINKS) && c0 < P.sinks);
        if (skip) {
            write_empty_slot<D>(P, slot);
            return;
        }
    }

    int docq = 0;
    if (P.mask_flags & BSM_MASK_DOCUMENT) docq = P.doc_ids[(int64_t)bm * P.capacity + p];
    const bool table = ADD && P.bias;
    const float slope = ADD && !table ? P.alibi_slopes[h] : 0.0f;
    const ModK mk = mod_k<SOFTCAP>(P.scale, slope, SOFTCAP ? P.softcap : 1.0f);
    const float bias_f = mod_f<SOFTCAP>(SOFTCAP ? P.softcap : 1.0f);
    const float *brow = table ? P.bias + (int64_t)h * (2 * P.bias_r + 1) + P.bias_r : nullptr;  // entry of distance 0

    // The wave's 64-key blocks, looked up before the query row is loaded so
    // that the list and page-table reads overlap it: lane s < 2 kWaveTiles
    // holds block s's first key (-1: no block) and the offsets of its first
    // K and V rows.  A paged block lies in one page (page sizes are
    // multiples of 64); an out-of-range table entry is clamped, so a bad
    // table reads a wrong page, never outside the pool.
    int blk_key0 = -1;
    int64_t blk_koff = 0, blk_voff = 0;
    if (lane < 2 * kWaveTiles) {
        const int te = kSlotTiles * slot_i + kWaveTiles * wv + (lane >> 1);
        int key0 = -1;
        if (LISTED) {
            if (te < nlist) {
                const int j = te < nfull ? P.full_kv_idx[(int64_t)row * P.nt + te]
                                         : P.kv_idx[(int64_t)row * P.nt + te - nfull];
                key0 = clamp_tile(j, P.nt) * kTile + (lane & 1) * 64;
            }
        } else {
            key0 = te * kTile + (lane & 1) * 64;
        }
        if (key0 >= 0 && key0 < L) {
            blk_key0 = key0;
            if (P.block_table) {
                const int pg = min(max(P.block_table[(int64_t)b * P.table_stride + key0 / P.page_size], 0),
                                   P.num_pages - 1);
                const int64_t r = key0 % P.page_size;
                blk_koff = pg * P.k_sb + r * P.k_st;
                blk_voff = pg * P.v_sb + r * P.v_st;
            } else {
                blk_koff = b * P.k_sb + (int64_t)key0 * P.k_st;
                blk_voff = b * P.v_sb + (int64_t)key0 * P.v_st;
            }
        }
    }

    const elem_t *qrow = P.q + b * P.q_sb + h * P.q_sh;
    for (int d = threadIdx.x; d < D; d += kDecThreads) sq[d] = static_cast<float>(qrow[d]);
    __syncthreads();

    const elem_t *kb = P.k + h * P.k_sh;
    const elem_t *vb = P.v + h * P.v_sh;
    float m = -INFINITY, l = 0.0f;  // running max (log2 domain) and sum of the wave
    if constexpr (D <= 128) {
        // Lane l reads 16-byte pieces of rows: chunk c = l % kG (head
        // dims 8c .. 8c + 7) of row g = l / kG of each group of kKpi rows,
        // so one load instruction covers kKpi whole rows.  The query chunk
        // stays in registers.
        constexpr int kG = D / 8, kKpi = 64 / kG;
        const int c = lane % kG, g = lane / kG;
        float qc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qc[e] = sq[c * 8 + e];
        // after the reduction of the scores lane l holds the score of key
        // (l % kG) kKpi + l / kG of the block
        const int my_key = c * kKpi + g;
        float o[8];  // head dims 8c .. 8c + 7 over the rows g, g + kKpi, ...
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.0f;

#pragma unroll 1
        for (int sub = 0; sub < 2 * kWaveTiles; ++sub) {
            const int key0 = __builtin_amdgcn_readlane(blk_key0, sub);
            if (key0 < 0) continue;  // no block
            // rows key0 .. key0 + 63 of K and V
            const elem_t *kblk = kb + readlane64(blk_koff, sub), *vblk = vb + readlane64(blk_voff, sub);
            const uint64_t vis = __ballot(key0 + lane < L && dec_visible(P, bm, p, key0 + lane, window, docq));
            if (vis == 0) continue;  // nothing visible: the running state is unchanged
            // rows of invisible keys are replaced by the first visible one (a
            // cache hit), so every load stays in bounds and reads no extra line
            const int fv = __builtin_ctzll(vis);
            // every K and V piece of the block is requested before any is
            // used: the value rows do not depend on the scores, so both
            // stream at once
            dec_elem8 kk[kG], vv[kG];
#pragma unroll
            for (int i = 0; i < kG; ++i) {
                const int r = i * kKpi + g;
                const int re = (vis >> r) & 1 ? r : fv;
                kk[i] = *reinterpret_cast<const dec_elem8 *>(kblk + (int64_t)re * P.k_st + c * 8);
            }
#pragma unroll
            for (int i = 0; i < kG; ++i) {
                const int r = i * kKpi + g;
                const int re = (vis >> r) & 1 ? r : fv;
                vv[i] = *reinterpret_cast<const dec_elem8 *>(vblk + (int64_t)re * P.v_st + c * 8);
            }
            float part[kG];
#pragma unroll
            for (int i = 0; i < kG; ++i) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qc[e], static_cast<float>(kk[i][e]), acc);
                part[i] = acc;
            }
            // sum the kG partial dot products of each row across its kG lanes:
            // each halving step keeps the half of the rows selected by one lane
            // bit (highest first), so lane l ends with row index l % kG
#pragma unroll
            for (int n = kG; n > 1; n >>= 1) {
                const int half = n >> 1;
                const bool up = (c & half) != 0;
#pragma unroll
                for (int j = 0; j < half; ++j) {
                    const float send = up ? part[j] : part[j + half];
                    const float keep = up ? part[j + half] : part[j];
                    part[j] = keep + __shfl_xor(send, half);
                }
            }
            const int kv = key0 + my_key;
            float t = -INFINITY;
            if ((vis >> my_key) & 1) {
                // log2-domain modified score, as in the forward
                float add = -mk.slope_f * (float)(p - kv);
                if (table) add = bias_f * brow[min(max(p - kv, -P.bias_r), P.bias_r)];
                t = mod_apply<ADD, SOFTCAP>(part[0], add, mk);
            }
            // online softmax over this wave's 64 keys (log2 domain)
            float mx = t;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_new = fmaxf(m, mx);  // finite: some key is visible
            const float pk = fast_exp2(t - m_new);
            const float alpha = fast_exp2(m - m_new);
            float ps = pk;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
            l = l * alpha + ps;
            m = m_new;
            sp[wv][my_key] = pk;  // read back by every lane of this wave (LDS operations stay in order)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
            // value rows (invisible keys have p = 0 and hold the first visible row)
#pragma unroll
            for (int i = 0; i < kG; ++i) {
                const float pj = sp[wv][i * kKpi + g];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(pj, static_cast<float>(vv[i][e]), o[e]);
            }
        }
        // sum the output pieces of the kKpi row groups: lanes l < kG then hold
        // head dims 8l .. 8l + 7
#pragma unroll
        for (int off = kG; off < 64; off <<= 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off);
        }
        if (lane < kG) {
#pragma unroll
            for (int e = 0; e < 8; ++e) so[wv][lane * 8 + e] = o[e];
        }
    } else {
        // D = 256: lane = key for the scores (the query row broadcast from
        // LDS), then lane = head dimensions for the value sum, all 64 value
        // rows in flight (the row-piece layout above measured slower here)
        float o[kDimsPerLane];
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) o[i] = 0.0f;

#pragma unroll 1
        for (int sub = 0; sub < 2 * kWaveTiles; ++sub) {
            const int key0 = __builtin_amdgcn_readlane(blk_key0, sub);
            if (key0 < 0) continue;  // no block
            // rows key0 .. key0 + 63 of K and V
            const elem_t *kblk = kb + readlane64(blk_koff, sub), *vblk = vb + readlane64(blk_voff, sub);
            const int kv = key0 + lane;
            float t = -INFINITY;
            if (kv < L && dec_visible(P, bm, p, kv, window, docq)) {
                const elem_t *krow = kblk + (int64_t)lane * P.k_st;
                float acc = 0.0f;
#pragma unroll
                for (int d0 = 0; d0 < D; d0 += 8) {
                    const dec_elem8 kk = *reinterpret_cast<const dec_elem8 *>(krow + d0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(sq[d0 + e], static_cast<float>(kk[e]), acc);
                }
                // log2-domain modified score, as in the forward
                float add = -mk.slope_f * (float)(p - kv);
                if (table) add = bias_f * brow[min(max(p - kv, -P.bias_r), P.bias_r)];
                t = mod_apply<ADD, SOFTCAP>(acc, add, mk);
            }
            // online softmax over this wave's 64 keys (log2 domain)
            float mx = t;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_new = fmaxf(m, mx);
            const float pk = m_new == -INFINITY ? 0.0f : fast_exp2(t - m_new);
            const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m - m_new);
            float ps = pk;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
            l = l * alpha + ps;
            m = m_new;
            sp[wv][lane] = pk;  // read back by every lane of this wave (LDS operations stay in order)
#pragma unroll
            for (int i = 0; i < kDimsPerLane; ++i) o[i] *= alpha;
            if (mx != -INFINITY) {
                // the block's 64 value rows, their loads issued together
                // (keys past the live length have p = 0 and read a row
                // inside the cache instead)
                const int nk = min(64, L - key0);
                const elem_t *vbase = vblk + lane * kDimsPerLane;
                float vv[64][kDimsPerLane];
#pragma unroll
                for (int j = 0; j < 64; ++j) {
                    const int key = min(j, nk - 1);  // offset in the block
                    const elem_t *vrow = vbase + (int64_t)key * P.v_st;
#pragma unroll
                    for (int i = 0; i < kDimsPerLane; ++i) vv[j][i] = static_cast<float>(vrow[i]);
                }
#pragma unroll
                for (int j = 0; j < 64; ++j) {
                    const float pj = j < nk ? sp[wv][j] : 0.0f;
#pragma unroll
                    for (int i = 0; i < kDimsPerLane; ++i) o[i] = __builtin_fmaf(pj, vv[j][i], o[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) so[wv][lane * kDimsPerLane + i] = o[i];
    }
    // merge the waves (their outputs are in so)
    if (lane == 0) {
        sm[wv] = m;
        sl[wv] = l;
    }
    __syncthreads();
    if (wv == 0) {
        float M = sm[0];
        for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, sm[w]);
        float Ls = 0.0f, acc[kDimsPerLane];
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) acc[i] = 0.0f;
        for (int w = 0; w < kDecWaves; ++w) {
            const float f = (M == -INFINITY) ? 0.0f : fast_exp2(sm[w] - M);
            Ls += sl[w] * f;
#pragma unroll
            for (int i = 0; i < kDimsPerLane; ++i) acc[i] += so[w][lane * kDimsPerLane + i] * f;
        }
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) P.part_o[slot * D + lane * kDimsPerLane + i] = acc[i];
        if (lane == 0) {
            P.part_ml[slot * 2] = M;
            P.part_ml[slot * 2 + 1] = Ls;
        }
    }
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams P) {
    constexpr int kDimsPerLane = D / 64;
    const int bh = blockIdx.x, lane = threadIdx.x;
    const int b = bh / P.H, h = bh - b * P.H;
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < P.nslot; ++s) M = fmaxf(M, P.part_ml[((int64_t)bh * P.nslot + s) * 2]);
    float Ls = 0.0f, acc[kDimsPerLane];
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) acc[i] = 0.0f;
#pragma unroll 8
    for (int s = 0; s < P.nslot; ++s) {  // independent loads, unrolled so they overlap
        const int64_t slot = (int64_t)bh * P.nslot + s;
        const float f = (M == -INFINITY) ? 0.0f : fast_exp2(P.part_ml[slot * 2] - M);
        Ls += P.part_ml[slot * 2 + 1] * f;
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) acc[i] += P.part_o[slot * D + lane * kDimsPerLane + i] * f;
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    elem_t *orow = P.o + b * P.o_sb + h * P.o_sh;
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) orow[lane * kDimsPerLane + i] = static_cast<elem_t>(acc[i] * inv);
    if (lane == 0) P.lse[bh] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
}

template <int D, bool ALIBI, bool SOFTCAP>
void launch_mods(const DecodeParams &P, hipStream_t stream) {
    // (batch, head) fastest: consecutive workgroups go to different XCDs, so
    // the slots that hold keys -- the first ones at short live lengths --
    // spread over the whole chip instead of landing on one XCD
    const dim3 grid(P.B * P.H, P.nslot), block(kDecThreadsOf<D>);
    if (P.kv_num)
        hipLaunchKernelGGL((decode_partial_kernel<D, ALIBI, SOFTCAP, true>), grid, block, 0, stream, P);
    else
        hipLaunchKernelGGL((decode_partial_kernel<D, ALIBI, SOFTCAP, false>), grid, block, 0, stream, P);
}

template <int D>
hipError_t launch_d(const DecodeParams &P, uint32_t mod_flags, hipStream_t stream) {
    // the bias table takes the ALiBi instances (see decode_partial_kernel)
    const bool alibi = mod_flags & (BSM_MOD_ALIBI | BSM_MOD_BIAS), cap = mod_flags & BSM_MOD_SOFTCAP;
    if (alibi && cap)
        launch_mods<D, true, true>(P, stream);
    else if (alibi)
        launch_mods<D, true, false>(P, stream);
    else if (cap)
        launch_mods<D, false, true>(P, stream);
    else
        launch_mods<D, false, false>(P, stream);
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(P.B * P.H), dim3(64), 0, stream, P);
    return hipGetLastError();
}

}  // namespace

hipError_t BSM_ELEM_FN(launch_attn_decode)(const DecodeLaunch &d, float *part, hipStream_t stream) {
    const AttnParams &a = d.a;
    DecodeParams P{};
    P.B = a.B;
    P.H = a.H;
    P.capacity = a.T;
    P.D = d.D;
    P.nslot = decode_slots(a.T);
    P.nt = (a.T + kTile - 1) / kTile;
    P.kv_len = d.kv_len;
    P.kv_len_stride = d.kv_len_stride;
    P.mask_flags = a.mask_flags;
    P.table = a.table;
    P.sinks = a.sinks;
    P.prefix = a.prefix;
    P.scale = a.scale;
    P.softcap = a.softcap;
    P.doc_ids = a.doc_ids;
    P.window = a.window;
    P.mask_b = a.mask_b;
    P.alibi_slopes = a.alibi_slopes;
    P.bias = a.bias;
    P.bias_r = a.bias_r;
    P.kv_num = a.kv_num;
    P.kv_idx = a.kv_idx;
    P.full_kv_num = a.full_kv_num;
    P.full_kv_idx = a.full_kv_idx;
    P.block_table = d.block_table;
    P.table_stride = d.table_stride;
    P.page_size = d.page_size;
    P.num_pages = d.num_pages;
    P.q = static_cast<const elem_t *>(a.q);
    P.q_sb = a.q_sb;
    P.q_sh = a.q_sh;
    P.k = static_cast<const elem_t *>(a.k);
    P.k_sb = a.k_sb;
    P.k_sh = a.k_sh;
    P.k_st = a.k_st;
    P.v = static_cast<const elem_t *>(a.v);
    P.v_sb = a.v_sb;
    P.v_sh = a.v_sh;
    P.v_st = a.v_st;
    P.o = static_cast<elem_t *>(a.o);
    P.o_sb = a.o_sb;
    P.o_sh = a.o_sh;
    P.lse = a.lse;
    P.part_o = part;
    P.part_ml = part + (int64_t)a.B * a.H * P.nslot * d.D;
    if (d.D == 64) return launch_d<64>(P, a.mod_flags, stream);
    if (d.D == 256) return launch_d<256>(P, a.mod_flags, stream);
    return launch_d<128>(P, a.mod_flags, stream);
}

}  // namespace bsm
