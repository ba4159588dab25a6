// Internal parameter blocks and launchers shared by the host shim and the
// HIP kernels of the block-sparse masked attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsm.h"

namespace bsm {

constexpr int kTile = 128;          // mask granularity (query and key tiles)
constexpr int kTilePairs = kTile * kTile;

// Work orders: rows (columns) are ordered in blocks of kOrderBlock; distinct
// sort keys of the blocks (longer blocks share the last key).
constexpr int kOrderBlock = 16;
constexpr int kOrderKeys = 8192;

// Tile classes in the per-tile class matrix.
enum : uint8_t { kEmpty = 0, kPartial = 1, kFull = 2 };

struct MaskBuildParams {
    uint32_t flags;
    int32_t T;           // KV_LEN: keys
    int32_t q_len;       // Q_LEN: queries
    int32_t q_off;       // absolute position of query 0
    int32_t npos;        // positions of the document ids: max(T, q_off + q_len)
    int32_t nqt, nkt;    // query tiles, key tiles
    int32_t kb, nkb;     // key-block width of the row lists (128 or 64), key blocks ceil(T / kb)
    int32_t mask_b;
    int32_t nchunks;     // 256-position chunks of the monotonicity check (over npos)
    int32_t sinks;
    int32_t prefix;      // standard combination: causal term widened to kv < prefix (0: none);
                         // TABLE: the prefix term's length (0: term off)
    uint32_t table;      // TABLE: truth table over the five terms
    const int32_t *doc_ids;
    const int32_t *window;
    bsm_block_mask out;
    uint8_t *cls;        // [mask_b, nqt, nkb]: class of each row-list block
    int32_t *nonmono;    // [mask_b, nchunks]
    int32_t *order_ws;   // two arrays of order_ws_stride ints: sorted blocks of the row / column orders
    int32_t order_ws_stride;
};

struct AttnParams {
    int32_t B, H;
    int32_t T;           // KV_LEN: keys
    int32_t nt;          // key tiles, ceil(T / 128)
    int32_t kb, nkb;     // key-block width of the row lists (128 or 64), key blocks ceil(T / kb)
    int32_t q_len;       // Q_LEN: queries
    int32_t nqt;         // query tiles, ceil(q_len / 128)
    int32_t q_off;       // absolute position of query 0
    int32_t npos;        // positions of the document ids / ranges: max(T, q_off + q_len)
    uint32_t table;      // TABLE masks: truth table over the five terms
    int32_t mask_b;
    uint32_t mask_flags;
    uint32_t mod_flags;
    int32_t sinks;
    int32_t prefix;      // causal term widened to kv < prefix (0: plain causal or no causal term)
    float scale;
    float softcap;
    const int32_t *doc_ids;
    const int32_t *window;
    const float *alibi_slopes;
    const float *bias;   // BIAS: [H, 2 bias_r + 1] relative-position bias table
    int32_t bias_r;      // BIAS: its radius R
    // block mask
    const int32_t *kv_num, *kv_idx, *full_kv_num, *full_kv_idx;
    const int32_t *q_num, *q_idx, *full_q_num, *full_q_idx;
    const int32_t *doc_range;   // [mask_b, npos, 2] (first, last) of each position's document, or NULL
    const int32_t *kv_order, *q_order;  // work orders [mask_b * nqt, 4] / [mask_b * nt, 4]: longest first
    // tensors (bf16 or fp16 by the launcher called, strides in elements)
    const void *q; int64_t q_sb, q_sh, q_st;
    const void *k; int64_t k_sb, k_sh, k_st;
    const void *v; int64_t v_sb, v_sh, v_st;
    void *o; int64_t o_sb, o_sh, o_st;          // forward output / backward input
    const void *dout; int64_t do_sb, do_sh, do_st;
    void *dq; int64_t dq_sb, dq_sh, dq_st;
    void *dk; int64_t dk_sb, dk_sh, dk_st;
    void *dv; int64_t dv_sb, dv_sh, dv_st;
    float *lse;      // [B, H, q_len]
    float *delta;    // [B, H, q_len] (backward workspace): <dO, out> per query
    float *lse2;     // [B, H, q_len] (backward workspace): lse * log2(e), 0 where lse = -inf
    float *dslope_part;  // [B, H, nqt] (backward workspace): slope-gradient partial per query tile
    float *dslopes;      // [H] backward output dL/dslope, or NULL (not computed)
    float *dbias_part;   // BIAS: [B, H, nqt, 2 bias_r + 1] (backward workspace): bias-gradient partials
    float *dbias;        // BIAS: [H, 2 bias_r + 1] backward output dL/dbias, or NULL (not reduced)
    // forward item order: items per work-order entry, full blocks, entries in
    // the last block, and division magic numbers (set by the launcher)
    int32_t ord_r, ord_chunk_log2, ord_nblk, ord_p;
    uint32_t ord_m_cr, ord_m_p;
    // dK/dV workgroup placement: 0 contiguous ranges per XCD, 1 chunks dealt
    // to the XCDs in alternating rounds (set by the backward's launcher)
    int32_t col_chunked;
};

hipError_t launch_build_block_mask(const MaskBuildParams &p, hipStream_t stream);
// Attention launchers, one per head dimension and element type (bf16 / f16).
hipError_t launch_attn_fwd_d64_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_fwd_d128_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d64_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d128_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_fwd_d64_f16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_fwd_d128_f16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_fwd_d256_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_fwd_d256_f16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d256_bf16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d256_f16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d64_f16(const AttnParams &p, hipStream_t stream);
hipError_t launch_attn_bwd_d128_f16(const AttnParams &p, hipStream_t stream);
// Decoding step: one query per (b, h) at the last live position of a cache
// of p.T (capacity) positions; the block-mask row arrays of `a` are the
// optional block mask (kv_num NULL: none).  part = B*H*slots*(D + 2) floats.
struct DecodeLaunch {
    AttnParams a;
    int D;
    int32_t dtype;           // BSM_DTYPE_*
    const int32_t *kv_len;   // device live length(s)
    int32_t kv_len_stride;   // 0: one value; 1: one per batch element
    // paged K/V, or NULL block_table: see bsm_flex_attention_decode_paged
    const int32_t *block_table;
    int32_t table_stride, page_size, num_pages;
};
// A decoding workgroup ("slot") covers kDecodeSlotTiles 128-key tiles.
constexpr int kDecodeSlotTiles = 8;
inline int decode_slots(int capacity) {
    return (capacity + kDecodeSlotTiles * kTile - 1) / (kDecodeSlotTiles * kTile);
}
hipError_t launch_attn_decode_bf16(const DecodeLaunch &d, float *part, hipStream_t stream);
hipError_t launch_attn_decode_f16(const DecodeLaunch &d, float *part, hipStream_t stream);

// Copy of the first n_keys keys of each (b, h) of a paged K/V cache into
// contiguous rows (see bsm_gather_kv_pages).  Strides in bytes; sources are
// page-major ([page, head, row]), destinations [b, head, key].
struct GatherLaunch {
    int32_t B, H, row_bytes, page_size, num_pages, table_stride, n_keys;
    const int32_t *table;
    const char *k_src, *v_src;
    int64_t ks_b, ks_h, ks_t, vs_b, vs_h, vs_t;
    char *k_dst, *v_dst;
    int64_t kd_b, kd_h, kd_t, vd_b, vd_h, vd_t;
};
hipError_t launch_gather_pages(const GatherLaunch &g, hipStream_t stream);

}  // namespace bsm
