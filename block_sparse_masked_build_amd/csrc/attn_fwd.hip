// Block-sparse masked attention, forward pass, for gfx950.
//
// Method (speedrun notes "FlexAttention", Context and tile-summary
// paragraphs; tutorial "FlexAttention in PyTorch", "The two hooks" and
// Pattern 3): exact softmax attention in one fused tiled kernel that never
// writes the T x T scores; each query tile visits only the key tiles its
// block-mask row lists -- full tiles without any elementwise mask, partial
// tiles with it -- and every score goes through the score modifications
// (ALiBi, tanh soft-cap) before the softmax.
//
// Mapping to CDNA4:
//  * one workgroup of 4 waves per (batch, head, 128-row query tile); wave w
//    owns queries 32w..32w+31; lane l owns query l%32, lane half l/32 splits
//    the keys;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, so the
//    score and output accumulators of a query live in one lane pair: the
//    online softmax (running max m, running sum l, fp32) needs one cross-half
//    exchange per tile, and the output rescale is lane-local;
//  * Q stays in registers; K and V tiles are copied HBM -> LDS directly
//    (global_load_lds, 16 bytes per lane, no registers), row-major with
//    XOR-swizzled 16-byte chunks; the V^T operand comes from transposing LDS
//    reads (ds_read_tr16_b64), so no tile is ever transposed by hand;
//  * each listed 128-key tile is processed as two 64-key halves through
//    double-buffered LDS: one barrier per half, and every copy is issued a
//    whole half-iteration before it is read (K two halves ahead, V one);
//  * software pipeline inside each wave: the QK^T products of the next half
//    are interleaved with the exponentials of the current one, and the PV
//    products of the current half with the masking of the next one, so the
//    matrix cores and the vector ALU work at the same time;
//  * two workgroups per CU (at most 256 registers per lane), so one
//    workgroup's barrier waits are covered by the other's work;
//  * exp via exp2 with log2(e) and the score scale folded into one FMA; the
//    running maximum is only moved (and the output rescaled) when a score
//    exceeds it by more than 2^8.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "attn_common.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kHalf = 64;  // keys per pipeline step

// Per-query state of the online softmax.  m is the reference maximum (log2
// domain) the accumulators are scaled to; it is only moved when a new score
// exceeds it by more than 2^8, so most steps skip the rescale.  The result
// stays exact because o and l always share the same reference.
constexpr float kRescaleThreshold = 8.0f;

// Per-lane LDS byte offsets of the matrix-core operands inside a half tile.
// Both patterns are XOR-structured, so one base per role is kept and the
// offset of each operand is derived where it is used:
//   K operand of d step st:           k ^ (st << 5)
//   V operand of d block db, half u:  v + u * 8 rows ^ (db << 6)
template <int D>
struct OperandOffsets {
    int k;   // row n of key block 0, chunk hl ^ fk(n)
    int v;   // transposing-read address of d block 0, keys +0..3
};

template <int D>
__device__ inline void operand_offsets(OperandOffsets<D> &off) {
    using L = TileLayout<D>;
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
    // chunk (2 st + hl) ^ fk(n) = (2 st) ^ (hl ^ fk(n)) since 2 st and hl
    // occupy different bits; the row part n * kRowBytes is a multiple of 256.
    off.k = n * L::kRowBytes + ((hl ^ L::fk(n)) << 4);
    // ds_read_tr16_b64: lane j of a 16-lane group G supplies the address of
    // row K0 + j/4, columns d0 + 4 (j%4) .. +3; lane i then receives rows
    // K0..K0+3 of column d0 + i.  d0 = 32 db + 16 (G%2); K0 = 4 (G/2) (+8 for
    // the second half) inside each 16-key group.  fv depends on the row's low
    // bits only, which the +8 of the second half does not change for either
    // head dimension, and the d block adds 4 db to the chunk, i.e. XOR
    // (4 db) ^ ... = (db << 6) in bytes as 4 db stays clear of the other terms'
    // bits for D = 128 (chunk bits 2-3) and D = 64 (chunk bit 2).
    const int G = lane >> 4, j = lane & 15;
    const int r = 4 * (G >> 1) + (j >> 2);
    const int c = 2 * (G & 1) + ((j & 3) >> 1);
    off.v = r * L::kRowBytes + ((c ^ L::fv(r)) << 4) + ((j & 1) << 3);
}

template <int D>
__device__ inline int k_operand_offset(const OperandOffsets<D> &off, int st) {
    return off.k ^ (st << 5);
}

template <int D>
__device__ inline int v_operand_offset(const OperandOffsets<D> &off, int u, int db) {
    return (off.v ^ (db << 6)) + u * 8 * TileLayout<D>::kRowBytes;
}

// S^T = K Q^T for one half tile: lane (query n, half hl) gets, for key block
// kb (32 keys), the 16 scores of keys 32 kb + 8 (r/4) + 4 hl + r%4.
template <int D>
__device__ inline void fwd_qk(const elem_t *sk, const OperandOffsets<D> &off, const elem8 (&qf)[D / 16],
                              f32x16 (&s)[2]) {
    const char *kbytes = reinterpret_cast<const char *>(sk);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const elem8 a = *reinterpret_cast<const elem8 *>(kbytes + kb * 32 * TileLayout<D>::kRowBytes +
                                                                k_operand_offset(off, st));
            s[kb] = mfma32(a, qf[st], s[kb]);
        }
    }
}

// p = 2^(s c - m) as bf16 (the B operand of the PV products), summed into l
// in fp32 before rounding (so lse keeps fp32 accuracy).
__device__ inline void fwd_exp(const f32x16 (&s)[2], elem8 (&pb)[2][2], float &l, float c_mul, float m_use) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = fast_exp2(__builtin_fmaf(s[kb][s2 * 8 + e], c_mul, -m_use));
                l += pv;
                pb[kb][s2][e] = static_cast<elem_t>(pv);
            }
}

template <int D>
__device__ inline void fwd_pv(const elem_t *sv, const OperandOffsets<D> &off, const elem8 (&pb)[2][2],
                              f32x16 (&o)[D / 32]) {
    const char *vbytes = reinterpret_cast<const char *>(sv);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int rowbase = (kb * 32 + s2 * 16) * TileLayout<D>::kRowBytes;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const i16x4 lo = ds_read_tr16(reinterpret_cast<const elem_t *>(vbytes + rowbase + v_operand_offset(off, 0, db)));
                const i16x4 hi = ds_read_tr16(reinterpret_cast<const elem_t *>(vbytes + rowbase + v_operand_offset(off, 1, db)));
                const elem8 a = __builtin_bit_cast(elem8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = mfma32(a, pb[kb][s2], o[db]);
            }
        }
    }
}

// ---------------------------------------------------------------- schedule
// One workgroup per item -- one (batch, head, query tile) row of the block
// mask.  The hardware dispatcher hands workgroups to free slots in blockIdx
// order, so the order of blockIdx is the order of work: the block mask's
// work order (rows with the most listed tiles first, so short rows fill the
// end of the launch), arranged so that the rows running at the same time on
// one XCD share key and value tiles (see ItemOrder).

// Wave-uniform values of the item being worked on.
struct FwdArgs {
    const elem_t *kb, *vb;
    const int32_t *doc, *fidx, *pidx;
    int b, h, bm, row;
    int nfull, ntiles, nt, first;  // listed blocks (full, all), blocks per row, first listed block
    int kblk, spb;                  // block width (128 or 64 keys) and 64-key steps per block
    int qpos;  // this lane's absolute query position (the last query's for lanes past Q_LEN)
    float scale, scale_log2, slope, cap, inv_cap;
    ModK mk;  // folded score-modification constants
};

// This lane's query index (past Q_LEN on a cut-short last row), recomputed
// where needed rather than kept live through the item.
__device__ inline int lane_query(const FwdArgs &a) {
    return a.row * kTile + (threadIdx.x >> 6) * 32 + (threadIdx.x & 31);
}

template <bool ALIBI, bool SOFTCAP, bool GENERAL>
__device__ inline void item_args(const AttnParams &p, int rem, const WorkRec &rec, FwdArgs &a) {
    const int nt = p.nkb;  // key blocks of the row lists
    const int packed = min(max(rec.packed, 0), p.mask_b * p.nqt - 1);
    a.bm = packed / p.nqt;
    a.row = packed - a.bm * p.nqt;
    head_of(p, rem, a.bm, a.b, a.h);
    a.kb = static_cast<const elem_t *>(p.k) + a.b * p.k_sb + a.h * p.k_sh;
    a.vb = static_cast<const elem_t *>(p.v) + a.b * p.v_sb + a.h * p.v_sh;
    a.fidx = p.full_kv_idx + (int64_t)packed * nt;
    a.pidx = p.kv_idx + (int64_t)packed * nt;
    a.doc = (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids + (int64_t)a.bm * p.npos : nullptr;
    a.nfull = min(max(rec.nfull, 0), nt);
    a.ntiles = a.nfull + min(max(rec.npart, 0), nt);
    a.first = clamp_tile(rec.first, nt);
    a.nt = nt;
    a.kblk = GENERAL ? p.kb : kTile;  // 128-key tiles in the other kernel (see kv_ragged)
    a.spb = a.kblk / kHalf;
    a.qpos = p.q_off + min(lane_query(a), p.q_len - 1);
    a.scale = p.scale;
    a.scale_log2 = p.scale * kLog2e;
    a.slope = ALIBI ? p.alibi_slopes[a.h] : 0.0f;
    a.cap = SOFTCAP ? p.softcap : 1.0f;
    a.inv_cap = 1.0f / a.cap;
    a.mk = mod_k<SOFTCAP>(a.scale, a.slope, a.cap);
}

// Entries 0..127 of the query-tile row's tile list (full tiles first, then
// partial ones), one per lane in two registers, so that a step finds its key
// tile with one cross-lane read instead of a dependent memory load.  Longer
// lists (beyond 128 visible tiles in one row) read the rest from memory.
struct TileList {
    int lo, hi;  // entries lane and 64 + lane
};

__device__ inline int list_entry(const FwdArgs &a, int e) {
    int v = 0;
    if (e < a.nfull)
        v = a.fidx[e];
    else if (e < a.ntiles)
        v = a.pidx[e - a.nfull];
    return clamp_tile(v, a.nt);
}

__device__ inline int tile_at(const TileList &tl, const FwdArgs &a, int it) {
    if (it >= 128)
        return clamp_tile(it < a.nfull ? load_uniform(a.fidx + it) : load_uniform(a.pidx + it - a.nfull), a.nt);
    return __builtin_amdgcn_readlane(it < 64 ? tl.lo : tl.hi, it & 63);
}

// First key of the row's 64-key step t: listed block t / spb (full blocks
// first), and for 128-key blocks its half t % 2.
__device__ inline int row_step_key0(const TileList &tl, const FwdArgs &a, int t) {
    return a.spb == 2 ? tile_at(tl, a, t >> 1) * kTile + (t & 1) * kHalf : tile_at(tl, a, t) * kHalf;
}

// The same for step 1, before the tile list is loaded.  A row of a single
// 64-key block has no step 1: its key is then the block's own, so that the
// copy issued for it stays inside the tensor.
__device__ inline int step1_key0(const FwdArgs &a) {
    if (a.spb == 2) return a.first * kTile + kHalf;
    if (a.ntiles < 2) return a.first * kHalf;
    return clamp_tile(1 < a.nfull ? load_uniform(a.fidx + 1) : load_uniform(a.pidx + 1 - a.nfull), a.nt) * kHalf;
}

// Per-lane row data loaded at the start of an item: the query's document
// range and id.
struct RowLoad {
    int ds, de, docq;
};

// Row view of the mask (see make_row_mask) from the loaded row data; returns
// the mode the row needs (uniform over the workgroup: the document-range
// sentinel marks whole mask rows).
__device__ inline int finish_row_mask(const AttnParams &p, int qpos, const RowLoad &rl, int window, RowMask &rm) {
    int ds = rl.ds, de = rl.de;
    const bool gather = ds < 0;
    if (gather) {
        ds = 0;
        de = p.T - 1;
    }
    rm.docq = rl.docq;
    // keys past KV_LEN are never visible (the last key tile may be cut short)
    const int hi = min(min((p.mask_flags & BSM_MASK_CAUSAL) ? max(qpos, p.prefix - 1) : p.T - 1, de), p.T - 1);
    int lo = ds;
    bool sinks = false;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        const int64_t wlo = (int64_t)qpos - (int64_t)window + 1;
        if (wlo > lo) lo = wlo > p.T ? p.T : (int)wlo;
        sinks = (p.mask_flags & BSM_MASK_SINKS) && p.sinks > 0;
    }
    rm.lo = lo;
    rm.hi = hi;
    rm.slo = ds;
    rm.shi = sinks ? min(p.sinks - 1, hi) : ds - 1;
    return __builtin_amdgcn_readfirstlane(gather ? kGather : sinks ? kSinks : kPlain);
}

// LDS of the forward: double-buffered 64-key halves of K and V and the
// keys' document ids.
template <int D>
struct FwdSmem {
    elem_t k[2][kHalf * D];  // keys, rows swizzled by fk
    elem_t v[2][kHalf * D];  // values, rows swizzled by fv
    int32_t doc[2][kHalf];   // document ids of the keys
};

// Starts an item: copies of K and V of step 0 and K of step 1 (the two
// halves of the first listed tile) into buffers 0 / 0 / 1, and loads of the
// query rows, the tile list and the row data.  Every item has an even
// number of steps, so each item starts on buffer 0.
// Rows of a 64-key copy that exist, given n = KV_LEN (or positions) - its
// first key.  GENERAL (the general kernel, see kv_ragged): the last block may
// be cut short and its copies are clamped; otherwise every copy is whole and
// the clamping code is compiled out -- its mere presence in the step loop
// cost the forward 6-9% on whole-tile shapes.
template <bool GENERAL>
__device__ inline int rows_left(int n) { return GENERAL ? n : kHalf; }

template <int D, bool GENERAL>
__device__ __attribute__((always_inline)) inline void item_start(const AttnParams &p, FwdSmem<D> &sm, const FwdArgs &a, elem8 (&qf)[D / 16],
                                  TileList &tl, RowLoad &rl) {
    if (a.ntiles > 0) {
        // rows past KV_LEN (document ids: past the positions) repeat the last one
        const int k0 = a.first * a.kblk;
        const int k1 = step1_key0(a);
        if (a.doc) {
            issue_ints_to_lds_at<kHalf>(lds_addr(sm.doc[0]), a.doc + k0, rows_left<GENERAL>(p.npos - k0));
            issue_ints_to_lds_at<kHalf>(lds_addr(sm.doc[1]), a.doc + k1, rows_left<GENERAL>(p.npos - k1));
        }
        issue_tile_to_lds<D, kSwzK, kHalf>(sm.k[0], a.kb + (int64_t)k0 * p.k_st, p.k_st, rows_left<GENERAL>(p.T - k0));
        issue_tile_to_lds<D, kSwzV, kHalf>(sm.v[0], a.vb + (int64_t)k0 * p.v_st, p.v_st, rows_left<GENERAL>(p.T - k0));
        issue_tile_to_lds<D, kSwzK, kHalf>(sm.k[1], a.kb + (int64_t)k1 * p.k_st, p.k_st, rows_left<GENERAL>(p.T - k1));
    }
    const int hl = (threadIdx.x & 63) >> 5;
    const elem_t *qrow = static_cast<const elem_t *>(p.q) + a.b * p.q_sb + a.h * p.q_sh +
                         (int64_t)min(lane_query(a), p.q_len - 1) * p.q_st;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) qf[st] = *reinterpret_cast<const elem8 *>(qrow + st * 16 + hl * 8);
    const int lane = threadIdx.x & 63;
    tl.lo = list_entry(a, lane);
    tl.hi = a.ntiles > 64 ? list_entry(a, 64 + lane) : 0;
    rl.ds = 0;
    rl.de = p.T - 1;
    rl.docq = 0;
    if (a.doc) {
        const int32_t *dr = p.doc_range + ((int64_t)a.bm * p.npos + a.qpos) * 2;
        rl.ds = dr[0];
        rl.de = dr[1];
        rl.docq = a.doc[a.qpos];
    }
}

// Output of a finished item: out = o / l as bf16, lse = (m + log2 l) ln 2.
// Each wave's 32 rows go through its own 32 x D slice of LDS at `stage`
// and are stored as whole rows.
template <int D>
__device__ __attribute__((always_inline)) inline void store_item(const AttnParams &p, const FwdArgs &a,
                                                                 const f32x16 (&o)[D / 32], float m, float l,
                                                                 uint32_t stage) {
    const int hl = (threadIdx.x & 63) >> 5, wv = wave_id();
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.0f ? fast_rcp(l_tot) : 0.0f;
    const int q0w = a.row * kTile + wv * 32;  // the wave's first query index
    elem_t *ob = static_cast<elem_t *>(p.o) + a.b * p.o_sb + a.h * p.o_sh + (int64_t)q0w * p.o_st;
    store_rows_staged<D>(ob, p.o_st, o, inv, stage + (uint32_t)(wv * 32 * 2 * D), p.q_len - q0w);
    const int qidx = lane_query(a);
    if (hl == 0 && qidx < p.q_len)
        p.lse[((int64_t)a.b * p.H + a.h) * p.q_len + qidx] =
            l_tot > 0.0f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// The double-buffered, software-pipelined loop over one item's listed tiles
// (in 64-key steps); the caller has waited for the item's first copies and
// loads and passed a workgroup barrier.  Step t's scores (modified, masked)
// and their row maximum are computed during step t-1.  At the top of step t
// the copies issued at the top of step t-1 -- K(t+1) and V(t) -- have
// landed; the barrier also certifies that every wave has finished step t-1,
// freeing K buffer t%2 (last read for K(t)) and V buffer (t+1)%2 (last read
// for V(t-1)) for K(t+2) and V(t+1).
//
// A step first settles the online-softmax reference (moving it, and
// rescaling o and l, only when the new maximum exceeds it by more than the
// threshold), then runs one branch-free block: QK^T products of step t+1,
// exponentials and PV products of step t, score modifications, mask and row
// maximum of step t+1 -- so the compiler can interleave matrix-core products
// with all of the step's vector work.  Steps whose next tile is full and
// steps whose next tile is partial run in separate loops (the tile list
// holds full tiles first), so the elementwise mask needs no branch.
//
// The item's output is written at its end, staged through the K buffers,
// which no wave reads during the last step.
template <int D, bool ALIBI, bool SOFTCAP, int MODE, bool GENERAL, bool BIAS>
__device__ __attribute__((always_inline)) inline void item_run(const AttnParams &p, const FwdArgs &a, const TileList &tl, const RowMask &rm,
                                const elem8 (&qf)[D / 16], const OperandOffsets<D> &off, FwdSmem<D> &sm,
                                f32x16 (&o)[D / 32], float &m, float &l, const BiasLds &bl) {
    constexpr bool kMods = ALIBI || SOFTCAP || BIAS;
    static_assert(sizeof(sm.k) >= (kThreads / 64) * 32 * 2 * D, "output staging fits the K buffers");
    const float c_mul = kMods ? 1.0f : a.scale_log2;
    const int nsteps = a.spb * a.ntiles;  // 64-key steps
    auto reset = [&]() {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
        m = -INFINITY;
        l = 0.0f;
    };
    if (nsteps == 0) {  // nothing visible: out = 0, lse = -inf
        reset();
        store_item<D>(p, a, o, m, l, lds_addr(sm.k[0]));
        return;
    }
    auto step_key0 = [&](int t) { return row_step_key0(tl, a, t); };
    auto issue_k = [&](int t, int key0) {
        if (MODE == kGather || (MODE == kTable && a.doc))
            issue_ints_to_lds_at<kHalf>(lds_addr(sm.doc[t & 1]), a.doc + key0, rows_left<GENERAL>(p.npos - key0));
        issue_tile_to_lds<D, kSwzK, kHalf>(sm.k[t & 1], a.kb + (int64_t)key0 * p.k_st, p.k_st,
                                           rows_left<GENERAL>(p.T - key0));
    };
    auto issue_v = [&](int t, int key0) {
        issue_tile_to_lds<D, kSwzV, kHalf>(sm.v[t & 1], a.vb + (int64_t)key0 * p.v_st, p.v_st,
                                           rows_left<GENERAL>(p.T - key0));
    };
    // Row maximum of a step in the log2 domain (without score modifications
    // the scale is applied here and folded into the exponentials).
    auto step_max = [&](const f32x16 (&s)[2]) {
        const float mx = row_max(s);
        return kMods ? mx : mx * a.scale_log2;
    };
    // Moves the reference to the step maximum mx when it grew by more than
    // the threshold anywhere in the wave (o and l follow); returns the
    // reference the exponentials subtract.
    auto settle = [&](float mx) {
        if (__any(mx > m + kRescaleThreshold)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.0f : m_new));
            l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m = m_new;
        }
        return (m == -INFINITY) ? 0.0f : m;
    };

    f32x16 sa[2], sb[2];
    float mx;  // row maximum of the current step's scores
    const int k0 = a.first * a.kblk;
    int key_ahead = step1_key0(a);  // first key of step t+1 at the top of step t
    fwd_qk<D>(sm.k[0], off, qf, sa);
    row_mods<ALIBI, SOFTCAP, BIAS>(sa, k0, a.qpos, a.mk, bl);
    const bool table_docs = MODE == kTable && a.doc;
    if (a.nfull == 0) row_mask_flat<MODE>(lds_addr(sm.doc[0]), sa, k0, rm, table_docs);
    mx = step_max(sa);

    auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], int t, auto next_masked, auto first_step) {
        wait_vmcnt<0>();
        tile_barrier();
        OperandOffsets<D> offt = off;  // opaque per step: derived offsets are not hoisted
        asm volatile("" : "+v"(offt.k), "+v"(offt.v));
        // first keys of steps t+1 (carried from the previous step) and t+2
        const int key_next = key_ahead;
        key_ahead = (a.spb == 2 && ((t + 2) & 1)) ? key_ahead + kHalf : (t + 2 < nsteps ? step_key0(t + 2) : 0);
        if (t + 2 < nsteps) issue_k(t + 2, key_ahead);
        issue_v(t + 1, key_next);
        if (decltype(first_step)::value) reset();
        const float m_use = settle(mx);

        elem8 pb[2][2];
        fwd_qk<D>(sm.k[(t + 1) & 1], offt, qf, sn);
        fwd_exp(sc, pb, l, c_mul, m_use);
        fwd_pv<D>(sm.v[t & 1], offt, pb, o);
        row_mods<ALIBI, SOFTCAP, BIAS>(sn, key_next, a.qpos, a.mk, bl);
        if (decltype(next_masked)::value)
            row_mask_flat<MODE>(lds_addr(sm.doc[(t + 1) & 1]), sn, key_next, rm, table_docs);
        mx = step_max(sn);
        wait_lds_reads();  // this wave's reads of step t are done before the next barrier
    };
    // step 0 (unless it is the only one); its next step is the second half
    // of the first tile, or the second listed 64-key block
    if (nsteps > 1) {
        if (a.spb == 2 ? a.nfull > 0 : a.nfull > 1)
            step(sa, sb, 0, std::false_type(), std::true_type());
        else
            step(sa, sb, 0, std::true_type(), std::true_type());
        sa[0] = sb[0];  // the current scores live in sa between loops
        sa[1] = sb[1];
    } else {
        reset();
    }
    // Steps t < t_switch have a full next block.
    const int t_switch = min(max(a.spb * a.nfull - 1, 1), nsteps - 1);
    int t = 1;
    auto phase = [&](int t_end, auto next_masked) {
        for (; t + 1 < t_end; t += 2) {
            step(sa, sb, t, next_masked, std::false_type());
            step(sb, sa, t + 1, next_masked, std::false_type());
        }
        if (t < t_end) {
            step(sa, sb, t, next_masked, std::false_type());
            sa[0] = sb[0];
            sa[1] = sb[1];
            ++t;
        }
    };
    phase(t_switch, std::false_type());
    phase(nsteps - 1, std::true_type());
    // last step (t = nsteps - 1)
    wait_vmcnt<0>();
    tile_barrier();
    const float m_use = settle(mx);
    elem8 pb[2][2];
    fwd_exp(sa, pb, l, c_mul, m_use);
    fwd_pv<D>(sm.v[(nsteps - 1) & 1], off, pb, o);
    store_item<D>(p, a, o, m, l, lds_addr(sm.k[0]));
}

// One item per workgroup (workgroups past the last item exit at once).
// TABLE: a composed mask (its own kernel, so that the truth-table
// evaluation does not take registers from the other masks' kernels).
template <int D, bool ALIBI, bool SOFTCAP, bool TABLE, bool GENERAL>
__global__ __launch_bounds__(kThreads, (kWgPerCu<D, ALIBI || SOFTCAP>)) void fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) FwdSmem<D> sm;
    const ItemOrder ord(p, kQueues);
    const int k = ord.item(blockIdx.x / ord.Q);
    if (k >= ord.nitems) return;
    const int window = (p.mask_flags & BSM_MASK_WINDOW) ? load_uniform(p.window) : 0;
    int e, rem;
    ord.decode(k, e, rem);
    FwdArgs cur;
    item_args<ALIBI, SOFTCAP, GENERAL>(p, rem, load_rec(p.kv_order, e), cur);
    OperandOffsets<D> off;
    operand_offsets<D>(off);
    elem8 qf[D / 16];
    TileList tl;
    RowLoad rl;
    item_start<D, GENERAL>(p, sm, cur, qf, tl, rl);
    f32x16 o[D / 32];
    float m = -INFINITY, l = 0.0f;
    wait_vmcnt<0>();  // the item's first tiles, query rows, tile list and row data
    tile_barrier();
    RowMask rm;
    const BiasLds none = {};
    if (TABLE) {
        make_table_mask(p, cur.qpos, window, rl.docq, rm);
        item_run<D, ALIBI, SOFTCAP, kTable, GENERAL, false>(p, cur, tl, rm, qf, off, sm, o, m, l, none);
        return;
    }
    const int mode = finish_row_mask(p, cur.qpos, rl, window, rm);
    if (mode == kGather)
        item_run<D, ALIBI, SOFTCAP, kGather, GENERAL, false>(p, cur, tl, rm, qf, off, sm, o, m, l, none);
    else if (mode == kSinks)
        item_run<D, ALIBI, SOFTCAP, kSinks, GENERAL, false>(p, cur, tl, rm, qf, off, sm, o, m, l, none);
    else
        item_run<D, ALIBI, SOFTCAP, kPlain, GENERAL, false>(p, cur, tl, rm, qf, off, sm, o, m, l, none);
}

// The same with a relative-position bias table (no ALiBi), always on the
// general (clamped-copy) path.  The head's table goes to LDS: its loads are
// issued before the item's first tile copies, its LDS writes after the wait
// for them, before the barrier that starts the loop.  (A separate kernel
// body: routing fwd_kernel through a shared body changed the register
// allocation of its ALiBi and soft-cap instances.)
template <int D, bool SOFTCAP, bool TABLE>
__global__ __launch_bounds__(kThreads, (kWgPerCu<D, true>)) void fwd_bias_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) FwdSmem<D> sm;
    __shared__ float btab[kBiasMaxEntries];
    const ItemOrder ord(p, kQueues);
    const int k = ord.item(blockIdx.x / ord.Q);
    if (k >= ord.nitems) return;
    const int window = (p.mask_flags & BSM_MASK_WINDOW) ? load_uniform(p.window) : 0;
    int e, rem;
    ord.decode(k, e, rem);
    FwdArgs cur;
    item_args<false, SOFTCAP, true>(p, rem, load_rec(p.kv_order, e), cur);
    const int nb = 2 * p.bias_r + 1;
    float bstage[kBiasPerThread];
    stage_bias_load(p.bias + (int64_t)cur.h * nb, nb, bstage);
    OperandOffsets<D> off;
    operand_offsets<D>(off);
    elem8 qf[D / 16];
    TileList tl;
    RowLoad rl;
    item_start<D, true>(p, sm, cur, qf, tl, rl);
    f32x16 o[D / 32];
    float m = -INFINITY, l = 0.0f;
    wait_vmcnt<0>();  // the table, the item's first tiles, query rows, tile list and row data
    stage_bias_store(bstage, nb, mod_f<SOFTCAP>(cur.cap), lds_addr(btab));
    wait_lds_reads();  // (and writes) before the barrier
    tile_barrier();
    const BiasLds bl = {lds_addr(btab), p.bias_r};
    RowMask rm;
    if (TABLE) {
        make_table_mask(p, cur.qpos, window, rl.docq, rm);
        item_run<D, false, SOFTCAP, kTable, true, true>(p, cur, tl, rm, qf, off, sm, o, m, l, bl);
        return;
    }
    const int mode = finish_row_mask(p, cur.qpos, rl, window, rm);
    if (mode == kGather)
        item_run<D, false, SOFTCAP, kGather, true, true>(p, cur, tl, rm, qf, off, sm, o, m, l, bl);
    else if (mode == kSinks)
        item_run<D, false, SOFTCAP, kSinks, true, true>(p, cur, tl, rm, qf, off, sm, o, m, l, bl);
    else
        item_run<D, false, SOFTCAP, kPlain, true, true>(p, cur, tl, rm, qf, off, sm, o, m, l, bl);
}

template <int D, bool TABLE, bool GENERAL>
hipError_t launch_mods(const AttnParams &q, dim3 grid, bool alibi, bool cap, hipStream_t stream) {
    const dim3 block(kThreads);
    if (alibi && cap)
        hipLaunchKernelGGL((fwd_kernel<D, true, true, TABLE, GENERAL>), grid, block, 0, stream, q);
    else if (alibi)
        hipLaunchKernelGGL((fwd_kernel<D, true, false, TABLE, GENERAL>), grid, block, 0, stream, q);
    else if (cap)
        hipLaunchKernelGGL((fwd_kernel<D, false, true, TABLE, GENERAL>), grid, block, 0, stream, q);
    else
        hipLaunchKernelGGL((fwd_kernel<D, false, false, TABLE, GENERAL>), grid, block, 0, stream, q);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    AttnParams q = p;
    const dim3 grid(item_order(q)), block(kThreads);  // one workgroup per (queue, grab index) pair
    const bool alibi = p.mod_flags & BSM_MOD_ALIBI;
    const bool cap = p.mod_flags & BSM_MOD_SOFTCAP;
    if (p.mod_flags & BSM_MOD_BIAS) {
        const bool table = p.mask_flags & BSM_MASK_TABLE;
        if (table && cap)
            hipLaunchKernelGGL((fwd_bias_kernel<D, true, true>), grid, block, 0, stream, q);
        else if (table)
            hipLaunchKernelGGL((fwd_bias_kernel<D, false, true>), grid, block, 0, stream, q);
        else if (cap)
            hipLaunchKernelGGL((fwd_bias_kernel<D, true, false>), grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((fwd_bias_kernel<D, false, false>), grid, block, 0, stream, q);
        return hipGetLastError();
    }
    // composed masks always take the clamped copies (one kernel per mod)
    if (p.mask_flags & BSM_MASK_TABLE)
        return launch_mods<D, true, true>(q, grid, alibi, cap, stream);
    if (kv_ragged(p))
        return launch_mods<D, false, true>(q, grid, alibi, cap, stream);
    return launch_mods<D, false, false>(q, grid, alibi, cap, stream);
}

}  // namespace

// The build compiles this source once per head dimension (BSM_HEAD_DIM),
// so that the two halves compile in parallel; without it both are built.
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 64
hipError_t BSM_ELEM_FN(launch_attn_fwd_d64)(const AttnParams &p, hipStream_t stream) { return launch_d<64>(p, stream); }
#endif
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 128
hipError_t BSM_ELEM_FN(launch_attn_fwd_d128)(const AttnParams &p, hipStream_t stream) { return launch_d<128>(p, stream); }
#endif
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 256
hipError_t BSM_ELEM_FN(launch_attn_fwd_d256)(const AttnParams &p, hipStream_t stream) { return launch_d<256>(p, stream); }
#endif

}  // namespace bsm
