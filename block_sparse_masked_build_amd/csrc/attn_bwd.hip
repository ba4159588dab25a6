// Block-sparse masked attention, backward pass, for gfx950.
//
// Gradients of sum(out * dO) through the softmax, the mask and the score
// modifications (tutorial "FlexAttention in PyTorch", Pattern 3: ALiBi and
// soft-cap are differentiable and get a fused backward), visiting only the
// tiles the block mask lists (speedrun notes "FlexAttention", tile-summary
// paragraph).  With t the log2-domain score (after the modifications) and
// L = lse log2(e) from the forward, p = 2^(t - L) is recomputed and
//   Delta_q = <dO_q, out_q>
//   dS_qk   = p_qk (<dO_q, v_k> - Delta_q) * scale * (1 - tanh^2 if capped)
//   dQ = dS K,  dK = dS^T Q,  dV = P^T dO
// (dS is the gradient of the raw product q.k, hence the scale factor).
//
// Two kernels, no atomics (results are deterministic):
//  * dkdv_kernel: one workgroup of 4 waves per (batch, head, 128-key tile)
//    over the transposed (per key tile) full and partial query-tile lists.
//    Lane l of wave w owns key 32w + l%32 and keeps its K and V rows in
//    registers as the B operands of S = Q K^T and dP = dO V^T, so P and dS
//    come out of the matrix cores with the queries in registers -- the B
//    operand layout of dV^T += dO^T P and dK^T += Q^T dS.  Q and dO are
//    copied HBM -> LDS once per 64-query step and read row-wise (S, dP) and
//    transposed with ds_read_tr16_b64 (dV, dK) from the same copy.  The two
//    accumulators take 128 registers per lane at D = 128, so the kernel runs
//    one workgroup per CU with up to 512 registers per lane; at D = 64 it
//    fits 256 registers (no spill in its loops) and runs two;
//  * dq_kernel: one workgroup per (batch, head, 128-query tile) over the row
//    lists, lane = query as in the forward: S^T = K Q^T, dP^T = V dO^T,
//    dQ^T += K^T dS^T, with K and V copied per 64-key step and K read both
//    ways; two workgroups per CU.  It runs first and also computes Delta
//    and L of its rows from the row operands it loads anyway (plus the
//    output rows), writing them to the workspace that dkdv_kernel reads.
// Tile copies are asynchronous (global_load_lds) into double-buffered LDS,
// issued one step ahead, one barrier per step.  On partial tiles, 32 x 32
// blocks that hold no visible pair are skipped (no products at all), blocks
// that are entirely visible skip the elementwise test.
#include <type_traits>

#include "attn_common.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kHalf = 64;  // rows per pipeline step

// Soft-cap derivative from the log2-domain capped score t = cap tanh(.) log2 e:
// 1 - tanh^2, with tanh clamped so that masked scores (-inf) give 0.
__device__ inline float softcap_grad(float t, float inv_cap) {
    const float th = __builtin_amdgcn_fmed3f(t * (kLn2 * inv_cap), -1.0f, 1.0f);
    return 1.0f - th * th;
}

// Lane offsets of one pipeline step: those of a tile at LDS byte 0 moved by
// `base` (a tile base and buffer).  The swizzles XOR bits 5-7 of an offset,
// so adding a multiple of 256 before the XOR gives the same address as after
// it.  The result is opaque, so derived addresses are formed per step
// instead of being held in registers across the loop.
__device__ inline KvOffsets step_offsets(const KvOffsets &off, uint32_t base) {
    KvOffsets o;
    o.row = off.row + (int)base;
    o.tr = off.tr + (int)base;
    asm volatile("" : "+v"(o.row), "+v"(o.tr));
    return o;
}

// Start of pipeline step t (64 keys): with 128-key blocks (spb = 2) step t
// covers half t%2 of listed block t/2, with 64-key blocks (spb = 1) listed
// block t (full blocks first, then partial ones).
__device__ inline int step_row0(int t, int nfull, const int32_t *fidx, const int32_t *pidx, int nt, int spb) {
    const int it = spb == 2 ? t >> 1 : t;
    const int jj = clamp_tile(it < nfull ? load_uniform(fidx + it) : load_uniform(pidx + it - nfull), nt);
    return spb == 2 ? jj * kTile + (t & 1) * kHalf : jj * kHalf;
}

// ---------------------------------------------------------------- dQ

struct DqArgs {
    const elem_t *kb, *vb;
    int64_t k_st, v_st;
    const int32_t *fidx, *pidx, *doc;
    int nfull, nt, qpos;  // qpos: absolute position of this lane's query
    int qw0;              // absolute position of the wave's first query (BIAS)
    int kv_len, npos;
    int spb;              // 64-key steps per listed block: 2 (128-key blocks) or 1
    float scale, scale_log2, slope, cap, inv_cap;
    ModK mk;          // folded score-modification constants
    float l2, delta;  // this lane's query
};

// LDS of dq_kernel: double-buffered 64-key halves of K and V and the keys'
// document ids, addressed by byte address from the shared object.
template <int D>
struct DqSmem {
    elem_t k[2][kHalf * D];  // fkv swizzle
    elem_t v[2][kHalf * D];  // fkv swizzle
    int32_t doc[2][kHalf];
    float red[kThreads / 64];  // per-wave sums of the slope gradient
};

template <int D>
struct DqLds {
    static constexpr uint32_t kTileBytes = kHalf * D * 2;
    uint32_t k, v, doc;  // buffer 0; buffer 1 follows
};

// Bias-gradient sums of one wave (BIAS).  The gradient of table entry
// R + d sums g over the pairs at clipped distance d, so each step's
// 32 x 64 block of g is reduced along its diagonals.  Per 32-key block, the
// wave writes its 32 x 32 values to a private LDS scratch skewed so that
// each diagonal is one row (pair (query n, key c) at row n - c + 31, column
// n; positions no pair maps to stay zero), and lane j then sums row j in
// a fixed order and adds it to the wave's private accumulator: entries
// 0..2R for the clipped distances, then one slot per lane for distances
// beyond +R and one beyond -R.  Plain LDS reads and writes: within an
// instruction every lane has its own address, and a wave's LDS operations
// complete in order, so every sum is formed in program order and the
// item's partial row (bias_grad_flush) is identical from run to run.
constexpr int kDiagRows = 63;        // diagonals of a 32 x 32 block
constexpr int kDiagStride = 40;      // floats per scratch row: conflict-free skewed writes
constexpr int kDiagFloats = kDiagRows * kDiagStride;
constexpr int kBiasAccStride = kBiasMaxEntries + 128;

// qw0: absolute position of the wave's first query (lanes past Q_LEN carry
// g = 0, so their positions only decide where zeros are added).
__device__ inline void bias_grad_add(const float (&dsv)[2][16], int key0, int qw0, int R, uint32_t scr,
                                     uint32_t acc) {
    const int lane = threadIdx.x & 63, n = lane & 31, hl = lane >> 5;
    constexpr int kMaxC = 27;  // largest in-block key offset 8 g + e of a lane half
    // pair (n, c = 8 g + 4 hl + e) -> row n - c + 31, column n
    const uint32_t wbase = scr + 4u * (uint32_t)((n - 4 * hl - kMaxC + 31) * kDiagStride + n);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = (r >> 2) * 8 + (r & 3);
            lds_store<float>(wbase + 4u * (uint32_t)((kMaxC - c) * kDiagStride), dsv[kb][r]);
        }
        if (lane < kDiagRows) {
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 32 / 4; ++k) {
                const f32x4 v = lds_load<f32x4>(scr + 4u * (uint32_t)(lane * kDiagStride + 4 * k));
                sum += ((v[0] + v[1]) + v[2]) + v[3];
            }
            const int d = qw0 - key0 - 32 * kb + lane - 31;  // the row's distance q - kv
            const int idx = d > R ? 2 * R + 1 + lane : d < -R ? 2 * R + 65 + lane : d + R;
            const uint32_t a = acc + 4u * (uint32_t)idx;
            lds_store<float>(a, lds_load<float>(a) + sum);
        }
    }
}

// The item's partial row: entry j summed over the four waves in a fixed
// order, the overflow slots into the end entries.
__device__ inline void bias_grad_flush(uint32_t acc0, int R, float *row) {
    const int nb = 2 * R + 1;
    for (int j = threadIdx.x; j < nb; j += kThreads) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) v += lds_load<float>(acc0 + 4u * (uint32_t)(w * kBiasAccStride + j));
        if (j == nb - 1)
            for (int w = 0; w < kThreads / 64; ++w)
                for (int k = 0; k < 64; ++k) v += lds_load<float>(acc0 + 4u * (uint32_t)(w * kBiasAccStride + nb + k));
        if (j == 0)
            for (int w = 0; w < kThreads / 64; ++w)
                for (int k = 0; k < 64; ++k)
                    v += lds_load<float>(acc0 + 4u * (uint32_t)(w * kBiasAccStride + nb + 64 + k));
        row[j] = v;
    }
}

// SGRAD (with ALiBi only): also sums g_qk (k - q) over the visible keys of
// this lane's query into sg, the lane's share of dL/dslope[h] (g is dS
// before the scale, the gradient with respect to the score the ALiBi term
// is added to).  Per step, with the score at key key0 + 4 hl + c:
//   sum g (k - q) = sum g c + (key0 + 4 hl - q) sum g.
// GENERAL: the general kernel (see kv_ragged): the last key block's copies
// are clamped and the block width is read at run time; the other kernel has
// whole 128-key tiles compiled in (see the forward).
template <int D, bool ALIBI, bool SOFTCAP, bool SGRAD, int MODE, bool GENERAL, bool BIAS = false>
__device__ inline void dq_main(const DqArgs &a, const RowMask &rm, const elem8 (&qf)[D / 16],
                               const elem8 (&gf)[D / 16], const KvOffsets &off, const DqLds<D> &lds, int nsteps,
                               f32x16 (&dq)[D / 32], float &sg, const BiasLds &bl = {}, uint32_t bscr = 0,
                               uint32_t bacc = 0) {
    static_assert(!SGRAD || ALIBI, "the slope gradient needs the ALiBi term");
    constexpr bool kMods = ALIBI || SOFTCAP || BIAS;
    constexpr uint32_t kTB = DqLds<D>::kTileBytes;
    static_assert(kTB % 256 == 0, "buffer stride commutes with the swizzle");
    auto issue = [&](int t, int key0) {
        const uint32_t bf = t & 1;
        const int nk = GENERAL ? a.kv_len - key0 : kHalf;
        if (MODE == kGather || (MODE == kTable && a.doc))
            issue_ints_to_lds_at<kHalf>(lds.doc + bf * kHalf * 4, a.doc + key0, GENERAL ? a.npos - key0 : kHalf);
        issue_tile_to_lds_at<D, kSwzKV, kHalf>(lds.k + bf * kTB, a.kb + (int64_t)key0 * a.k_st, a.k_st, nk);
        issue_tile_to_lds_at<D, kSwzKV, kHalf>(lds.v + bf * kTB, a.vb + (int64_t)key0 * a.v_st, a.v_st, nk);
    };
    if (nsteps <= 0) return;
    int key0 = step_row0(0, a.nfull, a.fidx, a.pidx, a.nt, a.spb);
    issue(0, key0);
#pragma unroll 1
    for (int t = 0; t < nsteps; ++t) {
        wait_vmcnt<0>();
        tile_barrier();  // step t's tiles are visible; every wave is done with step t-1's buffers
        int key_next = 0;
        if (t + 1 < nsteps) {
            key_next = step_row0(t + 1, a.nfull, a.fidx, a.pidx, a.nt, a.spb);
            issue(t + 1, key_next);
        }
        const uint32_t bf = t & 1;
        // The buffer enters through the lane offsets, so that every read
        // addresses a fixed tile base plus one swizzled offset (the base
        // folds into the instruction's offset field).
        const uint32_t sk = lds.k, sv = lds.v;
        const KvOffsets offt = step_offsets(off, bf * kTB);
        const bool partial = (a.spb == 2 ? t >> 1 : t) >= a.nfull;
        bool skip[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            skip[kb] = partial && block_none_visible<MODE>(rm, key0 + kb * 32, key0 + kb * 32 + 31);

        // A skipped block takes scores of -inf (its probabilities are 0) and
        // dP of 0; the others start their sums from the first product.  The
        // fills are opaque so that the compiler keeps them on the skip branch
        // instead of writing them ahead of every step's products.
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (skip[kb]) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(s[kb][r]));  // -inf
                    asm volatile("v_mov_b32 %0, 0" : "=v"(dp[kb][r]));
                }
                continue;
            }
            const f32x16 zero = {};
            s[kb] = mfma32(read_rows_operand<D>(sk, offt, kb, 0), qf[0], zero);
            dp[kb] = mfma32(read_rows_operand<D>(sv, offt, kb, 0), gf[0], zero);
#pragma unroll
            for (int st = 1; st < D / 16; ++st) {
                s[kb] = mfma32(read_rows_operand<D>(sk, offt, kb, st), qf[st], s[kb]);
                dp[kb] = mfma32(read_rows_operand<D>(sv, offt, kb, st), gf[st], dp[kb]);
            }
        }
        row_mod_mask<ALIBI, SOFTCAP, MODE, BIAS>(lds.doc + bf * kHalf * 4, s, key0, a.qpos, a.mk, rm, partial,
                                                 MODE == kTable && a.doc, bl);
        elem8 dsb[2][2];
        float dsv[2][16];                // BIAS: the step's ds, added to the bias-gradient sums
        float sg_c = 0.0f, sg_s = 0.0f;  // SGRAD: sum ds c and sum ds over the step
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float tl = s[kb][r];
                const float pv = fast_exp2(kMods ? tl - a.l2 : __builtin_fmaf(tl, a.scale_log2, -a.l2));
                float ds = pv * (dp[kb][r] - a.delta);
                if (SOFTCAP) ds *= softcap_grad(tl, a.inv_cap);
                dsb[kb][r >> 3][r & 7] = static_cast<elem_t>(ds);
                if (BIAS) dsv[kb][r] = ds;
                if (SGRAD) {
                    sg_c = __builtin_fmaf(ds, (float)(kb * 32 + (r >> 2) * 8 + (r & 3)), sg_c);
                    sg_s += ds;
                }
            }
        if (SGRAD) {
            const int hl = (threadIdx.x & 63) >> 5;
            sg = __builtin_fmaf((float)(key0 + 4 * hl - a.qpos), sg_s, sg + sg_c);
        }
        if (BIAS) bias_grad_add(dsv, key0, a.qw0, bl.R, bscr, bacc);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (skip[kb]) continue;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    dq[db] = mfma32(read_cols_operand<D>(sk, offt, kb * 2 + s2, db), dsb[kb][s2], dq[db]);
        }
        wait_lds_reads();  // this wave's reads of step t are done before the next barrier
        key0 = key_next;
    }
}

// TABLE: a composed mask (its own kernel, so that the truth-table
// evaluation does not take registers from the other masks' kernels).
// BIAS: a relative-position bias table (no ALiBi; general path only),
// staged in LDS, with the per-wave bias-gradient sums (see bias_grad_add).
// The table, the four per-wave gradient arrays and diagonal scratches take
// 81 KB of LDS, so the BIAS
// kernels run one workgroup per CU.  (One kernel template: routing the
// kernel through a shared device-function body changed the register
// allocation of the other instances.)
template <int D, bool BIAS>
struct DqBiasSmem {
    float tab[BIAS ? kBiasMaxEntries : 1];
    float acc[BIAS ? (kThreads / 64) * kBiasAccStride : 1];
    float scr[BIAS ? (kThreads / 64) * kDiagFloats : 1];
};

template <int D, bool ALIBI, bool SOFTCAP, bool SGRAD, bool TABLE, bool GENERAL, bool BIAS>
__global__ __launch_bounds__(kThreads, (BIAS ? 1 : kWgPerCu<D, ALIBI || SOFTCAP>)) void dq_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) DqSmem<D> sm;
    __shared__ DqBiasSmem<D, BIAS> bsm;
    const uint32_t btab = lds_addr(bsm.tab), bacc = lds_addr(bsm.acc), bscr = lds_addr(bsm.scr);

    const int nt = p.nkb;  // key blocks of the row lists
    // Item: a query-tile row of the row work order (longest first) and a
    // head index, in the forward's item order.
    const ItemOrder ord(p, kQueues);
    const int k = ord.item(blockIdx.x / ord.Q);
    if (k >= ord.nitems) return;
    int e, rem;
    ord.decode(k, e, rem);
    const WorkRec rec = load_rec(p.kv_order, e);
    const int64_t row = min(max(rec.packed, 0), p.mask_b * p.nqt - 1);
    const int bm = (int)(row / p.nqt), i = (int)(row - (int64_t)bm * p.nqt);
    int b, h;
    head_of(p, rem, bm, b, h);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int qidx = i * kTile + wv * 32 + n;      // query index (past Q_LEN on a cut-short row)
    const int qrow = min(qidx, p.q_len - 1);       // the row this lane loads
    const int qpos = p.q_off + qrow;               // its absolute position

    const elem_t *qb = static_cast<const elem_t *>(p.q) + b * p.q_sb + h * p.q_sh;
    const elem_t *gb = static_cast<const elem_t *>(p.dout) + b * p.do_sb + h * p.do_sh;
    const elem_t *obr = static_cast<const elem_t *>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qrow * p.o_st;

    DqArgs a;
    a.kb = static_cast<const elem_t *>(p.k) + b * p.k_sb + h * p.k_sh;
    a.vb = static_cast<const elem_t *>(p.v) + b * p.v_sb + h * p.v_sh;
    a.k_st = p.k_st;
    a.v_st = p.v_st;
    a.nfull = min(max(rec.nfull, 0), nt);
    const int npart = min(max(rec.npart, 0), nt);
    a.fidx = p.full_kv_idx + row * nt;
    a.pidx = p.kv_idx + row * nt;
    a.doc = (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids + (int64_t)bm * p.npos : nullptr;
    a.nt = nt;
    a.qpos = qpos;
    a.kv_len = p.T;
    a.npos = p.npos;
    a.spb = GENERAL ? p.kb / kHalf : 2;  // 128-key tiles in the other kernel (see kv_ragged)
    a.scale = p.scale;
    a.scale_log2 = p.scale * kLog2e;
    a.slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    a.cap = SOFTCAP ? p.softcap : 1.0f;
    a.inv_cap = 1.0f / a.cap;
    a.mk = mod_k<SOFTCAP>(a.scale, a.slope, a.cap);
    const int64_t row_bh = ((int64_t)b * p.H + h) * p.q_len + qrow;
    const int nb = 2 * p.bias_r + 1;
    float bstage[kBiasPerThread];
    if (BIAS) stage_bias_load(p.bias + (int64_t)h * nb, nb, bstage);
    const float lse = p.lse[row_bh];
    a.l2 = lse == -INFINITY ? 0.0f : lse * kLog2e;
    const int nsteps = a.spb * (a.nfull + npart);

    RowMask rm;
    int mode = kTable;
    if (TABLE)
        make_table_mask(p, qpos, (p.mask_flags & BSM_MASK_WINDOW) ? load_uniform(p.window) : 0,
                        (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids[(int64_t)bm * p.npos + qpos] : 0, rm);
    else
        mode = make_row_mask(p, bm, qpos, rm);
    KvOffsets off;
    kv_offsets<D>(off);
    DqLds<D> lds;
    lds.k = lds_addr(&sm.k[0][0]);
    lds.v = lds_addr(&sm.v[0][0]);
    lds.doc = lds_addr(&sm.doc[0][0]);

    elem8 qf[D / 16], gf[D / 16];
    u32x4 of[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        qf[st] = *reinterpret_cast<const elem8 *>(qb + (int64_t)qrow * p.q_st + st * 16 + hl * 8);
        gf[st] = *reinterpret_cast<const elem8 *>(gb + (int64_t)qrow * p.do_st + st * 16 + hl * 8);
        of[st] = *reinterpret_cast<const u32x4 *>(obr + st * 16 + hl * 8);
    }
    // Delta = <dO, out> of this lane's query: each lane half holds half of
    // the row's columns.  Delta and L go to the workspace for dkdv_kernel.
    {
        float acc = 0.0f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc += elem_bits_to_float(u16_at(of[st], e)) * static_cast<float>(gf[st][e]);
        a.delta = acc + __shfl_xor(acc, 32);
        if (hl == 0 && qidx < p.q_len) {
            p.delta[row_bh] = a.delta;
            p.lse2[row_bh] = a.l2;
        }
    }
    // BIAS: lanes past Q_LEN (a copy of the last query) get p = 0, so that
    // they add nothing to the bias gradient; the table goes to LDS, and this
    // wave's gradient sums and diagonal scratch start at zero (the wave's
    // own LDS operations stay in order, the table is read after the first
    // step's barrier).
    const uint32_t bacc_w = bacc + 4u * (uint32_t)(wv * kBiasAccStride);
    const uint32_t bscr_w = bscr + 4u * (uint32_t)(wv * kDiagFloats);
    if (BIAS) {
        a.qw0 = p.q_off + i * kTile + wv * 32;
        if (qidx >= p.q_len) a.l2 = INFINITY;
        stage_bias_store(bstage, nb, mod_f<SOFTCAP>(a.cap), btab);
        for (int j = lane; j < kBiasAccStride; j += 64) lds_store<float>(bacc_w + 4u * (uint32_t)j, 0.0f);
        for (int j = lane; j < kDiagFloats; j += 64) lds_store<float>(bscr_w + 4u * (uint32_t)j, 0.0f);
        wait_lds_reads();  // (and writes)
    }
    const BiasLds bl = {btab, p.bias_r};
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;
    // No wait here: the first tile copies are issued while the row operands
    // load.  Loads complete in order, so the compiler's waits before their
    // uses only become more conservative with copies in flight, and the
    // first pipeline step waits for everything.

    float sg = 0.0f;
    if (TABLE)
        dq_main<D, ALIBI, SOFTCAP, SGRAD, kTable, GENERAL, BIAS>(a, rm, qf, gf, off, lds, nsteps, dq, sg, bl, bscr_w, bacc_w);
    else if (mode == kGather)
        dq_main<D, ALIBI, SOFTCAP, SGRAD, kGather, GENERAL, BIAS>(a, rm, qf, gf, off, lds, nsteps, dq, sg, bl, bscr_w, bacc_w);
    else if (mode == kSinks)
        dq_main<D, ALIBI, SOFTCAP, SGRAD, kSinks, GENERAL, BIAS>(a, rm, qf, gf, off, lds, nsteps, dq, sg, bl, bscr_w, bacc_w);
    else
        dq_main<D, ALIBI, SOFTCAP, SGRAD, kPlain, GENERAL, BIAS>(a, rm, qf, gf, off, lds, nsteps, dq, sg, bl, bscr_w, bacc_w);
    if (BIAS) {
        __syncthreads();  // every wave's sums are complete
        bias_grad_flush(bacc, p.bias_r, p.dbias_part + (((int64_t)b * p.H + h) * p.nqt + i) * nb);
    }

    // Slope gradient of the item: wave sums by a fixed butterfly, then the
    // four waves in order, one partial per (batch, head, query tile); lanes
    // past Q_LEN (a copy of the last query) do not count.
    if (SGRAD) {
        if (qidx >= p.q_len) sg = 0.0f;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sg += __shfl_xor(sg, o);
        if (lane == 0) sm.red[wv] = sg;
        __syncthreads();
        if (threadIdx.x == 0)
            p.dslope_part[((int64_t)b * p.H + h) * p.nqt + i] = ((sm.red[0] + sm.red[1]) + sm.red[2]) + sm.red[3];
    }

    // dQ rows of the wave, staged through the K buffers once every wave is
    // done with them (dS was accumulated without the scale).
    static_assert(sizeof(sm.k) >= (kThreads / 64) * 32 * 2 * D, "dQ staging fits the K buffers");
    tile_barrier();
    elem_t *dqp = static_cast<elem_t *>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)(qidx - n) * p.dq_st;
    store_rows_staged<D>(dqp, p.dq_st, dq, p.scale, lds.k + (uint32_t)(wv * 32 * 2 * D), p.q_len - (qidx - n));
}


// ---------------------------------------------------------------- dK, dV

// Column view of the mask for one key: the visible queries form [lo, hi]
// (causal: q >= key unless the key is in the prefix; window: q <= key + w - 1
// unless the key is a sink; the
// key's document).  Sinks only lift the window bound, so one interval always
// suffices.  In gather mode (documents not contiguous runs) the document is
// left out of the interval and dock holds the key's id for a per-query
// compare.
struct ColMask {
    int32_t lo, hi, dock;
    // composed mask (kTable): query indices from which the causal term holds
    // (q >= kpos) and below which the window term holds (q - kpos < window),
    // and the truth table shifted by the key's own sink and prefix bits, so
    // that bit (C + 2 Dc + 4 W) of it decides the pair
    int32_t cq0, wq1;
    uint32_t table;
};

// Column view of a composed mask for key kpos: [lo, hi] holds the queries
// that exist.
__device__ inline void make_col_table(const AttnParams &p, int bm, int kpos, int window, ColMask &cm) {
    cm.lo = 0;
    cm.hi = p.q_len - 1;
    cm.dock = (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids[(int64_t)bm * p.npos + kpos] : 0;
    const int64_t c0 = (int64_t)kpos - p.q_off;
    cm.cq0 = (int)(c0 < -(1 << 30) ? -(1 << 30) : c0);
    int64_t w1 = (p.mask_flags & BSM_MASK_WINDOW) ? (int64_t)kpos + window - p.q_off : -((int64_t)1 << 30);
    cm.wq1 = w1 < -(1 << 30) ? -(1 << 30) : (w1 > (1 << 30) ? (1 << 30) : (int)w1);
    const bool sink = (p.mask_flags & BSM_MASK_SINKS) && kpos < p.sinks;
    const bool pre = kpos < p.prefix;
    cm.table = p.table >> ((sink ? 8u : 0u) | (pre ? 16u : 0u));
}

__device__ inline bool make_col_mask(const AttnParams &p, int bm, int kpos, ColMask &cm) {
    cm.cq0 = 0;
    cm.wq1 = 0;
    cm.table = 0;
    // interval in absolute positions first, then in query indices
    int ds = 0, de = p.npos - 1;
    bool gather = false;
    cm.dock = 0;
    if (p.mask_flags & BSM_MASK_DOCUMENT) {
        const int32_t *dr = p.doc_range + ((int64_t)bm * p.npos + kpos) * 2;
        ds = dr[0];
        de = dr[1];
        gather = ds < 0;  // whole row flagged: every lane agrees
        if (gather) {
            ds = 0;
            de = p.npos - 1;
            cm.dock = p.doc_ids[(int64_t)bm * p.npos + kpos];
        }
    }
    // causal: queries from the key on, except for prefix keys, which every
    // query sees
    const int lo = max(((p.mask_flags & BSM_MASK_CAUSAL) && kpos >= p.prefix) ? kpos : 0, ds);
    int hi = de;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        const bool sink = (p.mask_flags & BSM_MASK_SINKS) && kpos < p.sinks;
        if (!sink) {
            int64_t whi = (int64_t)kpos + (int64_t)(*p.window) - 1;
            whi = whi < -1 ? -1 : (whi > p.npos - 1 ? p.npos - 1 : whi);
            hi = min(hi, (int)whi);
        }
    }
    cm.lo = max(lo - p.q_off, 0);
    cm.hi = min(hi - p.q_off, p.q_len - 1);
    return gather;
}

struct DkdvArgs {
    const elem_t *qb, *gb;
    int64_t q_st, do_st;
    const float *l2, *delta;  // this (batch, head)
    const int32_t *fidx, *pidx, *doc;  // doc: document ids from query 0's position on (NULL: none)
    int nfull, nt, kpos;      // nt: query tiles; kpos: this lane's key (clamped to KV_LEN - 1)
    int q_len, q_off;
    float scale, scale_log2, slope, cap, inv_cap;
    ModK mk;  // folded score-modification constants
};

// One pipeline step of dkdv is one listed 128-query tile.
template <int D>
struct DkdvSmem {
    elem_t q[2][kTile * D];   // queries (fkv swizzle)
    elem_t g[2][kTile * D];   // output gradients (fkv swizzle)
    float l2[2][kTile];
    float delta[2][kTile];
    int32_t doc[2][kTile];
};

// Byte addresses of buffer 0 of each DkdvSmem field (buffer 1 follows).
template <int D>
struct DkdvLds {
    static constexpr uint32_t kTileBytes = kTile * D * 2;
    uint32_t q, g, l2, delta, doc;
};

// Row operands (A of S = Q K^T and dP = dO V^T) of query block b.
template <int D>
__device__ inline void dkdv_read_rows(const KvOffsets &oq, const KvOffsets &og, int b, elem8 (&rq)[D / 16],
                                      elem8 (&rg)[D / 16]) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        rq[st] = read_rows_operand<D>(0, oq, b, st);
        rg[st] = read_rows_operand<D>(0, og, b, st);
    }
}

template <int D>
__device__ inline void dkdv_sdp(const elem8 (&rq)[D / 16], const elem8 (&rg)[D / 16], const elem8 (&kf)[D / 16],
                                const elem8 (&vf)[D / 16], f32x16 &s, f32x16 &dp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        s = mfma32(rq[st], kf[st], s);
        dp = mfma32(rg[st], vf[st], dp);
    }
}

// Bias terms of the column view (BIAS): query offset c = 8 (r/4) + r%4 <= 27
// of the block at distance t0 + c (t0 = the block's first query position in
// this lane half minus the key); one LDS read per term at a fixed offset
// when the wave's distances lie inside [-R, R], clipped per score otherwise.
constexpr int kColMaxOffset = 27;  // 3 * 8 + 3

__device__ inline void col_bias(float (&bt)[16], int t0, const BiasLds &bl) {
    if (__all(t0 >= -bl.R && t0 + kColMaxOffset <= bl.R)) {
        const uint32_t a0 = bl.tab + 4u * (uint32_t)(t0 + bl.R);
#pragma unroll
        for (int r = 0; r < 16; ++r) bt[r] = lds_load<float>(a0 + 4u * (uint32_t)((r >> 2) * 8 + (r & 3)));
    } else {
        const uint32_t a0 = bl.tab + 4u * (uint32_t)bl.R;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = min(max(t0 + (r >> 2) * 8 + (r & 3), -bl.R), bl.R);
            bt[r] = lds_load<float>(a0 + 4u * (uint32_t)d);  // d < 0 wraps back below a0
        }
    }
}

// p and dS / scale of query block b (queries q0 + 32 b + 4 hl + 8 (r/4) + r%4
// in register r) as the bf16 B operands of the dV and dK products.
// CMODE: kPlain (the interval), kGather (interval and a per-query document
// compare) or kTable (a composed mask, [lo, hi] the queries that exist).
template <bool ALIBI, bool SOFTCAP, int CMODE, bool MASKED, bool BIAS>
__device__ inline void dkdv_grads(const DkdvArgs &a, const ColMask &cm, uint32_t sl2, uint32_t sdl,
                                  uint32_t sdoc, int b, int q0, const f32x16 &s, const f32x16 &dp,
                                  elem8 (&pb)[2], elem8 (&dsb)[2], const BiasLds &bl) {
    constexpr bool kMods = ALIBI || SOFTCAP || BIAS;
    const int hl = (threadIdx.x & 63) >> 5;
    const int qbase = q0 + b * 32 + 4 * hl;
    int lo_t = cm.hi >= cm.lo ? cm.lo - qbase : 1 << 30;  // empty interval: no offset matches
    const int span = cm.hi >= cm.lo ? cm.hi - cm.lo : 0;
    // ALiBi term of the score at query offset c: -slope_f (q - kpos) =
    // c ns + n with ns = -slope_f and n = ns (qbase + q_off - kpos), the
    // query's absolute position being q_off + its index.
    float ns = -a.mk.slope_f;
    float n = ALIBI ? ns * (float)(qbase + a.q_off - a.kpos) : 0.0f;
    asm volatile("" : "+v"(lo_t), "+v"(n), "+v"(ns));
    // composed mask, query offset c: causal for c >= tc, window for c < tw
    int tc = 0, tw = 0;
    if (CMODE == kTable && MASKED) {
        tc = cm.cq0 - qbase;
        tw = cm.wq1 - qbase;
        asm volatile("" : "+v"(tc), "+v"(tw));
    }
    const bool docs = CMODE == kGather || (CMODE == kTable && a.doc);
    float bt[16];
    if (BIAS) col_bias(bt, qbase + a.q_off - a.kpos, bl);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int ql4 = b * 32 + g * 8 + hl * 4;
        const f32x4 L = lds_load<f32x4>(sl2 + 4 * ql4);
        const f32x4 Dl = lds_load<f32x4>(sdl + 4 * ql4);
        i32x4 dq4 = {0, 0, 0, 0};
        if (docs && MASKED) dq4 = lds_load<i32x4>(sdoc + 4 * ql4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = g * 4 + e;
            const int c = g * 8 + e;
            float pv, tl = 0.0f;
            if (kMods) {
                const float bias = ALIBI ? __builtin_fmaf((float)c, ns, n) : BIAS ? bt[r] : 0.0f;
                tl = mod_apply<ALIBI || BIAS, SOFTCAP>(s[r], bias, a.mk);
                pv = fast_exp2(tl - L[e]);
            } else {
                pv = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, -L[e]));
            }
            if (MASKED) {
                bool vis = (uint32_t)(c - lo_t) <= (uint32_t)span;
                const int dqv = e == 0 ? dq4.x : e == 1 ? dq4.y : e == 2 ? dq4.z : dq4.w;
                if (CMODE == kTable) {
                    const uint32_t idx = (c >= tc ? 1u : 0u) | (docs && dqv == cm.dock ? 2u : 0u) | (c < tw ? 4u : 0u);
                    vis = vis && ((cm.table >> idx) & 1u);
                } else if (CMODE == kGather) {
                    vis = vis && dqv == cm.dock;
                }
                pv = vis ? pv : 0.0f;
            }
            float ds = pv * (dp[r] - Dl[e]);
            if (SOFTCAP) ds *= softcap_grad(tl, a.inv_cap);
            pb[r >> 3][r & 7] = static_cast<elem_t>(pv);
            dsb[r >> 3][r & 7] = static_cast<elem_t>(ds);
        }
    }
}

// Transposed operands (A of dV^T += dO^T P and dK^T += Q^T dS) of block b.
template <int D>
__device__ inline void dkdv_read_cols(const KvOffsets &oq, const KvOffsets &og, int b, elem8 (&tq)[2][D / 32],
                                      elem8 (&tg)[2][D / 32]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            tg[s2][db] = read_cols_operand<D>(0, og, b * 2 + s2, db);
            tq[s2][db] = read_cols_operand<D>(0, oq, b * 2 + s2, db);
        }
}

template <int D>
__device__ inline void dkdv_acc(const elem8 (&tq)[2][D / 32], const elem8 (&tg)[2][D / 32], const elem8 (&pb)[2],
                                const elem8 (&dsb)[2], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            dv[db] = mfma32(tg[s2][db], pb[s2], dv[db]);
            dk[db] = mfma32(tq[s2][db], dsb[s2], dk[db]);
        }
}

// One 128-query tile against the wave's 32 keys, software-pipelined over its
// four 32-query blocks: the S / dP products of block b+1 are issued next to
// the gradient arithmetic of block b, and the row operands of block b+2 are
// read during the dV / dK products of block b.
template <int D, bool ALIBI, bool SOFTCAP, int CMODE, bool MASKED, bool BIAS>
__device__ inline void dkdv_tile(const DkdvArgs &a, const ColMask &cm, const elem8 (&kf)[D / 16],
                                 const elem8 (&vf)[D / 16], const KvOffsets &oq, const KvOffsets &og,
                                 uint32_t sl2, uint32_t sdl, uint32_t sdoc, int q0,
                                 f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const BiasLds &bl) {
    constexpr int NB = kTile / 32;
    elem8 rq[D / 16], rg[D / 16];
    f32x16 s[2], dp[2];
    dkdv_read_rows<D>(oq, og, 0, rq, rg);
    dkdv_sdp<D>(rq, rg, kf, vf, s[0], dp[0]);
    dkdv_read_rows<D>(oq, og, 1, rq, rg);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int cur = b & 1;
        if (b + 1 < NB) dkdv_sdp<D>(rq, rg, kf, vf, s[cur ^ 1], dp[cur ^ 1]);
        elem8 pb[2], dsb[2];
        dkdv_grads<ALIBI, SOFTCAP, CMODE, MASKED, BIAS>(a, cm, sl2, sdl, sdoc, b, q0, s[cur], dp[cur], pb, dsb, bl);
        elem8 tq[2][D / 32], tg[2][D / 32];
        dkdv_read_cols<D>(oq, og, b, tq, tg);
        if (b + 2 < NB) dkdv_read_rows<D>(oq, og, b + 2, rq, rg);
        dkdv_acc<D>(tq, tg, pb, dsb, dk, dv);
        __builtin_amdgcn_sched_barrier(0);  // keep each block's reads and products in their own window
    }
}

// GENERAL: Q_LEN is not a multiple of 128, so the last query tile's copies
// are clamped (compiled out otherwise).
template <int D, bool ALIBI, bool SOFTCAP, int CMODE, bool GENERAL, bool BIAS = false>
__device__ inline void dkdv_main(const DkdvArgs &a, const ColMask &cm, const elem8 (&kf)[D / 16],
                                 const elem8 (&vf)[D / 16], const KvOffsets &off, const DkdvLds<D> &lds,
                                 int ntiles, f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const BiasLds &bl = {}) {
    constexpr uint32_t kTB = DkdvLds<D>::kTileBytes, kWB = kTile * 4;
    static_assert(kTB % 256 == 0, "buffer stride commutes with the swizzle");
    auto tile_q0 = [&](int it) {
        return clamp_tile(it < a.nfull ? load_uniform(a.fidx + it) : load_uniform(a.pidx + it - a.nfull), a.nt) *
               kTile;
    };
    auto issue = [&](int t, int q0) {
        // rows past Q_LEN repeat the last query's
        const uint32_t bf = t & 1;
        const int nq = GENERAL ? a.q_len - q0 : kTile;
        issue_ints_to_lds_at<kTile>(lds.l2 + bf * kWB, reinterpret_cast<const int32_t *>(a.l2 + q0), nq);
        issue_ints_to_lds_at<kTile>(lds.delta + bf * kWB, reinterpret_cast<const int32_t *>(a.delta + q0), nq);
        if (CMODE == kGather || (CMODE == kTable && a.doc))
            issue_ints_to_lds_at<kTile>(lds.doc + bf * kWB, a.doc + q0, nq);
        issue_tile_to_lds_at<D, kSwzKV, kTile>(lds.q + bf * kTB, a.qb + (int64_t)q0 * a.q_st, a.q_st, nq);
        issue_tile_to_lds_at<D, kSwzKV, kTile>(lds.g + bf * kTB, a.gb + (int64_t)q0 * a.do_st, a.do_st, nq);
    };
    if (ntiles <= 0) return;
    int q0 = tile_q0(0);
    issue(0, q0);
    // One step per listed tile.  Full tiles and partial tiles run in two
    // loops of straight-line code, so that the accumulators never pass
    // through a branch merge (which makes the register allocator copy them).
    auto step = [&](int t, auto masked) {
        wait_vmcnt<0>();
        tile_barrier();  // tile t is visible; every wave is done with tile t-1's buffers
        int q_next = 0;
        if (t + 1 < ntiles) {
            q_next = tile_q0(t + 1);
            issue(t + 1, q_next);
        }
        const uint32_t bf = t & 1;
        // Tile base and buffer enter through the lane offsets (see dq_main):
        // the second tile's base lies beyond a read's 16-bit offset field.
        const KvOffsets oq = step_offsets(off, lds.q + bf * kTB), og = step_offsets(off, lds.g + bf * kTB);
        dkdv_tile<D, ALIBI, SOFTCAP, CMODE, decltype(masked)::value, BIAS>(
            a, cm, kf, vf, oq, og, lds.l2 + bf * kWB, lds.delta + bf * kWB, lds.doc + bf * kWB, q0, dk, dv, bl);
        wait_lds_reads();  // this wave's reads of tile t are done before the next barrier
        q0 = q_next;
    };
#pragma unroll 1
    for (int t = 0; t < a.nfull; ++t) step(t, std::false_type());
#pragma unroll 1
    for (int t = a.nfull; t < ntiles; ++t) step(t, std::true_type());
}

// BIAS: a relative-position bias table (no ALiBi), staged in LDS at btab.
template <int D, bool ALIBI, bool SOFTCAP, bool TABLE, bool GENERAL, bool BIAS>
__device__ __attribute__((always_inline)) inline void dkdv_body(const AttnParams &p, DkdvSmem<D> &sm,
                                                                uint32_t btab) {
    const int nt = p.nt;
    const int wg = p.col_chunked ? col_remap(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= p.B * p.H * nt) return;  // past the work (chunked placement; whole workgroup)
    const int bh = wg / nt;
    const int j = wg % nt;  // early key tiles first: under a causal mask they carry the most tiles
    const int b = bh / p.H, h = bh % p.H;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int kidx = j * kTile + wv * 32 + n;    // key (past KV_LEN on a cut-short tile)
    const int kpos = min(kidx, p.T - 1);         // the key this lane loads

    const elem_t *kb = static_cast<const elem_t *>(p.k) + b * p.k_sb + h * p.k_sh;
    const elem_t *vb = static_cast<const elem_t *>(p.v) + b * p.v_sb + h * p.v_sh;
    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t col = (int64_t)bm * nt + j;
    const int nb = 2 * p.bias_r + 1;
    float bstage[kBiasPerThread];
    if (BIAS) stage_bias_load(p.bias + (int64_t)h * nb, nb, bstage);

    DkdvArgs a;
    a.qb = static_cast<const elem_t *>(p.q) + b * p.q_sb + h * p.q_sh;
    a.gb = static_cast<const elem_t *>(p.dout) + b * p.do_sb + h * p.do_sh;
    a.q_st = p.q_st;
    a.do_st = p.do_st;
    a.l2 = p.lse2 + ((int64_t)b * p.H + h) * p.q_len;
    a.delta = p.delta + ((int64_t)b * p.H + h) * p.q_len;
    a.nfull = min(max(load_uniform(p.full_q_num + col), 0), p.nqt);
    const int npart = min(max(load_uniform(p.q_num + col), 0), p.nqt);
    a.fidx = p.full_q_idx + col * p.nqt;
    a.pidx = p.q_idx + col * p.nqt;
    a.doc = (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids + (int64_t)bm * p.npos + p.q_off : nullptr;
    a.nt = p.nqt;
    a.kpos = kpos;
    a.q_len = p.q_len;
    a.q_off = p.q_off;
    a.scale = p.scale;
    a.scale_log2 = p.scale * kLog2e;
    a.slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    a.cap = SOFTCAP ? p.softcap : 1.0f;
    a.inv_cap = 1.0f / a.cap;
    a.mk = mod_k<SOFTCAP>(a.scale, a.slope, a.cap);
    const int ntiles = a.nfull + npart;

    ColMask cm;
    bool gather = false;
    if (TABLE)
        make_col_table(p, bm, kpos, (p.mask_flags & BSM_MASK_WINDOW) ? load_uniform(p.window) : 0, cm);
    else
        gather = make_col_mask(p, bm, kpos, cm);
    // LDS is addressed by byte address, taken here from the shared object.
    DkdvLds<D> lds;
    lds.q = lds_addr(&sm.q[0][0]);
    lds.g = lds_addr(&sm.g[0][0]);
    lds.l2 = lds_addr(&sm.l2[0][0]);
    lds.delta = lds_addr(&sm.delta[0][0]);
    lds.doc = lds_addr(&sm.doc[0][0]);
    KvOffsets off;
    kv_offsets<D>(off);

    elem8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        kf[st] = *reinterpret_cast<const elem8 *>(kb + (int64_t)kpos * p.k_st + st * 16 + hl * 8);
        vf[st] = *reinterpret_cast<const elem8 *>(vb + (int64_t)kpos * p.v_st + st * 16 + hl * 8);
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[db][r] = 0.0f;
            dv[db][r] = 0.0f;
        }
    // No wait here: the first tile copies are issued while the key rows
    // load (see dq_kernel).  BIAS: the table's LDS writes are done before
    // the first step's barrier, after which it is read.
    if (BIAS) {
        stage_bias_store(bstage, nb, mod_f<SOFTCAP>(a.cap), btab);
        wait_lds_reads();  // (and writes)
    }
    const BiasLds bl = {btab, p.bias_r};
    if (TABLE)
        dkdv_main<D, ALIBI, SOFTCAP, kTable, GENERAL, BIAS>(a, cm, kf, vf, off, lds, ntiles, dk, dv, bl);
    else if (gather)
        dkdv_main<D, ALIBI, SOFTCAP, kGather, GENERAL, BIAS>(a, cm, kf, vf, off, lds, ntiles, dk, dv, bl);
    else
        dkdv_main<D, ALIBI, SOFTCAP, kPlain, GENERAL, BIAS>(a, cm, kf, vf, off, lds, ntiles, dk, dv, bl);

    // dK and dV rows of the wave, staged through the query and output-gradient
    // buffers once every wave is done with them (dS was accumulated without
    // the scale).
    static_assert(sizeof(sm.q) >= (kThreads / 64) * 32 * 2 * D, "dK staging fits the query buffers");
    static_assert(sizeof(sm.g) >= (kThreads / 64) * 32 * 2 * D, "dV staging fits the gradient buffers");
    tile_barrier();
    const uint32_t slice = (uint32_t)(wv * 32 * 2 * D);
    const int k0w = kidx - n;  // the wave's first key
    elem_t *dkp = static_cast<elem_t *>(p.dk) + b * p.dk_sb + h * p.dk_sh + (int64_t)k0w * p.dk_st;
    elem_t *dvp = static_cast<elem_t *>(p.dv) + b * p.dv_sb + h * p.dv_sh + (int64_t)k0w * p.dv_st;
    store_rows_staged<D>(dkp, p.dk_st, dk, p.scale, lds.q + slice, p.T - k0w);
    store_rows_staged<D>(dvp, p.dv_st, dv, 1.0f, lds.g + slice, p.T - k0w);
}

template <int D, bool ALIBI, bool SOFTCAP, bool TABLE, bool GENERAL>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void dkdv_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) DkdvSmem<D> sm;
    dkdv_body<D, ALIBI, SOFTCAP, TABLE, GENERAL, false>(p, sm, 0);
}

template <int D, bool SOFTCAP, bool TABLE>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void dkdv_bias_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) DkdvSmem<D> sm;
    __shared__ float btab[kBiasMaxEntries];
    dkdv_body<D, false, SOFTCAP, TABLE, true, true>(p, sm, lds_addr(btab));
}

// ---------------------------------------------------------------- dK, dV at D = 256
//
// At D = 256 the 32-key layout of dkdv_kernel would need about 900 registers
// (dK, dV and the K/V operands alone take 640) and 256 KB of LDS for its
// 128-query double buffers.  dkdv256_kernel instead gives each of four waves
// 16 keys (a workgroup takes half a 128-key tile, 64 keys, and reads that
// tile's column lists) and works in v_mfma_f32_16x16x32 blocks:
//  * S = Q K^T and dP = dO V^T per 16 queries x the wave's 16 keys, with the
//    K and V rows as B operands (lane = key l%16); lane l gets queries
//    4 (l/16) + 0..3 of the block in its four result registers;
//  * two such blocks give the eight query values a lane feeds as the B
//    operand (k slots) of dV^T += dO^T P and dK^T += Q^T dS over 32
//    queries: queries 4G..4G+3 and 16+4G..16+4G+3 for lane group
//    G = l/16, the order the transposing reads of dO and Q produce;
//  * each listed 128-query tile is taken in two 64-query steps through
//    double-buffered LDS (128 KB): one workgroup per CU, one wave per SIMD,
//    about 300 registers.
// 16x16x32 operand layout (wave64): A row i, k-slot kk in lane i + 16 (kk/8),
// element kk%8; B column j, k-slot kk in lane j + 16 (kk/8); D row i, column
// j in lane j + 16 (i/4), register i%4.
constexpr int kQStep = 64;  // queries per pipeline step

__device__ inline f32x4 mfma16(const elem8 &a, const elem8 &b, const f32x4 &c) {
#ifdef BSM_ELEM_FP16
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
#else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
#endif
}

// Per-lane LDS byte offsets of the 16x16x32 operands of an fkv tile (fkv
// swizzles the 16-byte chunk index by the row's low four bits):
//   row: A operand [16 rows][32 columns]: row 16 rb + l%16, columns
//        32 st + 8 (l/16) .. +7, logical chunk (l/16) + 4 st; the XOR with
//        fkv commutes with the 4 st bits: rb 16 rows + (row ^ (st << 6));
//   tr:  A operand [16 columns][32 rows] of the tile transposed, columns
//        16 db + l%16, rows 4G..4G+3 (+16: 16+4G..) of a 32-row block with
//        ds_read_tr16_b64: lane j of a 16-lane group G addresses row
//        4G + j/4, columns 16 db + 4 (j%4) .. +3, i.e. logical chunk
//        2 db + (j%4)/2, half j%2; the db part is an XOR of bits 5 and up.
struct Kv16Offsets {
    int row;
    int tr;
};

template <int D>
__device__ inline void kv16_offsets(Kv16Offsets &off) {
    using L = TileLayout<D>;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    off.row = r * L::kRowBytes + ((g ^ L::fkv(r)) << 4);
    const int tr_r = 4 * g + (r >> 2);
    off.tr = tr_r * L::kRowBytes + ((((r & 3) >> 1) ^ L::fkv(tr_r)) << 4) + ((r & 1) << 3);
}

__device__ inline Kv16Offsets step_offsets16(const Kv16Offsets &off, uint32_t base) {
    Kv16Offsets o;
    o.row = off.row + (int)base;
    o.tr = off.tr + (int)base;
    asm volatile("" : "+v"(o.row), "+v"(o.tr));
    return o;
}

template <int D>
__device__ inline elem8 read_rows16(const Kv16Offsets &off, int rb, int st) {
    return lds_load<elem8>((uint32_t)(rb * 16 * TileLayout<D>::kRowBytes + (off.row ^ (st << 6))));
}

template <int D>
__device__ inline elem8 read_cols16(const Kv16Offsets &off, int qb, int db) {
    constexpr int kRB = TileLayout<D>::kRowBytes;
    const uint32_t a = (uint32_t)(qb * 32 * kRB + (off.tr ^ (db << 5)));
    const i16x4 lo = ds_read_tr16_at(a);
    const i16x4 hi = ds_read_tr16_at(a + 16 * kRB);
    return __builtin_bit_cast(elem8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// p and dS / scale of 16-query block b16 of the step (queries
// q0 + 16 b16 + 4 G + e in register e): as dkdv_grads, for four registers.
template <bool ALIBI, bool SOFTCAP, int CMODE, bool MASKED>
__device__ inline void dkdv16_grads(const DkdvArgs &a, const ColMask &cm, uint32_t sl2, uint32_t sdl,
                                    uint32_t sdoc, int b16, int q0, const f32x4 &s, const f32x4 &dp,
                                    float (&pv_out)[4], float (&ds_out)[4]) {
    constexpr bool kMods = ALIBI || SOFTCAP;
    const int G = (threadIdx.x & 63) >> 4;
    const int qbase = q0 + b16 * 16 + 4 * G;
    int lo_t = cm.hi >= cm.lo ? cm.lo - qbase : 1 << 30;  // empty interval: no offset matches
    const int span = cm.hi >= cm.lo ? cm.hi - cm.lo : 0;
    float ns = -a.mk.slope_f;
    float n = ALIBI ? ns * (float)(qbase + a.q_off - a.kpos) : 0.0f;
    asm volatile("" : "+v"(lo_t), "+v"(n), "+v"(ns));
    int tc = 0, tw = 0;
    if (CMODE == kTable && MASKED) {
        tc = cm.cq0 - qbase;
        tw = cm.wq1 - qbase;
        asm volatile("" : "+v"(tc), "+v"(tw));
    }
    const bool docs = CMODE == kGather || (CMODE == kTable && a.doc);
    const int ql4 = b16 * 16 + 4 * G;
    const f32x4 L = lds_load<f32x4>(sl2 + 4 * ql4);
    const f32x4 Dl = lds_load<f32x4>(sdl + 4 * ql4);
    i32x4 dq4 = {0, 0, 0, 0};
    if (docs && MASKED) dq4 = lds_load<i32x4>(sdoc + 4 * ql4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float pv, tl = 0.0f;
        if (kMods) {
            const float bias = ALIBI ? __builtin_fmaf((float)e, ns, n) : 0.0f;
            tl = mod_apply<ALIBI, SOFTCAP>(s[e], bias, a.mk);
            pv = fast_exp2(tl - L[e]);
        } else {
            pv = fast_exp2(__builtin_fmaf(s[e], a.scale_log2, -L[e]));
        }
        if (MASKED) {
            bool vis = (uint32_t)(e - lo_t) <= (uint32_t)span;
            const int dqv = e == 0 ? dq4.x : e == 1 ? dq4.y : e == 2 ? dq4.z : dq4.w;
            if (CMODE == kTable) {
                const uint32_t idx = (e >= tc ? 1u : 0u) | (docs && dqv == cm.dock ? 2u : 0u) | (e < tw ? 4u : 0u);
                vis = vis && ((cm.table >> idx) & 1u);
            } else if (CMODE == kGather) {
                vis = vis && dqv == cm.dock;
            }
            pv = vis ? pv : 0.0f;
        }
        float ds = pv * (dp[e] - Dl[e]);
        if (SOFTCAP) ds *= softcap_grad(tl, a.inv_cap);
        pv_out[e] = pv;
        ds_out[e] = ds;
    }
}

// One 64-query step against the wave's 16 keys, in two 32-query blocks.
template <int D, bool ALIBI, bool SOFTCAP, int CMODE, bool MASKED>
__device__ inline void dkdv16_step(const DkdvArgs &a, const ColMask &cm, const elem8 (&kf)[D / 32],
                                   const elem8 (&vf)[D / 32], const Kv16Offsets &oq, const Kv16Offsets &og,
                                   uint32_t sl2, uint32_t sdl, uint32_t sdoc, int q0, f32x4 (&dk)[D / 16],
                                   f32x4 (&dv)[D / 16]) {
#pragma unroll
    for (int qb = 0; qb < kQStep / 32; ++qb) {
        float pv[2][4], dsv[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b16 = qb * 2 + h;
            f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < D / 32; ++st) {
                s = mfma16(read_rows16<D>(oq, b16, st), kf[st], s);
                dp = mfma16(read_rows16<D>(og, b16, st), vf[st], dp);
            }
            dkdv16_grads<ALIBI, SOFTCAP, CMODE, MASKED>(a, cm, sl2, sdl, sdoc, b16, q0, s, dp, pv[h], dsv[h]);
        }
        elem8 pb, dsb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pb[e] = static_cast<elem_t>(pv[0][e]);
            pb[4 + e] = static_cast<elem_t>(pv[1][e]);
            dsb[e] = static_cast<elem_t>(dsv[0][e]);
            dsb[4 + e] = static_cast<elem_t>(dsv[1][e]);
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            dv[db] = mfma16(read_cols16<D>(og, qb, db), pb, dv[db]);
            dk[db] = mfma16(read_cols16<D>(oq, qb, db), dsb, dk[db]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep each block's reads and products in their own window
    }
}

// LDS of dkdv256_kernel: double-buffered 64-query halves of the listed query
// tiles (queries and output gradients) and their L, Delta and document ids.
template <int D>
struct Dkdv16Smem {
    elem_t q[2][kQStep * D];  // fkv swizzle
    elem_t g[2][kQStep * D];
    float l2[2][kQStep];
    float delta[2][kQStep];
    int32_t doc[2][kQStep];
};

// The step loop: two 64-query steps per listed 128-query tile (full tiles
// first), copies issued one step ahead, one barrier per step.
template <int D, bool ALIBI, bool SOFTCAP, int CMODE, bool GENERAL>
__device__ inline void dkdv16_main(const DkdvArgs &a, const ColMask &cm, const elem8 (&kf)[D / 32],
                                   const elem8 (&vf)[D / 32], const Kv16Offsets &off, Dkdv16Smem<D> &sm,
                                   int ntiles, f32x4 (&dk)[D / 16], f32x4 (&dv)[D / 16]) {
    constexpr uint32_t kTB = kQStep * D * 2, kWB = kQStep * 4;
    static_assert(kTB % 256 == 0, "buffer stride commutes with the swizzle");
    const uint32_t lq = lds_addr(&sm.q[0][0]), lg = lds_addr(&sm.g[0][0]);
    const uint32_t ll2 = lds_addr(&sm.l2[0][0]), ldl = lds_addr(&sm.delta[0][0]), ldoc = lds_addr(&sm.doc[0][0]);
    auto step_q0 = [&](int t) {
        const int it = t >> 1;
        return clamp_tile(it < a.nfull ? load_uniform(a.fidx + it) : load_uniform(a.pidx + it - a.nfull), a.nt) *
                   kTile + (t & 1) * kQStep;
    };
    auto issue = [&](int t, int q0) {
        // rows past Q_LEN repeat the last query's
        const uint32_t bf = t & 1;
        const int nq = GENERAL ? a.q_len - q0 : kQStep;
        issue_ints_to_lds_at<kQStep>(ll2 + bf * kWB, reinterpret_cast<const int32_t *>(a.l2 + q0), nq);
        issue_ints_to_lds_at<kQStep>(ldl + bf * kWB, reinterpret_cast<const int32_t *>(a.delta + q0), nq);
        if (CMODE == kGather || (CMODE == kTable && a.doc))
            issue_ints_to_lds_at<kQStep>(ldoc + bf * kWB, a.doc + q0, nq);
        issue_tile_to_lds_at<D, kSwzKV, kQStep>(lq + bf * kTB, a.qb + (int64_t)q0 * a.q_st, a.q_st, nq);
        issue_tile_to_lds_at<D, kSwzKV, kQStep>(lg + bf * kTB, a.gb + (int64_t)q0 * a.do_st, a.do_st, nq);
    };
    const int nsteps = 2 * ntiles;
    if (nsteps <= 0) return;
    int q0 = step_q0(0);
    issue(0, q0);
    auto step = [&](int t, auto masked) {
        wait_vmcnt<0>();
        tile_barrier();  // step t is visible; every wave is done with step t-1's buffers
        int q_next = 0;
        if (t + 1 < nsteps) {
            q_next = step_q0(t + 1);
            issue(t + 1, q_next);
        }
        const uint32_t bf = t & 1;
        const Kv16Offsets oq = step_offsets16(off, lq + bf * kTB), og = step_offsets16(off, lg + bf * kTB);
        dkdv16_step<D, ALIBI, SOFTCAP, CMODE, decltype(masked)::value>(
            a, cm, kf, vf, oq, og, ll2 + bf * kWB, ldl + bf * kWB, ldoc + bf * kWB, q0, dk, dv);
        wait_lds_reads();  // this wave's reads of step t are done before the next barrier
        q0 = q_next;
    };
#pragma unroll 1
    for (int t = 0; t < 2 * a.nfull; ++t) step(t, std::false_type());
#pragma unroll 1
    for (int t = 2 * a.nfull; t < nsteps; ++t) step(t, std::true_type());
}

// dK (times mul) or dV rows of the wave's 16 keys from the 16x16 blocks
// (lane: key l%16, d = 16 db + 4 (l/16) + 0..3 in block db), staged through
// the wave's slice of LDS at `stage` (16-byte chunks XOR-swizzled by the
// row) and stored as whole rows; rows below nrows are stored.
template <int D>
__device__ inline void store16_staged(elem_t *dst, int64_t ld, const f32x4 (&acc)[D / 16], float mul,
                                      uint32_t stage, int nrows) {
    constexpr int kRowBytes = 2 * D, kChunks = kRowBytes / 16, kPerLane = 16 * kChunks / 64;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        u32x2 w;  // columns 16 db + 4 g + 0..3: chunk 2 db + g/2, half g%2
        w.x = pack_elem2(acc[db][0] * mul, acc[db][1] * mul);
        w.y = pack_elem2(acc[db][2] * mul, acc[db][3] * mul);
        lds_store<u32x2>(stage + r * kRowBytes + (((2 * db + (g >> 1)) ^ r) * 16) + (g & 1) * 8, w);
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int row = lane >> 2, c = kPerLane * (lane & 3) + i;  // 16 rows, kPerLane chunks per lane
        const u32x4 v = lds_load<u32x4>(stage + row * kRowBytes + ((c ^ row) * 16));
        if (row < nrows) *reinterpret_cast<u32x4 *>(dst + (int64_t)row * ld + c * 8) = v;
    }
}

template <int D, bool ALIBI, bool SOFTCAP, bool TABLE, bool GENERAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv256_kernel(AttnParams p) {
    static_assert(D == 256, "the 16-key layout serves D = 256");
    __shared__ __attribute__((aligned(1024))) Dkdv16Smem<D> sm;
    const int nt = p.nt;
    const int wg = p.col_chunked ? col_remap(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= 2 * p.B * p.H * nt) return;  // past the work (chunked placement; whole workgroup)
    const int bh = wg / (2 * nt);
    const int jh = wg % (2 * nt);  // early key tiles first
    const int j = jh >> 1, half = jh & 1;
    const int b = bh / p.H, h = bh % p.H;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int kidx = j * kTile + half * kQStep + wv * 16 + n;  // key (past KV_LEN on a cut-short tile)
    const int kpos = min(kidx, p.T - 1);                         // the key this lane loads

    const elem_t *kb = static_cast<const elem_t *>(p.k) + b * p.k_sb + h * p.k_sh;
    const elem_t *vb = static_cast<const elem_t *>(p.v) + b * p.v_sb + h * p.v_sh;
    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t col = (int64_t)bm * nt + j;

    DkdvArgs a;
    a.qb = static_cast<const elem_t *>(p.q) + b * p.q_sb + h * p.q_sh;
    a.gb = static_cast<const elem_t *>(p.dout) + b * p.do_sb + h * p.do_sh;
    a.q_st = p.q_st;
    a.do_st = p.do_st;
    a.l2 = p.lse2 + ((int64_t)b * p.H + h) * p.q_len;
    a.delta = p.delta + ((int64_t)b * p.H + h) * p.q_len;
    a.nfull = min(max(load_uniform(p.full_q_num + col), 0), p.nqt);
    const int npart = min(max(load_uniform(p.q_num + col), 0), p.nqt);
    a.fidx = p.full_q_idx + col * p.nqt;
    a.pidx = p.q_idx + col * p.nqt;
    a.doc = (p.mask_flags & BSM_MASK_DOCUMENT) ? p.doc_ids + (int64_t)bm * p.npos + p.q_off : nullptr;
    a.nt = p.nqt;
    a.kpos = kpos;
    a.q_len = p.q_len;
    a.q_off = p.q_off;
    a.scale = p.scale;
    a.scale_log2 = p.scale * kLog2e;
    a.slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    a.cap = SOFTCAP ? p.softcap : 1.0f;
    a.inv_cap = 1.0f / a.cap;
    a.mk = mod_k<SOFTCAP>(a.scale, a.slope, a.cap);
    const int ntiles = a.nfull + npart;

    ColMask cm;
    bool gather = false;
    if (TABLE)
        make_col_table(p, bm, kpos, (p.mask_flags & BSM_MASK_WINDOW) ? load_uniform(p.window) : 0, cm);
    else
        gather = make_col_mask(p, bm, kpos, cm);
    Kv16Offsets off;
    kv16_offsets<D>(off);

    // K and V rows of the lane's key as B operands: d = 32 st + 8 g .. +7
    elem8 kf[D / 32], vf[D / 32];
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
        kf[st] = *reinterpret_cast<const elem8 *>(kb + (int64_t)kpos * p.k_st + st * 32 + g * 8);
        vf[st] = *reinterpret_cast<const elem8 *>(vb + (int64_t)kpos * p.v_st + st * 32 + g * 8);
    }
    f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        dk[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        dv[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // No wait here: the first copies are issued while the key rows load.
    if (TABLE)
        dkdv16_main<D, ALIBI, SOFTCAP, kTable, GENERAL>(a, cm, kf, vf, off, sm, ntiles, dk, dv);
    else if (gather)
        dkdv16_main<D, ALIBI, SOFTCAP, kGather, GENERAL>(a, cm, kf, vf, off, sm, ntiles, dk, dv);
    else
        dkdv16_main<D, ALIBI, SOFTCAP, kPlain, GENERAL>(a, cm, kf, vf, off, sm, ntiles, dk, dv);

    // dK and dV rows of the wave (8 KB each per wave), staged through the
    // query and output-gradient buffers once every wave is done with them.
    static_assert(sizeof(sm.q) >= (kThreads / 64) * 16 * 2 * D, "dK staging fits the query buffers");
    static_assert(sizeof(sm.g) >= (kThreads / 64) * 16 * 2 * D, "dV staging fits the gradient buffers");
    tile_barrier();
    const uint32_t slice = (uint32_t)(wv * 16 * 2 * D);
    const int k0w = kidx - n;  // the wave's first key
    elem_t *dkp = static_cast<elem_t *>(p.dk) + b * p.dk_sb + h * p.dk_sh + (int64_t)k0w * p.dk_st;
    elem_t *dvp = static_cast<elem_t *>(p.dv) + b * p.dv_sb + h * p.dv_sh + (int64_t)k0w * p.dv_st;
    store16_staged<D>(dkp, p.dk_st, dk, p.scale, lds_addr(&sm.q[0][0]) + slice, p.T - k0w);
    store16_staged<D>(dvp, p.dv_st, dv, 1.0f, lds_addr(&sm.g[0][0]) + slice, p.T - k0w);
}

// dL/dbias: the per-(batch, head, query tile) partial rows of the BIAS
// dq_kernel summed over the batch and the query tiles in a fixed order: a
// workgroup takes 32 entries of one head, its 8 row groups sum the rows
// g, g + 8, ... in turn, and the groups are added in order.
__global__ __launch_bounds__(kThreads) void bias_reduce_kernel(const float *part, float *dbias, int B, int H,
                                                                 int nqt, int nb) {
    constexpr int kGroups = kThreads / 32;
    __shared__ float red[kGroups][32];
    const int h = blockIdx.y, e = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int j = blockIdx.x * 32 + e;
    float acc = 0.0f;
    if (j < nb)
        for (int r = g; r < B * nqt; r += kGroups) {
            const int b = r / nqt, i = r - b * nqt;
            acc += part[(((int64_t)b * H + h) * nqt + i) * nb + j];
        }
    red[g][e] = acc;
    __syncthreads();
    if (g == 0 && j < nb) {
        float v = 0.0f;
        for (int k = 0; k < kGroups; ++k) v += red[k][e];
        dbias[(int64_t)h * nb + j] = v;
    }
}

// dL/dslope[h]: the per-(batch, head, query tile) partials of dq_kernel
// summed over the batch and the query tiles in a fixed order (strided
// per-thread sums, then a fixed tree), so the result is deterministic.
__global__ __launch_bounds__(kThreads) void slope_reduce_kernel(const float *part, float *dslopes, int B, int H,
                                                                  int nt) {
    __shared__ float red[kThreads];
    const int h = blockIdx.x, n = B * nt;
    float acc = 0.0f;
    for (int j = threadIdx.x; j < n; j += kThreads) {
        const int b = j / nt, i = j - b * nt;
        acc += part[((int64_t)b * H + h) * nt + i];
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) dslopes[h] = red[0];
}

// dq_kernel runs the rows in the forward's item order (longest rows first,
// neighbouring rows of a head together on an XCD); dkdv_kernel runs one
// workgroup per (batch, head, key tile), early key tiles first.  Measured on
// the 64K doc+window, causal-in-chunks and ALiBi + soft-cap workloads, the
// column work order gained for dK/dV only with soft-capped documents and lost
// elsewhere, while the row order for dQ gained or held everywhere.
//
// dK/dV placement.  The workgroups of the key tiles go to the XCDs in
// contiguous ranges, so neighbouring tiles share their query tiles in one
// L2.  Under a plain causal mask (no document, window or composed table) a
// head's early tiles carry the most work, and when the ranges do not hold
// whole heads the XCDs get unequal shares (1.66x between the heaviest and
// the lightest at B1 H6 T65536); there the tiles go out in chunks dealt to
// the XCDs in alternating rounds instead (col_remap).  Measured at B1 H6
// T65536: causal 25.1 -> 21.4 ms; the chunked placement was 3.8% slower on
// the doc+window workload and 6% slower with ALiBi + soft-capped documents,
// which keep the ranges.
inline unsigned dkdv_grid_of(AttnParams &q, int per_head) {
    const int64_t n = (int64_t)q.B * q.H * per_head;
    const uint32_t f = q.mask_flags;
    const bool plain_causal = (f & BSM_MASK_CAUSAL) && !(f & (BSM_MASK_DOCUMENT | BSM_MASK_WINDOW | BSM_MASK_TABLE));
    q.col_chunked = plain_causal && n % (8 * (int64_t)per_head) != 0;
    return q.col_chunked ? col_grid(n) : (unsigned)n;
}

template <int D, bool ALIBI, bool SOFTCAP, bool TABLE>
void launch_main(const AttnParams &p, hipStream_t stream) {
    AttnParams q = p;
    const dim3 dq_grid(item_order(q)), block(kThreads);
    // Composed masks always take the clamped copies; otherwise only a key
    // (query) length off the block grid makes dQ's (dK/dV's) copies clamped.
    // (The non-clamped branches name GENERAL = TABLE: with TABLE they are never
    // taken, and the name then matches the clamped kernel instead of adding
    // an unused one.)
    const bool kv_r = TABLE || kv_ragged(p), q_r = TABLE || p.q_len % kTile != 0;
    // dq_kernel writes Delta and L of every query row (every row is one of
    // its items), which dkdv_kernel reads.
    if (ALIBI && p.dslopes) {
        if (kv_r)
            hipLaunchKernelGGL((dq_kernel<D, ALIBI, SOFTCAP, ALIBI, TABLE, true, false>), dq_grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((dq_kernel<D, ALIBI, SOFTCAP, ALIBI, TABLE, TABLE, false>), dq_grid, block, 0, stream, q);
        hipLaunchKernelGGL(slope_reduce_kernel, dim3(p.H), block, 0, stream, p.dslope_part, p.dslopes, p.B, p.H,
                           p.nqt);
    } else {
        if (kv_r)
            hipLaunchKernelGGL((dq_kernel<D, ALIBI, SOFTCAP, false, TABLE, true, false>), dq_grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((dq_kernel<D, ALIBI, SOFTCAP, false, TABLE, TABLE, false>), dq_grid, block, 0, stream, q);
    }
    if constexpr (D == 256) {  // 16 keys per wave, half a key tile per workgroup
        const dim3 grid256(dkdv_grid_of(q, 2 * p.nt));
        if (q_r)
            hipLaunchKernelGGL((dkdv256_kernel<D, ALIBI, SOFTCAP, TABLE, true>), grid256, block, 0, stream, q);
        else
            hipLaunchKernelGGL((dkdv256_kernel<D, ALIBI, SOFTCAP, TABLE, TABLE>), grid256, block, 0, stream, q);
    } else {
        const dim3 dkdv_grid(dkdv_grid_of(q, p.nt));
        if (q_r)
            hipLaunchKernelGGL((dkdv_kernel<D, ALIBI, SOFTCAP, TABLE, true>), dkdv_grid, block, 0, stream, q);
        else
            hipLaunchKernelGGL((dkdv_kernel<D, ALIBI, SOFTCAP, TABLE, TABLE>), dkdv_grid, block, 0, stream, q);
    }
}

// With a bias table: the bias kernels (general path), then the reduction of
// the bias-gradient partials when the caller asked for the gradient.
template <int D, bool SOFTCAP, bool TABLE>
void launch_bias(const AttnParams &p, hipStream_t stream) {
    AttnParams q = p;
    const dim3 dq_grid(item_order(q)), block(kThreads);
    hipLaunchKernelGGL((dq_kernel<D, false, SOFTCAP, false, TABLE, true, true>), dq_grid, block, 0, stream, q);
    if (p.dbias) {
        const int nb = 2 * p.bias_r + 1;
        hipLaunchKernelGGL(bias_reduce_kernel, dim3((nb + 31) / 32, p.H), block, 0, stream,
                           p.dbias_part, p.dbias, p.B, p.H, p.nqt, nb);
    }
    const dim3 dkdv_grid(dkdv_grid_of(q, p.nt));
    hipLaunchKernelGGL((dkdv_bias_kernel<D, SOFTCAP, TABLE>), dkdv_grid, block, 0, stream, q);
}

template <int D, bool TABLE>
void launch_mods(const AttnParams &p, hipStream_t stream) {
    const bool alibi = p.mod_flags & BSM_MOD_ALIBI;
    const bool cap = p.mod_flags & BSM_MOD_SOFTCAP;
    if (p.mod_flags & BSM_MOD_BIAS) {
        if constexpr (D != 256) {  // the host rejects a bias table at D = 256
            if (cap)
                launch_bias<D, true, TABLE>(p, stream);
            else
                launch_bias<D, false, TABLE>(p, stream);
        }
        return;
    }
    if (alibi && cap)
        launch_main<D, true, true, TABLE>(p, stream);
    else if (alibi)
        launch_main<D, true, false, TABLE>(p, stream);
    else if (cap)
        launch_main<D, false, true, TABLE>(p, stream);
    else
        launch_main<D, false, false, TABLE>(p, stream);
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    if (p.mask_flags & BSM_MASK_TABLE)
        launch_mods<D, true>(p, stream);
    else
        launch_mods<D, false>(p, stream);
    return hipGetLastError();
}

}  // namespace

// The build compiles this source once per head dimension (BSM_HEAD_DIM),
// so that the two halves compile in parallel; without it both are built.
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 64
hipError_t BSM_ELEM_FN(launch_attn_bwd_d64)(const AttnParams &p, hipStream_t stream) { return launch_d<64>(p, stream); }
#endif
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 128
hipError_t BSM_ELEM_FN(launch_attn_bwd_d128)(const AttnParams &p, hipStream_t stream) { return launch_d<128>(p, stream); }
#endif
#if !defined(BSM_HEAD_DIM) || BSM_HEAD_DIM == 256
hipError_t BSM_ELEM_FN(launch_attn_bwd_d256)(const AttnParams &p, hipStream_t stream) { return launch_d<256>(p, stream); }
#endif

}  // namespace bsm
