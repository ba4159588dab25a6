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
__device__ inline void fwd_qk(const __bf16 *sk, const OperandOffsets<D> &off, const bf16x8 (&qf)[D / 16],
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
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbytes + kb * 32 * TileLayout<D>::kRowBytes +
                                                                k_operand_offset(off, st));
            s[kb] = mfma32(a, qf[st], s[kb]);
        }
    }
}

// Running-maximum update for one half tile (and the rescale of o and l when
// the maximum moved by more than the threshold).  Returns the reference the
// exponentials use.
template <int D, bool KMODS>
__device__ inline float fwd_max_update(const f32x16 (&s)[2], f32x16 (&o)[D / 32], float &m, float &l,
                                       float scale_log2) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (!KMODS) mx *= scale_log2;
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
}

// p = 2^(s c - m) as bf16 (the B operand of the PV products), summed into l
// in fp32 before rounding (so lse keeps fp32 accuracy).
__device__ inline void fwd_exp(const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float &l, float c_mul, float m_use) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = fast_exp2(__builtin_fmaf(s[kb][s2 * 8 + e], c_mul, -m_use));
                l += pv;
                pb[kb][s2][e] = static_cast<__bf16>(pv);
            }
}

template <int D>
__device__ inline void fwd_pv(const __bf16 *sv, const OperandOffsets<D> &off, const bf16x8 (&pb)[2][2],
                              f32x16 (&o)[D / 32]) {
    const char *vbytes = reinterpret_cast<const char *>(sv);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int rowbase = (kb * 32 + s2 * 16) * TileLayout<D>::kRowBytes;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const i16x4 lo = ds_read_tr16(reinterpret_cast<const __bf16 *>(vbytes + rowbase + v_operand_offset(off, 0, db)));
                const i16x4 hi = ds_read_tr16(reinterpret_cast<const __bf16 *>(vbytes + rowbase + v_operand_offset(off, 1, db)));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = mfma32(a, pb[kb][s2], o[db]);
            }
        }
    }
}

struct FwdArgs {
    const __bf16 *kb, *vb;
    int64_t k_st, v_st;
    const int32_t *doc, *fidx, *pidx;
    int nfull, nt, qpos;
    float scale, scale_log2, slope, cap, inv_cap;
};

// The double-buffered, software-pipelined loop over the listed tiles (in
// 64-key steps).  Step t's scores are computed during step t-1.  At the top
// of step t the copies issued at the top of step t-1 -- K(t+1) and V(t) --
// have landed; the barrier also certifies that every wave has finished step
// t-1, freeing K buffer t%2 (last read for K(t)) and V buffer (t+1)%2 (last
// read for V(t-1)) for K(t+2) and V(t+1).
template <int D, bool ALIBI, bool SOFTCAP, int MODE>
__device__ inline void fwd_main(const FwdArgs &a, const RowMask &rm, const bf16x8 (&qf)[D / 16],
                                const OperandOffsets<D> &off, __bf16 (&skb)[2][kHalf * D],
                                __bf16 (&svb)[2][kHalf * D], int32_t (&sdb)[2][kHalf], int nsteps,
                                f32x16 (&o)[D / 32], float &m, float &l) {
    constexpr bool kMods = ALIBI || SOFTCAP;
    const float c_mul = kMods ? 1.0f : a.scale_log2;
    auto step_key0 = [&](int t) {
        const int it = t >> 1;
        const int jj = clamp_tile(it < a.nfull ? load_uniform(a.fidx + it) : load_uniform(a.pidx + it - a.nfull),
                                  a.nt);
        return jj * kTile + (t & 1) * kHalf;
    };
    auto issue_k = [&](int t, int key0) {
        if (MODE == kGather) issue_ints_to_lds<kHalf>(sdb[t & 1], a.doc + key0);
        issue_tile_to_lds<D, kSwzK, kHalf>(skb[t & 1], a.kb + (int64_t)key0 * a.k_st, a.k_st);
    };
    auto issue_v = [&](int t, int key0) {
        issue_tile_to_lds<D, kSwzV, kHalf>(svb[t & 1], a.vb + (int64_t)key0 * a.v_st, a.v_st);
    };
    if (nsteps <= 0) return;

    f32x16 sa[2], sb[2];
    {
        const int k0 = step_key0(0);
        issue_k(0, k0);
        issue_v(0, k0);
        if (nsteps > 1) issue_k(1, step_key0(1));
        wait_vmcnt<0>();
        tile_barrier();
        fwd_qk<D>(skb[0], off, qf, sa);
        row_mod_mask<ALIBI, SOFTCAP, MODE>(lds_addr(sdb[0]), sa, k0, a.qpos, a.scale, a.slope, a.cap, a.inv_cap, rm,
                                           0 >= a.nfull);
    }
    // One pipelined step: exponentials and PV of step t (scores in sc), QK^T
    // and mask of step t+1 (into sn).  Unrolled by two below so that sc and
    // sn swap roles without register copies.
    auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], int t) {
        wait_vmcnt<0>();
        tile_barrier();
        OperandOffsets<D> offt = off;  // opaque per step: derived offsets are not hoisted
        asm volatile("" : "+v"(offt.k), "+v"(offt.v));
        const int key_next = step_key0(t + 1);
        if (t + 2 < nsteps) issue_k(t + 2, step_key0(t + 2));
        issue_v(t + 1, key_next);

        const float m_use = fwd_max_update<D, kMods>(sc, o, m, l, a.scale_log2);
        bf16x8 pb[2][2];
        // next step's QK^T products, interleaved with this step's exponentials
        fwd_qk<D>(skb[(t + 1) & 1], offt, qf, sn);
        fwd_exp(sc, pb, l, c_mul, m_use);
        // this step's PV products, interleaved with the next step's mask
        fwd_pv<D>(svb[t & 1], offt, pb, o);
        row_mod_mask<ALIBI, SOFTCAP, MODE>(lds_addr(sdb[(t + 1) & 1]), sn, key_next, a.qpos, a.scale, a.slope, a.cap,
                                           a.inv_cap, rm, ((t + 1) >> 1) >= a.nfull);
        wait_lds_reads();  // this wave's reads of step t are done before the next barrier
    };
    auto last = [&](f32x16 (&sc)[2], int t) {
        wait_vmcnt<0>();
        tile_barrier();
        const float m_use = fwd_max_update<D, kMods>(sc, o, m, l, a.scale_log2);
        bf16x8 pb[2][2];
        fwd_exp(sc, pb, l, c_mul, m_use);
        fwd_pv<D>(svb[t & 1], off, pb, o);
    };
    int t = 0;
    for (; t + 2 < nsteps; t += 2) {
        step(sa, sb, t);
        step(sb, sa, t + 1);
    }
    if (nsteps - t == 2) {
        step(sa, sb, t);
        last(sb, t + 1);
    } else {
        last(sa, t);
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(AttnParams p) {
    // Double-buffered half tiles.  Separate LDS objects per role so that no
    // compiler-inserted wait ties reads of one to copies into another.
    __shared__ __attribute__((aligned(1024))) __bf16 skb[2][kHalf * D];  // keys, rows swizzled by fk
    __shared__ __attribute__((aligned(1024))) __bf16 svb[2][kHalf * D];  // values, rows swizzled by fv
    __shared__ __attribute__((aligned(16))) int32_t sdb[2][kHalf];       // document ids of the keys

    const int nt = p.nt;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = wg / nt;
    const int i = nt - 1 - (wg % nt);  // later query tiles first: under a causal
                                       // mask they carry the most tiles
    const int b = bh / p.H, h = bh % p.H;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int qpos = i * kTile + wv * 32 + n;

    const __bf16 *qb = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t row = (int64_t)bm * nt + i;

    FwdArgs a;
    a.kb = static_cast<const __bf16 *>(p.k) + b * p.k_sb + h * p.k_sh;
    a.vb = static_cast<const __bf16 *>(p.v) + b * p.v_sb + h * p.v_sh;
    a.k_st = p.k_st;
    a.v_st = p.v_st;
    // Counts and indices are clamped to the grid so that a corrupt block mask
    // gives wrong numbers instead of out-of-bounds reads.
    a.nfull = min(max(load_uniform(p.full_kv_num + row), 0), nt);
    const int npart = min(max(load_uniform(p.kv_num + row), 0), nt);
    a.fidx = p.full_kv_idx + row * nt;
    a.pidx = p.kv_idx + row * nt;
    a.nt = nt;
    a.qpos = qpos;
    a.scale = p.scale;
    a.scale_log2 = p.scale * kLog2e;
    a.slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    a.cap = SOFTCAP ? p.softcap : 1.0f;
    a.inv_cap = 1.0f / a.cap;
    const int nsteps = 2 * (a.nfull + npart);  // 64-key steps

    const bool doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    a.doc = doc_on ? p.doc_ids + (int64_t)bm * p.T : nullptr;
    RowMask rm;
    const int mode = make_row_mask(p, bm, qpos, rm);

    OperandOffsets<D> off;
    operand_offsets<D>(off);

    bf16x8 qf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
        qf[st] = *reinterpret_cast<const bf16x8 *>(qb + (int64_t)qpos * p.q_st + st * 16 + hl * 8);

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    wait_vmcnt<0>();  // Q, the document range and id are in registers before any tile copy

    if (mode == kGather)
        fwd_main<D, ALIBI, SOFTCAP, kGather>(a, rm, qf, off, skb, svb, sdb, nsteps, o, m, l);
    else if (mode == kSinks)
        fwd_main<D, ALIBI, SOFTCAP, kSinks>(a, rm, qf, off, skb, svb, sdb, nsteps, o, m, l);
    else
        fwd_main<D, ALIBI, SOFTCAP, kPlain>(a, rm, qf, off, skb, svb, sdb, nsteps, o, m, l);

    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __bf16 *ob = static_cast<__bf16 *>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qpos * p.o_st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w.x = pack_bf16x2(o[db][g * 4 + 0] * inv, o[db][g * 4 + 1] * inv);
            w.y = pack_bf16x2(o[db][g * 4 + 2] * inv, o[db][g * 4 + 3] * inv);
            *reinterpret_cast<u32x2 *>(ob + db * 32 + g * 8 + hl * 4) = w;
        }
    }
    if (hl == 0) {
        const float lse = l_tot > 0.0f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
        p.lse[((int64_t)b * p.H + h) * p.T + qpos] = lse;
    }
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    const dim3 grid(p.B * p.H * p.nt), block(kThreads);
    const bool alibi = p.mod_flags & BSM_MOD_ALIBI;
    const bool cap = p.mod_flags & BSM_MOD_SOFTCAP;
    if (alibi && cap)
        hipLaunchKernelGGL((fwd_kernel<D, true, true>), grid, block, 0, stream, p);
    else if (alibi)
        hipLaunchKernelGGL((fwd_kernel<D, true, false>), grid, block, 0, stream, p);
    else if (cap)
        hipLaunchKernelGGL((fwd_kernel<D, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_kernel<D, false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams &p, int D, hipStream_t stream) {
    if (D == 64) return launch_d<64>(p, stream);
    return launch_d<128>(p, stream);
}

}  // namespace bsm
