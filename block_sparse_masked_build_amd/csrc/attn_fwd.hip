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
//  * the copies run asynchronously: the next K tile is requested as soon as
//    every wave is done with QK^T, the next V tile as soon as PV is done, so
//    HBM latency hides behind the softmax and the other matrix product;
//  * two workgroups per CU (at most 256 registers per lane), so one
//    workgroup's tile loads and softmax overlap the other's matrix products;
//  * exp via exp2 with log2(e) and the score scale folded into one FMA; the
//    running maximum is only moved (and the output rescaled) when a score
//    exceeds it by more than 2^8.
#include "attn_common.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;

struct RowMask {
    int32_t klo, khi;   // visible window/causal interval of keys
    int32_t sink_end;   // keys < sink_end are visible through the sink term
    int32_t docq;       // document id of the query (0 without the document term)
};

// Per-query state of the online softmax.  m is the reference maximum (log2
// domain) the accumulators are scaled to; it is only moved when a new score
// exceeds it by more than 2^8, so most tiles skip the rescale.  The result
// stays exact because o and l always share the same reference.
constexpr float kRescaleThreshold = 8.0f;

// Per-lane LDS byte offsets of the matrix-core operands inside a tile.
template <int D>
struct OperandOffsets {
    int k[D / 16];        // A operand of S^T = K Q^T, per 16-wide d step (row = lane's key in block 0)
    int v[2][D / 32];     // transposing reads of V, per half (keys +0..3 / +8..11) and d block
};

template <int D>
__device__ inline void operand_offsets(OperandOffsets<D> &off) {
    using L = TileLayout<D>;
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) off.k[st] = n * L::kRowBytes + (((2 * st + hl) ^ L::fk(n)) << 4);
    // ds_read_tr16_b64: lane j of a 16-lane group G supplies the address of
    // row K0 + j/4, columns d0 + 4 (j%4) .. +3; lane i then receives rows
    // K0..K0+3 of column d0 + i.  d0 = 32 db + 16 (G%2); K0 = 4 (G/2) (+8 for
    // the second half) inside each 16-key group.
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = 8 * u + 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int c = db * 4 + 2 * (G & 1) + ((j & 3) >> 1);
            off.v[u][db] = r * L::kRowBytes + ((c ^ L::fv(r)) << 4) + ((j & 1) << 3);
        }
    }
}

// S^T = K Q^T for one tile: lane (query n, half hl) gets, for key block kb,
// the 16 scores of keys 32 kb + 8 (r/4) + 4 hl + r%4, r = 0..15.
template <int D>
__device__ inline void fwd_qk(const __bf16 *sk, const OperandOffsets<D> &off, const bf16x8 (&qf)[D / 16],
                              f32x16 (&s)[4]) {
    const char *kbytes = reinterpret_cast<const char *>(sk);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbytes + kb * 32 * TileLayout<D>::kRowBytes + off.k[st]);
            s[kb] = mfma32(a, qf[st], s[kb]);
        }
    }
    sched_interleave<4 * (D / 16), 4>();
}

// Score modifications (to the log2 domain) and, on partial tiles, the mask.
template <bool ALIBI, bool SOFTCAP, bool MASKED>
__device__ inline void fwd_mod_mask(const int32_t *sdoc, f32x16 (&s)[4], int j, int qpos, float scale, float slope,
                                    float cap, float inv_cap, const RowMask &rm) {
    constexpr bool kMods = ALIBI || SOFTCAP;
    const int hl = (threadIdx.x & 63) >> 5;
    const int kbase = j * kTile + hl * 4;
    // Mask bounds relative to this tile.  Kept opaque so that the compiler
    // compares them with the per-register key offsets inside the loop instead
    // of hoisting 3 x 64 loop-invariant thresholds into registers.
    int lo_t = rm.klo - kbase, hi_t = rm.khi - kbase, se_t = rm.sink_end - kbase;
    if (MASKED) asm volatile("" : "+v"(lo_t), "+v"(hi_t), "+v"(se_t));
    int rel = qpos - kbase;
    if (ALIBI) asm volatile("" : "+v"(rel));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int4 dk = {0, 0, 0, 0};
            if (MASKED) dk = *reinterpret_cast<const int4 *>(&sdoc[kb * 32 + g * 8 + hl * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int c = kb * 32 + g * 8 + e;  // key - kbase
                float t = s[kb][r];
                if (kMods) {
                    float y = t * scale;
                    if (ALIBI) y -= slope * (float)(rel - c);
                    if (SOFTCAP) y = cap * tanh_exp2(y * inv_cap);
                    t = y * kLog2e;
                }
                if (MASKED) {
                    // Without the document term the staged ids and docq are all 0.
                    const int dkv = e == 0 ? dk.x : e == 1 ? dk.y : e == 2 ? dk.z : dk.w;
                    const bool vis = (c >= lo_t || c < se_t) && c <= hi_t && dkv == rm.docq;
                    t = vis ? t : -INFINITY;
                }
                s[kb][r] = t;
            }
        }
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__device__ inline void fwd_softmax(f32x16 (&s)[4], f32x16 (&o)[D / 32], float &m, float &l, float scale_log2) {
    constexpr bool kMods = ALIBI || SOFTCAP;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (!kMods) mx *= scale_log2;
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
    const float m_use = (m == -INFINITY) ? 0.0f : m;
    const float c_mul = kMods ? 1.0f : scale_log2;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(__builtin_fmaf(s[kb][r], c_mul, -m_use));
            l += pv;
            s[kb][r] = pv;
        }
}

template <int D>
__device__ inline void fwd_pv(const __bf16 *sv, const OperandOffsets<D> &off, const f32x16 (&s)[4],
                              f32x16 (&o)[D / 32]) {
    const char *vbytes = reinterpret_cast<const char *>(sv);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[kb][s2 * 8 + e]);
            const int rowbase = (kb * 32 + s2 * 16) * TileLayout<D>::kRowBytes;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const i16x4 lo = ds_read_tr16(reinterpret_cast<const __bf16 *>(vbytes + rowbase + off.v[0][db]));
                const i16x4 hi = ds_read_tr16(reinterpret_cast<const __bf16 *>(vbytes + rowbase + off.v[1][db]));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = mfma32(a, pb, o[db]);
            }
        }
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(AttnParams p) {
    // Separate LDS objects so the compiler can tell the copies into one from
    // reads of another (its wait-count insertion tracks them per object).
    __shared__ __attribute__((aligned(1024))) __bf16 sk[kTile * D];   // keys, rows swizzled by fk
    __shared__ __attribute__((aligned(1024))) __bf16 sv[kTile * D];   // values, rows swizzled by fv
    __shared__ __attribute__((aligned(16))) int32_t sdoc[kTile];      // document ids of the keys
    constexpr int kInstr = tile_lds_instr<D>();

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
    const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + b * p.k_sb + h * p.k_sh;
    const __bf16 *vb = static_cast<const __bf16 *>(p.v) + b * p.v_sb + h * p.v_sh;

    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t row = (int64_t)bm * nt + i;
    // Counts and indices are clamped to the grid so that a corrupt block mask
    // gives wrong numbers instead of out-of-bounds reads.
    const int nfull = min(max(load_uniform(p.full_kv_num + row), 0), nt);
    const int npart = min(max(load_uniform(p.kv_num + row), 0), nt);
    const int32_t *fidx = p.full_kv_idx + row * nt;
    const int32_t *pidx = p.kv_idx + row * nt;
    const int total = nfull + npart;

    const bool doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    const int32_t *doc = doc_on ? p.doc_ids + (int64_t)bm * p.T : nullptr;
    RowMask rm;
    rm.docq = doc_on ? doc[qpos] : 0;
    rm.khi = (p.mask_flags & BSM_MASK_CAUSAL) ? qpos : p.T - 1;
    rm.klo = -1;
    rm.sink_end = 0;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        int64_t lo = (int64_t)qpos - (int64_t)(*p.window) + 1;
        lo = lo < -1 ? -1 : (lo > p.T ? p.T : lo);
        rm.klo = (int32_t)lo;
        if ((p.mask_flags & BSM_MASK_SINKS) && p.sinks > 0) rm.sink_end = p.sinks;
    }
    if (!doc_on && tid < kTile) sdoc[tid] = 0;  // compared against docq = 0
    wait_lds_reads();                            // the fill is complete before the first barrier

    const float scale = p.scale;
    const float scale_log2 = p.scale * kLog2e;
    const float slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    const float cap = SOFTCAP ? p.softcap : 1.0f;
    const float inv_cap = 1.0f / cap;

    OperandOffsets<D> off;
    operand_offsets<D>(off);

    auto tile_at = [&](int it) {
        return clamp_tile(it < nfull ? load_uniform(fidx + it) : load_uniform(pidx + it - nfull), nt);
    };
    // Copies in flight per wave, in issue order: [doc(it), K(it)] then V(it).
    auto issue_k = [&](int jj) {
        if (doc_on) issue_ints_to_lds(sdoc, doc + jj * kTile);
        issue_tile_to_lds<D, false>(sk, kb_ + (int64_t)jj * kTile * p.k_st, p.k_st);
    };
    auto issue_v = [&](int jj) { issue_tile_to_lds<D, true>(sv, vb + (int64_t)jj * kTile * p.v_st, p.v_st); };

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
    wait_vmcnt<0>();  // Q and the query's document id are in registers before any tile copy

    int j = total > 0 ? tile_at(0) : 0;
    if (total > 0) {
        issue_k(j);
        issue_v(j);
    }
    for (int it = 0; it < total; ++it) {
        const bool more = it + 1 < total;
        const int jn = more ? tile_at(it + 1) : 0;
        // Copies in flight per wave, oldest first: [doc(it)] K(it), V(it).
        wait_vmcnt<kInstr>();  // doc(it), K(it) landed
        tile_barrier();        // ... in every wave
        f32x16 s[4];
        fwd_qk<D>(sk, off, qf, s);
        if (it < nfull) {
            if (ALIBI || SOFTCAP) fwd_mod_mask<ALIBI, SOFTCAP, false>(sdoc, s, j, qpos, scale, slope, cap, inv_cap, rm);
        } else {
            fwd_mod_mask<ALIBI, SOFTCAP, true>(sdoc, s, j, qpos, scale, slope, cap, inv_cap, rm);
        }
        wait_lds_reads();
        tile_barrier();        // every wave is done reading K(it) and doc(it)
        if (more) issue_k(jn);
        fwd_softmax<D, ALIBI, SOFTCAP>(s, o, m, l, scale_log2);
        // In flight now: V(it), then [doc(it+1)] K(it+1).
        if (more) {
            if (doc_on) wait_vmcnt<kInstr + 1>(); else wait_vmcnt<kInstr>();
        } else {
            wait_vmcnt<0>();
        }
        tile_barrier();        // V(it) landed in every wave
        fwd_pv<D>(sv, off, s, o);
        wait_lds_reads();
        tile_barrier();        // every wave is done reading V(it)
        if (more) issue_v(jn);
        j = jn;
    }

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
