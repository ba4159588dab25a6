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
//  * Q stays in registers; K is staged row-major in LDS, V transposed (keys
//    contiguous, bits 2/3 of the key swapped so each MFMA operand is one
//    16-byte read); rows padded by 16 bytes against bank conflicts;
//  * the next listed tile is loaded from HBM into registers while the current
//    one computes (one LDS buffer, register double-buffering);
//  * exp via exp2 with log2(e) folded into the score scale.
#include "attn_common.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;

template <int D>
struct FwdSmem {
    static constexpr int KS = D + 8;       // K row stride (elements)
    static constexpr int VS = kTile + 8;   // V^T row stride (elements)
    __bf16 k[kTile * KS];
    __bf16 vt[D * VS];
    int32_t doc[kTile];
};

template <int D>
struct TilePrefetch {
    static constexpr int KCH = kTile * D / 8 / kThreads;  // 16-byte K chunks per thread
    static constexpr int VU = 32 * (D / 8) / kThreads;     // (4-key group, d-chunk) units per thread
    uint4 k[KCH];
    uint4 v[VU][4];
    int32_t doc;
};

template <int D>
__device__ inline void prefetch_tile(TilePrefetch<D> &pf, const __bf16 *kbase, const __bf16 *vbase,
                                     int64_t k_st, int64_t v_st, const int32_t *doc, int j) {
    const int tid = threadIdx.x;
    const int key0 = j * kTile;
#pragma unroll
    for (int it = 0; it < TilePrefetch<D>::KCH; ++it) {
        const int c = it * kThreads + tid;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        pf.k[it] = *reinterpret_cast<const uint4 *>(kbase + (int64_t)(key0 + row) * k_st + col);
    }
#pragma unroll
    for (int it = 0; it < TilePrefetch<D>::VU; ++it) {
        const int u = it * kThreads + tid;
        const int g = u / (D / 8), cc = (u % (D / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pf.v[it][e] = *reinterpret_cast<const uint4 *>(vbase + (int64_t)(key0 + 4 * g + e) * v_st + cc);
    }
    if (doc != nullptr && tid < kTile) pf.doc = doc[key0 + tid];
}

__device__ inline uint32_t u16_at(const uint4 &x, int i) {
    const uint32_t w = (i >> 1) == 0 ? x.x : (i >> 1) == 1 ? x.y : (i >> 1) == 2 ? x.z : x.w;
    return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D>
__device__ inline void store_tile(FwdSmem<D> &sm, const TilePrefetch<D> &pf, bool has_doc) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < TilePrefetch<D>::KCH; ++it) {
        const int c = it * kThreads + tid;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4 *>(&sm.k[row * FwdSmem<D>::KS + col]) = pf.k[it];
    }
#pragma unroll
    for (int it = 0; it < TilePrefetch<D>::VU; ++it) {
        const int u = it * kThreads + tid;
        const int g = u / (D / 8), cc = (u % (D / 8)) * 8;
        const int slot = vt_slot(4 * g);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            uint2 w;
            w.x = u16_at(pf.v[it][0], dd) | (u16_at(pf.v[it][1], dd) << 16);
            w.y = u16_at(pf.v[it][2], dd) | (u16_at(pf.v[it][3], dd) << 16);
            *reinterpret_cast<uint2 *>(&sm.vt[(cc + dd) * FwdSmem<D>::VS + slot]) = w;
        }
    }
    if (has_doc && tid < kTile) sm.doc[tid] = pf.doc;
}

struct RowMask {
    int32_t klo, khi;   // visible window/causal interval of keys
    int32_t sink_end;   // keys < sink_end are visible through the sink term
    int32_t docq;
    bool doc_on;
};

template <int D, bool ALIBI, bool SOFTCAP, bool MASKED>
__device__ inline void fwd_tile(const FwdSmem<D> &sm, const bf16x8 (&qf)[D / 16],
                                f32x16 (&o)[D / 32], float &m, float &l, int j, int qpos,
                                float scale_log2, float scale, float slope, float cap,
                                float inv_cap, const RowMask &rm) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                &sm.k[(kb * 32 + n) * FwdSmem<D>::KS + st * 16 + hl * 8]);
            s[kb] = mfma32(a, qf[st], s[kb]);
        }
    }
    float mx = -INFINITY;
    const int kbase = j * kTile;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int4 dk = {0, 0, 0, 0};
            if (MASKED && rm.doc_on)
                dk = *reinterpret_cast<const int4 *>(&sm.doc[kb * 32 + g * 8 + hl * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int kpos = kbase + kb * 32 + g * 8 + hl * 4 + e;
                float t;
                if (!ALIBI && !SOFTCAP) {
                    t = s[kb][r] * scale_log2;
                } else {
                    float y = s[kb][r] * scale;
                    if (ALIBI) y -= slope * (float)(qpos - kpos);
                    if (SOFTCAP) y = cap * tanh_exp2(y * inv_cap);
                    t = y * kLog2e;
                }
                if (MASKED) {
                    bool vis = (kpos >= rm.klo || kpos < rm.sink_end) && kpos <= rm.khi;
                    if (rm.doc_on) {
                        const int dkv = e == 0 ? dk.x : e == 1 ? dk.y : e == 2 ? dk.z : dk.w;
                        vis = vis && (dkv == rm.docq);
                    }
                    t = vis ? t : -INFINITY;
                }
                s[kb][r] = t;
                mx = fmaxf(mx, t);
            }
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - m_use);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    m = m_new;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = fast_exp2(s[kb][s2 * 8 + e] - m_use);
                l += pv[e];
            }
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(pv[e]);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    &sm.vt[(db * 32 + n) * FwdSmem<D>::VS + kb * 32 + s2 * 16 + hl * 8]);
                o[db] = mfma32(a, pb, o[db]);
            }
        }
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;

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

    bf16x8 qf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
        qf[st] = *reinterpret_cast<const bf16x8 *>(qb + (int64_t)qpos * p.q_st + st * 16 + hl * 8);

    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t row = (int64_t)bm * nt + i;
    // Counts and indices are clamped to the grid so that a corrupt block mask
    // gives wrong numbers instead of out-of-bounds reads.
    const int nfull = min(max(p.full_kv_num[row], 0), nt);
    const int npart = min(max(p.kv_num[row], 0), nt);
    const int32_t *fidx = p.full_kv_idx + row * nt;
    const int32_t *pidx = p.kv_idx + row * nt;
    const int total = nfull + npart;

    const bool doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    const int32_t *doc = doc_on ? p.doc_ids + (int64_t)bm * p.T : nullptr;
    RowMask rm;
    rm.doc_on = doc_on;
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

    const float scale = p.scale;
    const float scale_log2 = p.scale * kLog2e;
    const float slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    const float cap = SOFTCAP ? p.softcap : 1.0f;
    const float inv_cap = 1.0f / cap;

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -INFINITY, l = 0.0f;

    TilePrefetch<D> pf;
    if (total > 0)
        prefetch_tile<D>(pf, kb_, vb, p.k_st, p.v_st, doc, clamp_tile(nfull > 0 ? fidx[0] : pidx[0], nt));
    for (int it = 0; it < total; ++it) {
        const int j = clamp_tile(it < nfull ? fidx[it] : pidx[it - nfull], nt);
        __syncthreads();
        store_tile<D>(sm, pf, doc_on);
        __syncthreads();
        if (it + 1 < total) {
            const int jn = clamp_tile((it + 1) < nfull ? fidx[it + 1] : pidx[it + 1 - nfull], nt);
            prefetch_tile<D>(pf, kb_, vb, p.k_st, p.v_st, doc, jn);
        }
        if (it < nfull)
            fwd_tile<D, ALIBI, SOFTCAP, false>(sm, qf, o, m, l, j, qpos, scale_log2, scale, slope,
                                               cap, inv_cap, rm);
        else
            fwd_tile<D, ALIBI, SOFTCAP, true>(sm, qf, o, m, l, j, qpos, scale_log2, scale, slope,
                                              cap, inv_cap, rm);
    }

    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __bf16 *ob = static_cast<__bf16 *>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qpos * p.o_st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(o[db][g * 4 + 0] * inv, o[db][g * 4 + 1] * inv);
            w.y = pack_bf16x2(o[db][g * 4 + 2] * inv, o[db][g * 4 + 3] * inv);
            *reinterpret_cast<uint2 *>(ob + db * 32 + g * 8 + hl * 4) = w;
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
