// Block-sparse masked attention, backward pass, for gfx950.
//
// Gradients of sum(out * dO) through the softmax, the mask and the score
// modifications (tutorial "FlexAttention in PyTorch", Pattern 3: ALiBi and
// soft-cap are differentiable and get a fused backward), visiting only the
// tiles the block mask lists (speedrun notes "FlexAttention", tile-summary
// paragraph).  With p = exp(s - lse) recomputed from the forward's lse:
//   Delta_q = <dO_q, out_q>
//   dS_qk   = p_qk (<dO_q, v_k> - Delta_q) * (1 - (s_qk / c)^2 if capped)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
//
// Three kernels, no atomics (results are deterministic):
//  * delta_kernel: Delta per query row (16 lanes per row, 16-byte loads);
//  * dkdv_kernel: one workgroup per (batch, head, 128-key tile), iterating
//    the transposed (per key tile) full and partial query-tile lists; lane l
//    of wave w owns key 32w + l%32, so P and dS come out of the matrix cores
//    with queries in registers -- exactly the k-operand layout the dV and dK
//    products need; Q and dO are staged both row-major and transposed in LDS;
//  * dq_kernel: one workgroup per (batch, head, 128-query tile) over the row
//    lists, lane l owning query 32w + l%32 as in the forward; K is staged
//    row-major and transposed, V row-major.
#include "attn_common.hpp"

namespace bsm {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- Delta

template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(AttnParams p) {
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPB = kThreads / LPR;        // rows per block
    const int64_t rows = (int64_t)p.B * p.H * p.T;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = (threadIdx.x % LPR) * 8;
    float acc = 0.0f;
    if (r < rows) {
        const int64_t t = r % p.T, bh = r / p.T;
        const int64_t b = bh / p.H, h = bh % p.H;
        const u32x4 o = *reinterpret_cast<const u32x4 *>(static_cast<const __bf16 *>(p.o) + b * p.o_sb +
                                                          h * p.o_sh + t * p.o_st + c);
        const u32x4 g = *reinterpret_cast<const u32x4 *>(static_cast<const __bf16 *>(p.dout) + b * p.do_sb +
                                                          h * p.do_sh + t * p.do_st + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ov = __builtin_bit_cast(float, u16_at(o, e) << 16);
            const float gv = __builtin_bit_cast(float, u16_at(g, e) << 16);
            acc += ov * gv;
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (r < rows && threadIdx.x % LPR == 0) p.delta[r] = acc;
}

// ------------------------------------------------------- shared helpers

// Log2-domain score of one (query, key) pair and, through y, the final
// natural-domain score (needed for the soft-cap derivative).  Same arithmetic
// as the forward kernel.
template <bool ALIBI, bool SOFTCAP>
__device__ inline float score_log2(float raw, int qpos, int kpos, float scale_log2, float scale,
                                   float slope, float cap, float inv_cap, float &y) {
    if (!ALIBI && !SOFTCAP) {
        y = 0.0f;
        return raw * scale_log2;
    }
    float v = raw * scale;
    if (ALIBI) v -= slope * (float)(qpos - kpos);
    if (SOFTCAP) v = cap * tanh_exp2(v * inv_cap);
    y = v;
    return v * kLog2e;
}

// 128 rows x D of a bf16 [T, D] matrix, loaded as (4-row group, 8-column
// chunk) units so that each unit can be written row-major and transposed.
template <int D>
struct RowsUnits {
    static constexpr int U = 32 * (D / 8) / kThreads;
    u32x4 v[U][4];
};

template <int D>
__device__ inline void load_rows(RowsUnits<D> &ru, const __bf16 *base, int64_t st, int row0) {
#pragma unroll
    for (int it = 0; it < RowsUnits<D>::U; ++it) {
        const int u = it * kThreads + threadIdx.x;
        const int g = u / (D / 8), cc = (u % (D / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ru.v[it][e] = *reinterpret_cast<const u32x4 *>(base + (int64_t)(row0 + 4 * g + e) * st + cc);
    }
}

template <int D>
__device__ inline void store_rows(const RowsUnits<D> &ru, __bf16 *rowmajor, int ld_rm, __bf16 *transposed,
                                  int ld_t) {
#pragma unroll
    for (int it = 0; it < RowsUnits<D>::U; ++it) {
        const int u = it * kThreads + threadIdx.x;
        const int g = u / (D / 8), cc = (u % (D / 8)) * 8;
        if (rowmajor != nullptr) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<u32x4 *>(&rowmajor[(4 * g + e) * ld_rm + cc]) = ru.v[it][e];
        }
        if (transposed != nullptr) store_transposed_4x8(transposed, ld_t, 4 * g, cc, ru.v[it]);
    }
}

// Writes a D^T-layout accumulator block (lane = row of dst, registers =
// 16 columns col0 + 8*(r/4) + 4*half + r%4) as bf16.
__device__ inline void store_acc_rows(__bf16 *dst, const f32x16 &acc, int col0, int hl, float mul) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = pack_bf16x2(acc[g * 4 + 0] * mul, acc[g * 4 + 1] * mul);
        w.y = pack_bf16x2(acc[g * 4 + 2] * mul, acc[g * 4 + 3] * mul);
        *reinterpret_cast<u32x2 *>(dst + col0 + g * 8 + hl * 4) = w;
    }
}

// ---------------------------------------------------------------- dK, dV

template <int D>
struct DkdvSmem {
    static constexpr int RS = D + 8;       // row-major stride
    static constexpr int TS = kTile + 8;   // transposed stride
    __bf16 q[kTile * RS];
    __bf16 qt[D * TS];
    __bf16 dout[kTile * RS];
    __bf16 doutt[D * TS];
    float lse2[kTile];
    float delta[kTile];
    int32_t doc[kTile];
};

// One listed query tile for the wave's 32 keys, one 32-query block at a time
// (keeps 32 score registers live instead of 128).
template <int D, bool ALIBI, bool SOFTCAP, bool MASKED>
__device__ inline void dkdv_tile(const DkdvSmem<D> &sm, const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                 f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], int i, int kpos, int qlo, int qhi,
                                 int dockey, bool doc_on, float scale_log2, float scale, float slope,
                                 float cap, float inv_cap) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
    const int qbase = i * kTile;
#pragma unroll 1
    for (int qb = 0; qb < 4; ++qb) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.0f;
            dp[r] = 0.0f;
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int off = (qb * 32 + n) * DkdvSmem<D>::RS + st * 16 + hl * 8;
            s = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.q[off]), kf[st], s);
            dp = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.dout[off]), vf[st], dp);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ql = qb * 32 + g * 8 + hl * 4;
            const float4 L = *reinterpret_cast<const float4 *>(&sm.lse2[ql]);
            const float4 Dl = *reinterpret_cast<const float4 *>(&sm.delta[ql]);
            int4 dq4 = {0, 0, 0, 0};
            if (MASKED && doc_on) dq4 = *reinterpret_cast<const int4 *>(&sm.doc[ql]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int qpos = qbase + ql + e;
                float y;
                const float t = score_log2<ALIBI, SOFTCAP>(s[r], qpos, kpos, scale_log2, scale, slope, cap,
                                                           inv_cap, y);
                const float le = e == 0 ? L.x : e == 1 ? L.y : e == 2 ? L.z : L.w;
                const float de = e == 0 ? Dl.x : e == 1 ? Dl.y : e == 2 ? Dl.z : Dl.w;
                float pv = fast_exp2(t - le);
                if (MASKED) {
                    bool vis = qpos >= qlo && qpos <= qhi;
                    if (doc_on) {
                        const int dq = e == 0 ? dq4.x : e == 1 ? dq4.y : e == 2 ? dq4.z : dq4.w;
                        vis = vis && dq == dockey;
                    }
                    pv = vis ? pv : 0.0f;
                }
                float ds = pv * (dp[r] - de) * scale;
                if (SOFTCAP) ds *= 1.0f - (y * inv_cap) * (y * inv_cap);
                s[r] = pv;
                dp[r] = ds;
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 pb, db16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pb[e] = static_cast<__bf16>(s[s2 * 8 + e]);
                db16[e] = static_cast<__bf16>(dp[s2 * 8 + e]);
            }
#pragma unroll
            for (int dbk = 0; dbk < D / 32; ++dbk) {
                const int off = (dbk * 32 + n) * DkdvSmem<D>::TS + qb * 32 + s2 * 16 + hl * 8;
                dv[dbk] = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.doutt[off]), pb, dv[dbk]);
                dk[dbk] = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.qt[off]), db16, dk[dbk]);
            }
        }
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) DkdvSmem<D> sm;
    const int nt = p.nt;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = wg / nt;
    const int j = wg % nt;  // early key tiles first: under a causal mask they carry the most tiles
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int kpos = j * kTile + wv * 32 + n;

    const __bf16 *qb_ = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
    const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + b * p.k_sb + h * p.k_sh;
    const __bf16 *vb_ = static_cast<const __bf16 *>(p.v) + b * p.v_sb + h * p.v_sh;
    const __bf16 *gb_ = static_cast<const __bf16 *>(p.dout) + b * p.do_sb + h * p.do_sh;

    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        kf[st] = *reinterpret_cast<const bf16x8 *>(kb_ + (int64_t)kpos * p.k_st + st * 16 + hl * 8);
        vf[st] = *reinterpret_cast<const bf16x8 *>(vb_ + (int64_t)kpos * p.v_st + st * 16 + hl * 8);
    }

    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t col = (int64_t)bm * nt + j;
    const int nfull = min(max(p.full_q_num[col], 0), nt);
    const int npart = min(max(p.q_num[col], 0), nt);
    const int32_t *fidx = p.full_q_idx + col * nt;
    const int32_t *pidx = p.q_idx + col * nt;
    const int total = nfull + npart;

    // Visible queries of this key: qlo <= q <= qhi (causal / window / sink),
    // and the same document.
    const bool doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    const int32_t *doc = doc_on ? p.doc_ids + (int64_t)bm * p.T : nullptr;
    const int dockey = doc_on ? doc[kpos] : 0;
    const int qlo = (p.mask_flags & BSM_MASK_CAUSAL) ? kpos : 0;
    int qhi = p.T - 1;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        const bool sink = (p.mask_flags & BSM_MASK_SINKS) && kpos < p.sinks;
        if (!sink) {
            int64_t hi = (int64_t)kpos + (int64_t)(*p.window) - 1;
            hi = hi < -1 ? -1 : (hi > p.T - 1 ? p.T - 1 : hi);
            qhi = (int)hi;
        }
    }

    const float scale = p.scale;
    const float scale_log2 = p.scale * kLog2e;
    const float slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    const float cap = SOFTCAP ? p.softcap : 1.0f;
    const float inv_cap = 1.0f / cap;
    const float *lse_bh = p.lse + ((int64_t)b * p.H + h) * p.T;
    const float *delta_bh = p.delta + ((int64_t)b * p.H + h) * p.T;

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[d][r] = 0.0f;
            dv[d][r] = 0.0f;
        }

    for (int it = 0; it < total; ++it) {
        const int i = clamp_tile(it < nfull ? fidx[it] : pidx[it - nfull], nt);
        // Q and dO staged one after the other: one set of staging registers.
        RowsUnits<D> ur;
        load_rows<D>(ur, qb_, p.q_st, i * kTile);
        float l2 = 0.0f, dl = 0.0f;
        int dq = 0;
        if (tid < kTile) {
            const float lse = lse_bh[i * kTile + tid];
            l2 = lse == -INFINITY ? 0.0f : lse * kLog2e;
            dl = delta_bh[i * kTile + tid];
            if (doc_on) dq = doc[i * kTile + tid];
        }
        __syncthreads();
        store_rows<D>(ur, sm.q, DkdvSmem<D>::RS, sm.qt, DkdvSmem<D>::TS);
        load_rows<D>(ur, gb_, p.do_st, i * kTile);
        store_rows<D>(ur, sm.dout, DkdvSmem<D>::RS, sm.doutt, DkdvSmem<D>::TS);
        if (tid < kTile) {
            sm.lse2[tid] = l2;
            sm.delta[tid] = dl;
            sm.doc[tid] = dq;
        }
        __syncthreads();
        if (it < nfull)
            dkdv_tile<D, ALIBI, SOFTCAP, false>(sm, kf, vf, dk, dv, i, kpos, qlo, qhi, dockey, doc_on,
                                                scale_log2, scale, slope, cap, inv_cap);
        else
            dkdv_tile<D, ALIBI, SOFTCAP, true>(sm, kf, vf, dk, dv, i, kpos, qlo, qhi, dockey, doc_on,
                                               scale_log2, scale, slope, cap, inv_cap);
    }

    __bf16 *dkp = static_cast<__bf16 *>(p.dk) + b * p.dk_sb + h * p.dk_sh + (int64_t)kpos * p.dk_st;
    __bf16 *dvp = static_cast<__bf16 *>(p.dv) + b * p.dv_sb + h * p.dv_sh + (int64_t)kpos * p.dv_st;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
        store_acc_rows(dkp, dk[d], d * 32, hl, 1.0f);
        store_acc_rows(dvp, dv[d], d * 32, hl, 1.0f);
    }
}

// ---------------------------------------------------------------- dQ

template <int D>
struct DqSmem {
    static constexpr int RS = D + 8;
    static constexpr int TS = kTile + 8;
    __bf16 k[kTile * RS];
    __bf16 kt[D * TS];
    __bf16 v[kTile * RS];
    int32_t doc[kTile];
};

struct QueryMask {
    int32_t klo, khi, sink_end, docq;
    bool doc_on;
};

// One listed key tile for the wave's 32 queries, one 32-key block at a time.
template <int D, bool ALIBI, bool SOFTCAP, bool MASKED>
__device__ inline void dq_tile(const DqSmem<D> &sm, const bf16x8 (&qf)[D / 16], const bf16x8 (&gf)[D / 16],
                               f32x16 (&dq)[D / 32], int j, int qpos, float L, float Dl, const QueryMask &qm,
                               float scale_log2, float scale, float slope, float cap, float inv_cap) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
    const int kbase = j * kTile;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.0f;
            dp[r] = 0.0f;
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int off = (kb * 32 + n) * DqSmem<D>::RS + st * 16 + hl * 8;
            s = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.k[off]), qf[st], s);
            dp = mfma32(*reinterpret_cast<const bf16x8 *>(&sm.v[off]), gf[st], dp);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int4 dk4 = {0, 0, 0, 0};
            if (MASKED && qm.doc_on) dk4 = *reinterpret_cast<const int4 *>(&sm.doc[kb * 32 + g * 8 + hl * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int kpos = kbase + kb * 32 + g * 8 + hl * 4 + e;
                float y;
                const float t = score_log2<ALIBI, SOFTCAP>(s[r], qpos, kpos, scale_log2, scale, slope, cap,
                                                           inv_cap, y);
                float pv = fast_exp2(t - L);
                if (MASKED) {
                    bool vis = (kpos >= qm.klo || kpos < qm.sink_end) && kpos <= qm.khi;
                    if (qm.doc_on) {
                        const int dkv = e == 0 ? dk4.x : e == 1 ? dk4.y : e == 2 ? dk4.z : dk4.w;
                        vis = vis && dkv == qm.docq;
                    }
                    pv = vis ? pv : 0.0f;
                }
                float ds = pv * (dp[r] - Dl) * scale;
                if (SOFTCAP) ds *= 1.0f - (y * inv_cap) * (y * inv_cap);
                s[r] = ds;
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 db16;
#pragma unroll
            for (int e = 0; e < 8; ++e) db16[e] = static_cast<__bf16>(s[s2 * 8 + e]);
#pragma unroll
            for (int d = 0; d < D / 32; ++d) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    &sm.kt[(d * 32 + n) * DqSmem<D>::TS + kb * 32 + s2 * 16 + hl * 8]);
                dq[d] = mfma32(a, db16, dq[d]);
            }
        }
    }
}

template <int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) DqSmem<D> sm;
    const int nt = p.nt;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = wg / nt;
    const int i = nt - 1 - (wg % nt);
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int qpos = i * kTile + wv * 32 + n;

    const __bf16 *qb_ = static_cast<const __bf16 *>(p.q) + b * p.q_sb + h * p.q_sh;
    const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + b * p.k_sb + h * p.k_sh;
    const __bf16 *vb_ = static_cast<const __bf16 *>(p.v) + b * p.v_sb + h * p.v_sh;
    const __bf16 *gb_ = static_cast<const __bf16 *>(p.dout) + b * p.do_sb + h * p.do_sh;

    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        qf[st] = *reinterpret_cast<const bf16x8 *>(qb_ + (int64_t)qpos * p.q_st + st * 16 + hl * 8);
        gf[st] = *reinterpret_cast<const bf16x8 *>(gb_ + (int64_t)qpos * p.do_st + st * 16 + hl * 8);
    }
    const int64_t row_bh = ((int64_t)b * p.H + h) * p.T + qpos;
    const float lse = p.lse[row_bh];
    const float L = lse == -INFINITY ? 0.0f : lse * kLog2e;
    const float Dl = p.delta[row_bh];

    const int bm = p.mask_b == 1 ? 0 : b;
    const int64_t row = (int64_t)bm * nt + i;
    const int nfull = min(max(p.full_kv_num[row], 0), nt);
    const int npart = min(max(p.kv_num[row], 0), nt);
    const int32_t *fidx = p.full_kv_idx + row * nt;
    const int32_t *pidx = p.kv_idx + row * nt;
    const int total = nfull + npart;

    QueryMask qm;
    qm.doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    const int32_t *doc = qm.doc_on ? p.doc_ids + (int64_t)bm * p.T : nullptr;
    qm.docq = qm.doc_on ? doc[qpos] : 0;
    qm.khi = (p.mask_flags & BSM_MASK_CAUSAL) ? qpos : p.T - 1;
    qm.klo = -1;
    qm.sink_end = 0;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        int64_t lo = (int64_t)qpos - (int64_t)(*p.window) + 1;
        lo = lo < -1 ? -1 : (lo > p.T ? p.T : lo);
        qm.klo = (int32_t)lo;
        if ((p.mask_flags & BSM_MASK_SINKS) && p.sinks > 0) qm.sink_end = p.sinks;
    }

    const float scale = p.scale;
    const float scale_log2 = p.scale * kLog2e;
    const float slope = ALIBI ? p.alibi_slopes[h] : 0.0f;
    const float cap = SOFTCAP ? p.softcap : 1.0f;
    const float inv_cap = 1.0f / cap;

    f32x16 dq[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[d][r] = 0.0f;

    for (int it = 0; it < total; ++it) {
        const int j = clamp_tile(it < nfull ? fidx[it] : pidx[it - nfull], nt);
        RowsUnits<D> uk, uv;
        load_rows<D>(uk, kb_, p.k_st, j * kTile);
        load_rows<D>(uv, vb_, p.v_st, j * kTile);
        int dk = 0;
        if (qm.doc_on && tid < kTile) dk = doc[j * kTile + tid];
        __syncthreads();
        store_rows<D>(uk, sm.k, DqSmem<D>::RS, sm.kt, DqSmem<D>::TS);
        store_rows<D>(uv, sm.v, DqSmem<D>::RS, nullptr, 0);
        if (tid < kTile) sm.doc[tid] = dk;
        __syncthreads();
        if (it < nfull)
            dq_tile<D, ALIBI, SOFTCAP, false>(sm, qf, gf, dq, j, qpos, L, Dl, qm, scale_log2, scale, slope, cap,
                                              inv_cap);
        else
            dq_tile<D, ALIBI, SOFTCAP, true>(sm, qf, gf, dq, j, qpos, L, Dl, qm, scale_log2, scale, slope, cap,
                                             inv_cap);
    }

    __bf16 *dqp = static_cast<__bf16 *>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qpos * p.dq_st;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) store_acc_rows(dqp, dq[d], d * 32, hl, 1.0f);
}

template <int D, bool ALIBI, bool SOFTCAP>
void launch_main(const AttnParams &p, hipStream_t stream) {
    const dim3 grid(p.B * p.H * p.nt), block(kThreads);
    hipLaunchKernelGGL((dkdv_kernel<D, ALIBI, SOFTCAP>), grid, block, 0, stream, p);
    hipLaunchKernelGGL((dq_kernel<D, ALIBI, SOFTCAP>), grid, block, 0, stream, p);
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    constexpr int RPB = kThreads / (D / 8);
    const int64_t rows = (int64_t)p.B * p.H * p.T;
    hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, stream, p);
    const bool alibi = p.mod_flags & BSM_MOD_ALIBI;
    const bool cap = p.mod_flags & BSM_MOD_SOFTCAP;
    if (alibi && cap)
        launch_main<D, true, true>(p, stream);
    else if (alibi)
        launch_main<D, true, false>(p, stream);
    else if (cap)
        launch_main<D, false, true>(p, stream);
    else
        launch_main<D, false, false>(p, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnParams &p, int D, hipStream_t stream) {
    if (D == 64) return launch_d<64>(p, stream);
    return launch_d<128>(p, stream);
}

}  // namespace bsm
