// Block-sparse masked attention for decoding: one query per (batch, head)
// at the last position of the key/value cache, for gfx950.
//
// Method (tutorial "FlexAttention in PyTorch", "Decoding and paged KV
// caches": during generation the query length is 1 and the mask is taken
// against the current key length; a dedicated path serves short queries).
// The query sits at position p = kv_len - 1 and sees key kv when the mask
// predicate holds for (p, kv); its scores go through the same score
// modifications as the forward's.
//
// Mapping to CDNA4: a single query has no matrix-product shape, and the
// work is a stream of K and V read once, so the path is HBM-bound and runs on
// the vector units:
//  * decode_partial_kernel: one workgroup of 4 waves per (chunk of 1024 keys,
//    batch x head).  Lane = key for the scores (the query row is broadcast
//    from LDS), then lane = head dimension for the value sum (each key's
//    value row read as one coalesced 256-byte line).  fp32 online softmax per
//    wave, waves merged through LDS; the chunk's (max, sum, unnormalised
//    output) go to the workspace.  Chunks holding no visible key skip their
//    loads.
//  * decode_combine_kernel: one workgroup per (batch, head) merges the chunks
//    through their log-sum-exps and writes out (bf16) and lse (fp32, natural
//    log).
#include <cmath>

#include "bsm_internal.hpp"

namespace bsm {
namespace {

typedef __bf16 dec_bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;

struct DecodeParams {
    int32_t B, H, kv_len, D, nsplit;
    uint32_t mask_flags, mod_flags;
    int32_t sinks, prefix;
    float scale, softcap;
    const int32_t *doc_ids;      // [mask_b, kv_len] or NULL
    const int32_t *window;       // device scalar or NULL
    int32_t mask_b;
    const float *alibi_slopes;   // [H] or NULL
    const __bf16 *q; int64_t q_sb, q_sh;
    const __bf16 *k; int64_t k_sb, k_sh, k_st;
    const __bf16 *v; int64_t v_sb, v_sh, v_st;
    __bf16 *o; int64_t o_sb, o_sh;
    float *lse;                  // [B, H]
    float *part_o;               // [B*H, nsplit, D]
    float *part_ml;              // [B*H, nsplit, 2]: running max and sum
};

// Visibility of key kv for the query at p (the mask predicate written out;
// with the query last, the causal term and its prefix widening admit every
// key at or before p).
__device__ inline bool dec_visible(const DecodeParams &P, int b, int p, int kv, int window, int docq) {
    if ((P.mask_flags & BSM_MASK_CAUSAL) && kv > p && !(kv < P.prefix)) return false;
    if (P.mask_flags & BSM_MASK_DOCUMENT) {
        const int bm = P.mask_b == 1 ? 0 : b;
        if (P.doc_ids[(int64_t)bm * P.kv_len + kv] != docq) return false;
    }
    if (P.mask_flags & BSM_MASK_WINDOW) {
        const bool in_win = (int64_t)p - kv < window;
        const bool sink = (P.mask_flags & BSM_MASK_SINKS) && kv < P.sinks;
        if (!in_win && !sink) return false;
    }
    return true;
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(DecodeParams P) {
    constexpr int kChunk = 1024;          // keys per workgroup
    constexpr int kPerWave = kChunk / kDecWaves;
    constexpr int kDimsPerLane = D / 64;  // output dims per lane: lane * kDimsPerLane + i
    __shared__ float sq[D];               // the query row, fp32
    __shared__ float sp[kDecWaves][64];   // probabilities of a wave's 64 keys
    __shared__ float sm[kDecWaves], sl[kDecWaves];
    __shared__ float so[kDecWaves][D];

    const int split = blockIdx.x, bh = blockIdx.y;
    const int b = bh / P.H, h = bh - b * P.H;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int p = P.kv_len - 1;
    const int window = (P.mask_flags & BSM_MASK_WINDOW) ? *P.window : 0;
    int docq = 0;
    if (P.mask_flags & BSM_MASK_DOCUMENT) docq = P.doc_ids[(int64_t)(P.mask_b == 1 ? 0 : b) * P.kv_len + p];
    const float slope = (P.mod_flags & BSM_MOD_ALIBI) ? P.alibi_slopes[h] : 0.0f;
    const bool capped = P.mod_flags & BSM_MOD_SOFTCAP;

    // A chunk wholly before the window (and holding no sink) sees nothing:
    // its partial is (-inf, 0, 0) without touching K or V.
    if (P.mask_flags & BSM_MASK_WINDOW) {
        const int64_t c0 = (int64_t)split * kChunk, c1 = min((int64_t)(split + 1) * kChunk, (int64_t)P.kv_len);
        const bool before = (int64_t)p - (c1 - 1) >= window;
        const bool sink = (P.mask_flags & BSM_MASK_SINKS) && c0 < P.sinks;
        if (before && !sink) {
            const int64_t slot = (int64_t)bh * P.nsplit + split;
            for (int d = threadIdx.x; d < D; d += kDecThreads) P.part_o[slot * D + d] = 0.0f;
            if (threadIdx.x == 0) {
                P.part_ml[slot * 2] = -INFINITY;
                P.part_ml[slot * 2 + 1] = 0.0f;
            }
            return;
        }
    }

    const __bf16 *qrow = P.q + b * P.q_sb + h * P.q_sh;
    for (int d = threadIdx.x; d < D; d += kDecThreads) sq[d] = static_cast<float>(qrow[d]);
    __syncthreads();

    const __bf16 *kb = P.k + b * P.k_sb + h * P.k_sh;
    const __bf16 *vb = P.v + b * P.v_sb + h * P.v_sh;
    float m = -INFINITY, l = 0.0f;
    float o[kDimsPerLane];
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) o[i] = 0.0f;

    const int k_begin = split * kChunk + wv * kPerWave;
#pragma unroll 1
    for (int sub = 0; sub < kPerWave; sub += 64) {
        const int kv = k_begin + sub + lane;
        float s = -INFINITY;
        if (kv < P.kv_len && dec_visible(P, b, p, kv, window, docq)) {
            const __bf16 *krow = kb + (int64_t)kv * P.k_st;
            float acc = 0.0f;
#pragma unroll
            for (int d0 = 0; d0 < D; d0 += 8) {
                const dec_bf16x8 kk = *reinterpret_cast<const dec_bf16x8 *>(krow + d0);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(sq[d0 + e], static_cast<float>(kk[e]), acc);
            }
            s = acc * P.scale;
            if (P.mod_flags & BSM_MOD_ALIBI) s -= slope * (float)(p - kv);
            if (capped) s = P.softcap * tanhf(s / P.softcap);
        }
        // online softmax over this wave's 64 keys
        float mx = s;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_new = fmaxf(m, mx);
        const float pk = m_new == -INFINITY ? 0.0f : __expf(s - m_new);
        const float alpha = m_new == -INFINITY ? 1.0f : __expf(m - m_new);
        float ps = pk;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
        l = l * alpha + ps;
        m = m_new;
        sp[wv][lane] = pk;  // read back by every lane of this wave (LDS operations stay in order)
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) o[i] *= alpha;
        const int nk = min(64, P.kv_len - (k_begin + sub));
        if (mx != -INFINITY) {
            // value rows of the wave's keys, 16 at a time with their loads
            // issued together (keys past the cache end contribute p = 0 and
            // read the last row instead)
            const __bf16 *vbase = vb + lane * kDimsPerLane;
#pragma unroll 1
            for (int j0 = 0; j0 < 64; j0 += 16) {
                float vv[16][kDimsPerLane];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = min(k_begin + sub + j0 + j, P.kv_len - 1);
                    const __bf16 *vrow = vbase + (int64_t)key * P.v_st;
#pragma unroll
                    for (int i = 0; i < kDimsPerLane; ++i) vv[j][i] = static_cast<float>(vrow[i]);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float pj = j0 + j < nk ? sp[wv][j0 + j] : 0.0f;
#pragma unroll
                    for (int i = 0; i < kDimsPerLane; ++i) o[i] = __builtin_fmaf(pj, vv[j][i], o[i]);
                }
            }
        }
    }
    // merge the four waves
    if (lane == 0) {
        sm[wv] = m;
        sl[wv] = l;
    }
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) so[wv][lane * kDimsPerLane + i] = o[i];
    __syncthreads();
    if (wv == 0) {
        float M = sm[0];
        for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, sm[w]);
        float L = 0.0f, acc[kDimsPerLane];
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) acc[i] = 0.0f;
        for (int w = 0; w < kDecWaves; ++w) {
            const float f = (M == -INFINITY) ? 0.0f : __expf(sm[w] - M);
            L += sl[w] * f;
#pragma unroll
            for (int i = 0; i < kDimsPerLane; ++i) acc[i] += so[w][lane * kDimsPerLane + i] * f;
        }
        const int64_t slot = (int64_t)bh * P.nsplit + split;
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) P.part_o[slot * D + lane * kDimsPerLane + i] = acc[i];
        if (lane == 0) {
            P.part_ml[slot * 2] = M;
            P.part_ml[slot * 2 + 1] = L;
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
    for (int s = 0; s < P.nsplit; ++s) M = fmaxf(M, P.part_ml[((int64_t)bh * P.nsplit + s) * 2]);
    float L = 0.0f, acc[kDimsPerLane];
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) acc[i] = 0.0f;
#pragma unroll 8
    for (int s = 0; s < P.nsplit; ++s) {  // independent loads, unrolled so they overlap
        const int64_t slot = (int64_t)bh * P.nsplit + s;
        const float f = (M == -INFINITY) ? 0.0f : __expf(P.part_ml[slot * 2] - M);
        L += P.part_ml[slot * 2 + 1] * f;
#pragma unroll
        for (int i = 0; i < kDimsPerLane; ++i) acc[i] += P.part_o[slot * D + lane * kDimsPerLane + i] * f;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    __bf16 *orow = P.o + b * P.o_sb + h * P.o_sh;
#pragma unroll
    for (int i = 0; i < kDimsPerLane; ++i) orow[lane * kDimsPerLane + i] = static_cast<__bf16>(acc[i] * inv);
    if (lane == 0) P.lse[bh] = L > 0.0f ? M + logf(L) : -INFINITY;
}

template <int D>
hipError_t launch_d(const DecodeParams &P, hipStream_t stream) {
    hipLaunchKernelGGL((decode_partial_kernel<D>), dim3(P.nsplit, P.B * P.H), dim3(kDecThreads), 0, stream, P);
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(P.B * P.H), dim3(64), 0, stream, P);
    return hipGetLastError();
}

}  // namespace

int decode_splits(int kv_len) { return (kv_len + 1023) / 1024; }

hipError_t launch_attn_decode(const AttnParams &a, int D, float *part, hipStream_t stream) {
    DecodeParams P{};
    P.B = a.B;
    P.H = a.H;
    P.kv_len = a.T;
    P.D = D;
    P.nsplit = decode_splits(a.T);
    P.mask_flags = a.mask_flags;
    P.mod_flags = a.mod_flags;
    P.sinks = a.sinks;
    P.prefix = a.prefix;
    P.scale = a.scale;
    P.softcap = a.softcap;
    P.doc_ids = a.doc_ids;
    P.window = a.window;
    P.mask_b = a.mask_b;
    P.alibi_slopes = a.alibi_slopes;
    P.q = static_cast<const __bf16 *>(a.q);
    P.q_sb = a.q_sb;
    P.q_sh = a.q_sh;
    P.k = static_cast<const __bf16 *>(a.k);
    P.k_sb = a.k_sb;
    P.k_sh = a.k_sh;
    P.k_st = a.k_st;
    P.v = static_cast<const __bf16 *>(a.v);
    P.v_sb = a.v_sb;
    P.v_sh = a.v_sh;
    P.v_st = a.v_st;
    P.o = static_cast<__bf16 *>(a.o);
    P.o_sb = a.o_sb;
    P.o_sh = a.o_sh;
    P.lse = a.lse;
    P.part_o = part;
    P.part_ml = part + (int64_t)a.B * a.H * P.nsplit * D;
    if (D == 64) return launch_d<64>(P, stream);
    return launch_d<128>(P, stream);
}

}  // namespace bsm
