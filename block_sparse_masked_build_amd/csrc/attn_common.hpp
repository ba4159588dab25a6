// Device helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include "bsm_internal.hpp"

namespace bsm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32] on the bf16 matrix cores.
// Operand layout (wave64): A row i, k-slot kk sits in lane i + 32*(kk/8),
// element kk%8; B column j, k-slot kk in lane j + 32*(kk/8), element kk%8;
// D row i, column j in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
__device__ inline f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh(x) = 1 - 2 / (exp(2x) + 1), with exp(2x) = 2^(2x log2 e).
// Saturates to +-1 for large |x| (2^inf = inf -> rcp = 0; 2^-inf = 0).
__device__ inline float tanh_exp2(float x) {
    const float e = fast_exp2(x * (2.0f * kLog2e));
    return 1.0f - 2.0f * fast_rcp(e + 1.0f);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Linear workgroup id -> id with consecutive ids on one XCD.  Workgroups are
// dispatched round-robin over the 8 XCDs (each with its own L2), so mapping
// slot s of XCD x to a contiguous range keeps neighbouring query tiles of one
// head -- which read the same key/value tiles -- in the same L2.
__device__ inline int xcd_remap(int L, int N) {
    constexpr int kXcd = 8;
    const int per = N / kXcd, rem = N % kXcd;
    const int x = L % kXcd, slot = L / kXcd;
    return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

__device__ inline int clamp_tile(int j, int nt) { return j < 0 ? 0 : (j >= nt ? nt - 1 : j); }

// Key slot inside a 16-key group of the transposed value tile: bits 2 and 3
// of the key index are swapped, so that the 8 keys one lane feeds to a
// 32x32x16 product (keys {4h..4h+3} and {8+4h..8+4h+3} of the group, h the
// lane half) are contiguous.
__device__ inline int vt_slot(int key) {
    return (key & ~15) | (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
}

}  // namespace bsm
