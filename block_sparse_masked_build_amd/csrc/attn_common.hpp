// Device helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include "bsm_internal.hpp"

namespace bsm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Scheduling hints for a straight-line block of N (LDS read -> MFMA) pairs:
// issue `ahead` reads first, then alternate one product and one read, then
// drain the last products.
template <int N, int ahead>
__device__ inline void sched_interleave() {
    __builtin_amdgcn_sched_group_barrier(0x100, ahead, 0);
#pragma unroll
    for (int x = 0; x < N - ahead; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, ahead, 0);
}

// Same for a block of N products whose B operands come from VALU work (the
// probabilities): reads and VALU are left free, products are spread out.
template <int N, int ahead>
__device__ inline void sched_interleave_valu() {
    __builtin_amdgcn_sched_group_barrier(0x100, ahead, 0);
#pragma unroll
    for (int x = 0; x < N - ahead; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, ahead, 0);
}

// Workgroup barrier ordering LDS accesses only: the tiles exchanged through
// it live in LDS, so global loads still in flight need not be waited for.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// Tiles in LDS.  A 128 x D bf16 tile is stored row-major without padding; the
// 16-byte chunks of row r are permuted by XOR with a row-dependent value so
// that the two read patterns below hit distinct banks:
//   * 16-byte reads of one chunk column by 32 consecutive rows (the A operand
//     of S^T = K Q^T): f_K spreads 16 consecutive rows over 16 bank groups;
//   * transposing 8-byte reads (ds_read_tr16_b64) of 4 chunks by 8
//     consecutive rows (the A operand of O^T += V^T P^T): f_V spreads 4
//     consecutive rows x 4 chunks over 16 bank groups.
template <int D>
struct TileLayout;

template <>
struct TileLayout<128> {
    static constexpr int kRowBytes = 256;
    static constexpr int kChunks = 16;
    __device__ static int fk(int r) { return r & 15; }
    __device__ static int fv(int r) { return (r & 3) << 2; }
};

template <>
struct TileLayout<64> {
    static constexpr int kRowBytes = 128;
    static constexpr int kChunks = 8;
    __device__ static int fk(int r) { return (r >> 1) & 7; }
    __device__ static int fv(int r) { return ((r >> 1) & 1) << 2; }
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ inline uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}

// One asynchronous HBM -> LDS copy per lane: 16 bytes from `g` land at LDS
// byte lds_base + 16 * lane (lds_base wave-uniform, passed through M0).
// Issued as inline assembly so that the compiler's wait-count pass, which
// cannot tell which LDS object a pending copy writes and would otherwise
// drain every copy before any LDS read, leaves the accounting to the caller
// (wait_vmcnt before the barrier that publishes the tile).
__device__ inline void copy16_to_lds(const void *g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g)
                 : "memory", "m0");
}

// Same with the scalar-base address form: 16 bytes from gbase + voff (gbase
// wave-uniform in scalar registers, voff a 32-bit per-lane offset), so no
// per-lane 64-bit address arithmetic is needed.
__device__ inline uint64_t uniform_u64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline void copy16_to_lds_s(const void *gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff),
                   "s"(uniform_u64((uint64_t)(uintptr_t)gbase))
                 : "memory", "m0");
}

// Same, 4 bytes per lane (lanes land at lds_base + 4 * lane).
__device__ inline void copy4_to_lds(const void *g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g)
                 : "memory", "m0");
}

// Asynchronous global -> LDS copies of this wave's quarter of a 128-row tile
// (one 16-byte chunk per lane per instruction; lane l of an instruction lands
// at byte 16 l of a 1 KiB LDS block, so the lane picks the global chunk that
// belongs there under the swizzle).  Completion is tracked by vmcnt.
// Addresses are a wave-uniform base (scalar registers) plus a 32-bit per-lane
// offset; with the swizzles above only a handful of distinct offsets occur.
// Index of this thread's wave as a scalar (wave-uniform) value, so that the
// uniform parts of copy addresses are computed by the scalar unit.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <int D, bool IS_V, int ROWS = kTile>
__device__ inline void issue_tile_to_lds(__bf16 *lds_tile, const __bf16 *g_row0, int64_t row_stride) {
    using L = TileLayout<D>;
    constexpr int kRowsPerInstr = 1024 / L::kRowBytes;
    constexpr int kInstr = ROWS / kRowsPerInstr / 4;
    static_assert(kInstr >= 1, "at least one copy per wave");
    const int wv = wave_id(), lane = threadIdx.x & 63;
    const int64_t row_bytes = row_stride * 2;
    const char *wbase = reinterpret_cast<const char *>(g_row0) + (int64_t)(wv * kInstr * kRowsPerInstr) * row_bytes;
    const int q = lane / L::kChunks;  // row inside the instruction's block
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
        // (wv * kInstr + x) * kRowsPerInstr is a multiple of 16 plus a
        // function of x only, so the swizzle depends on (x, q) alone.
        const int r16 = (x * kRowsPerInstr + q) & 15;
        const int c = (lane % L::kChunks) ^ (IS_V ? L::fv(r16) : L::fk(r16));
        const uint32_t voff = (uint32_t)(q * row_bytes) + (uint32_t)(c * 16);
        const char *xbase = wbase + (int64_t)(x * kRowsPerInstr) * row_bytes;
        copy16_to_lds_s(xbase, voff, lds_addr(lds_tile + ((wv * kInstr + x) * kRowsPerInstr) * D));
    }
}

template <int D>
constexpr int tile_lds_instr() { return kTile / (1024 / TileLayout<D>::kRowBytes) / 4; }

// N int32 values, N/4 per wave (wave w copies entries w N/4 .. (w+1) N/4 - 1).
template <int N = kTile>
__device__ inline void issue_ints_to_lds(int32_t *lds, const int32_t *g) {
    constexpr int kPer = N / 4;
    const int wv = wave_id(), lane = threadIdx.x & 63;
    if (lane < kPer) copy4_to_lds(g + wv * kPer + lane, lds_addr(lds + wv * kPer));
}

// s_waitcnt on vmcnt only (gfx9 encoding; expcnt and lgkmcnt left at max).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ inline i16x4 ds_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

// Barrier for the asynchronous tile copies.  A fenced __syncthreads would
// wait for every copy in flight (the copies write LDS, so a workgroup
// release must drain them); here the caller states what must be complete:
//   wait_vmcnt<N>() before it: this wave's copies except the newest N landed;
//   wait_lds_reads() before it: this wave's LDS reads have returned.
// The empty asm with a memory clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ inline void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ inline void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xc07f & ~(15 << 8)); }

// Wave-uniform load of data the kernel never writes (block-mask counts and
// indices): through the constant address space it becomes a scalar load,
// tracked by lgkmcnt rather than vmcnt, so it never waits on tile copies.
__device__ inline int32_t load_uniform(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)(p);
}

// Scheduling pattern for a straight-line block of N_MFMA matrix products
// whose A operands come from LDS (READS_PER reads each) mixed with
// independent VALU work: AHEAD reads first, then per product one MFMA, its
// share of the following reads and VALU_PER vector instructions.
template <int N_MFMA, int READS_PER, int AHEAD, int VALU_PER>
__device__ inline void sched_interleave_mfma_valu() {
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int x = 0; x < N_MFMA; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, READS_PER, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
    }
}

__device__ inline int clamp_tile(int j, int nt) { return j < 0 ? 0 : (j >= nt ? nt - 1 : j); }

// Key slot inside a 16-key group of the transposed value tile: bits 2 and 3
// of the key index are swapped, so that the 8 keys one lane feeds to a
// 32x32x16 product (keys {4h..4h+3} and {8+4h..8+4h+3} of the group, h the
// lane half) are contiguous.
__device__ inline int vt_slot(int key) {
    return (key & ~15) | (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
}

// 16-bit element i (0..7) of a 16-byte vector.
__device__ inline uint32_t u16_at(const u32x4 &x, int i) {
    const uint32_t w = (i >> 1) == 0 ? x.x : (i >> 1) == 1 ? x.y : (i >> 1) == 2 ? x.z : x.w;
    return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// Writes the transpose of a 4-row x 8-column bf16 block (rows r0..r0+3, one
// 16-byte vector each, columns c0..c0+7) into a [column][row] LDS array with
// row stride `ld`: column c gets the 4 values as one 8-byte store at the
// permuted slot vt_slot(r0) (r0 a multiple of 4).
__device__ inline void store_transposed_4x8(__bf16 *dst, int ld, int r0, int c0, const u32x4 (&v)[4]) {
    const int slot = vt_slot(r0);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        u32x2 w;
        w.x = u16_at(v[0], dd) | (u16_at(v[1], dd) << 16);
        w.y = u16_at(v[2], dd) | (u16_at(v[3], dd) << 16);
        *reinterpret_cast<u32x2 *>(&dst[(c0 + dd) * ld + slot]) = w;
    }
}

}  // namespace bsm
