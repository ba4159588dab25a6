// Device helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include "bsm_internal.hpp"

namespace bsm {

// Element type of q, k, v, out and the gradients, and of the matrix-core
// operands formed from them: bf16, or fp16 when the source is compiled with
// BSM_ELEM_FP16.  Each attention source is compiled once per type; the
// launchers it exports carry the type in their names (BSM_ELEM_FN).
#ifdef BSM_ELEM_FP16
typedef _Float16 elem_t;
#define BSM_ELEM_SUFFIX f16
#else
typedef __bf16 elem_t;
#define BSM_ELEM_SUFFIX bf16
#endif
#define BSM_CAT2(a, b) a##_##b
#define BSM_CAT(a, b) BSM_CAT2(a, b)
#define BSM_ELEM_FN(name) BSM_CAT(name, BSM_ELEM_SUFFIX)

typedef elem_t elem8 __attribute__((ext_vector_type(8)));
typedef elem_t elem4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32] on the matrix cores (bf16 or fp16
// operands, fp32 accumulation).
// Operand layout (wave64): A row i, k-slot kk sits in lane i + 32*(kk/8),
// element kk%8; B column j, k-slot kk in lane j + 32*(kk/8), element kk%8;
// D row i, column j in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
__device__ inline f32x16 mfma32(const elem8 &a, const elem8 &b, const f32x16 &c) {
#ifdef BSM_ELEM_FP16
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}

// An element given by its 16 bits, as fp32.
__device__ inline float elem_bits_to_float(uint32_t bits) {
#ifdef BSM_ELEM_FP16
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
#else
    return __builtin_bit_cast(float, bits << 16);
#endif
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Score modifications with their constants folded once per item.  The
// modified score leaves in the log2 domain:
//   plain / ALiBi:  t = (s scale - slope (q - kv)) log2 e = s a + b
//   soft-capped:    t = cap tanh(z) log2 e with z = (s scale - slope (q - kv)) / cap,
//                   tanh z = 1 - 2 / (e^{2z} + 1), e^{2z} = 2^u, u = s a + b,
//                   so t = c1 - c2 / (2^u + 1)
// with a = scale f, b = -slope f (q - kv) and f = log2 e (plain) or
// 2 log2 e / cap (soft-capped), c1 = cap log2 e, c2 = 2 cap log2 e.  The
// ALiBi term b of each score is one fused multiply-add of its key offset.
// Saturation: 2^u = inf gives t = c1, 2^u = 0 gives t = c1 - c2 = -cap log2 e.
struct ModK {
    float a, slope_f;  // score multiplier, slope in the same domain
    float c1, c2;      // soft-cap constants
};

// The domain factor f (an additive term b enters as b f).
template <bool SOFTCAP>
__device__ inline float mod_f(float cap) { return SOFTCAP ? 2.0f * kLog2e / cap : kLog2e; }

template <bool SOFTCAP>
__device__ inline ModK mod_k(float scale, float slope, float cap) {
    const float f = mod_f<SOFTCAP>(cap);
    return {scale * f, slope * f, cap * kLog2e, 2.0f * cap * kLog2e};
}

// t from a raw score s and its ALiBi term b (ignored without ALiBi).
template <bool ALIBI, bool SOFTCAP>
__device__ inline float mod_apply(float s, float b, const ModK &k) {
    const float u = ALIBI ? __builtin_fmaf(s, k.a, b) : s * k.a;
    if (!SOFTCAP) return u;
    return __builtin_fmaf(-k.c2, fast_rcp(fast_exp2(u) + 1.0f), k.c1);
}

__device__ inline uint32_t pack_elem2(float lo, float hi) {
    const elem_t a = static_cast<elem_t>(lo);
    const elem_t b = static_cast<elem_t>(hi);
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

// Key-tile workgroup -> work index for the column kernels in chunked
// placement.  Workgroup L runs on XCD L % 8 and is that XCD's (L / 8)-th.
// Work indices go out in chunks of kColChunk consecutive ones (neighbouring
// key tiles read the same query tiles, so a chunk shares one L2), dealt to
// the 8 XCDs in rounds whose direction alternates (0..7, then 7..0): under a
// causal mask a head's early tiles carry the most work and it falls
// steadily, so each XCD gets an even share.  The grid is rounded up to whole
// rounds (col_grid); indices past the work exit at once.  A bijection of
// [0, col_grid(n)).
constexpr int kColChunk = 16;
inline unsigned col_grid(int64_t n) {
    const int64_t r = 8 * kColChunk;
    return (unsigned)((n + r - 1) / r * r);
}
__device__ inline int col_remap(int L) {
    const int x = L % 8, s = L / 8, round = s / kColChunk;
    const int xcd_pos = (round & 1) ? 7 - x : x;
    return (8 * round + xcd_pos) * kColChunk + s % kColChunk;
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
// Tiles in LDS.  A tile of rows x D bf16 is stored row-major without padding;
// the 16-byte chunks of row r are permuted by XOR with a row-dependent value
// so that the read patterns used on the tile hit distinct banks:
//   * row reads: 16-byte reads of one chunk column by 32 consecutive rows (a
//     matrix-core operand taken row by row) -- fk spreads 16 consecutive rows
//     over 16 bank groups;
//   * transposing reads: 8-byte ds_read_tr16_b64 of 4 chunks by 8
//     consecutive rows (an operand taken column by column) -- fv spreads 4
//     consecutive rows x 4 chunks over 16 bank groups;
//   * both patterns on one tile: fkv has fv's low-row bits in chunk bits 2-3
//     (so transposing reads stay conflict-free) and row bits 2-3 in chunk
//     bits 0-1 (so 16 consecutive rows still get 16 distinct chunks).
enum TileSwizzle { kSwzK = 0, kSwzV = 1, kSwzKV = 2 };

template <int D>
struct TileLayout;

template <>
struct TileLayout<128> {
    static constexpr int kRowBytes = 256;
    static constexpr int kChunks = 16;
    __device__ static int fk(int r) { return r & 15; }
    __device__ static int fv(int r) { return (r & 3) << 2; }
    __device__ static int fkv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};

template <>
struct TileLayout<64> {
    static constexpr int kRowBytes = 128;
    static constexpr int kChunks = 8;
    __device__ static int fk(int r) { return (r >> 1) & 7; }
    __device__ static int fv(int r) { return ((r >> 1) & 1) << 2; }
    __device__ static int fkv(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
};

// D = 256: 512-byte rows start on the same bank, as the 256-byte ones do,
// so the D = 128 patterns (four row bits into the chunk index) serve.
template <>
struct TileLayout<256> {
    static constexpr int kRowBytes = 512;
    static constexpr int kChunks = 32;
    __device__ static int fk(int r) { return r & 15; }
    __device__ static int fv(int r) { return (r & 3) << 2; }
    __device__ static int fkv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};

template <int D, int SWZ>
__device__ inline int tile_swizzle(int r) {
    using L = TileLayout<D>;
    return SWZ == kSwzK ? L::fk(r) : SWZ == kSwzV ? L::fv(r) : L::fkv(r);
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into LDS.  A generic address of LDS is the
// shared aperture base (zero low half) plus the LDS offset, so the low 32
// bits are the offset; taking them directly avoids a generic-to-LDS cast,
// whose null test the backend can emit as an illegal compare against the
// aperture register.
__device__ inline uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

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

// Same with a base that is already wave-uniform (from uniform_u64), so the
// per-copy offsets added to it stay scalar arithmetic.
__device__ inline void copy16_to_lds_u(uint64_t gbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(gbase)
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

// nvalid: rows g_row0 .. g_row0 + nvalid - 1 exist (wave-uniform; it may be
// <= 0 for a tile half wholly past the end, as long as row g_row0 + nvalid -
// 1 lies inside the tensor).  A whole tile takes the plain copies; in a tile
// cut short by the length a lane whose row lies past nvalid copies that last
// row instead, so the tile is read inside the tensor -- its extra rows are
// masked by the caller.  Both forms address a wave-uniform base plus a
// per-lane offset below kRowsPerInstr rows.
template <int D, int SWZ, int ROWS>
__device__ inline void issue_tile_to_lds_at(uint32_t lds_tile, const elem_t *g_row0, int64_t row_stride,
                                            int nvalid = ROWS) {
    using L = TileLayout<D>;
    constexpr int kRowsPerInstr = 1024 / L::kRowBytes;
    constexpr int kInstr = ROWS / kRowsPerInstr / 4;
    static_assert(kInstr >= 1, "at least one copy per wave");
    const int wv = wave_id(), lane = threadIdx.x & 63;
    const int64_t row_bytes = row_stride * 2;
    const int q = lane / L::kChunks;  // row inside the instruction's block
    nvalid = __builtin_amdgcn_readfirstlane(nvalid);
    if (nvalid >= ROWS) {
        // The wave's base goes to scalar registers once; the instructions'
        // bases below it are scalar adds.
        const uint64_t wbase = uniform_u64((uint64_t)(uintptr_t)(reinterpret_cast<const char *>(g_row0) +
                                                                 (int64_t)(wv * kInstr * kRowsPerInstr) * row_bytes));
#pragma unroll
        for (int x = 0; x < kInstr; ++x) {
            // (wv * kInstr + x) * kRowsPerInstr is a multiple of 16 plus a
            // function of x only, so the swizzle depends on (x, q) alone.
            const int r16 = (x * kRowsPerInstr + q) & 15;
            const int c = (lane % L::kChunks) ^ tile_swizzle<D, SWZ>(r16);
            const uint32_t voff = (uint32_t)(q * row_bytes) + (uint32_t)(c * 16);
            const uint64_t xbase = wbase + (uint64_t)((int64_t)(x * kRowsPerInstr) * row_bytes);
            copy16_to_lds_u(xbase, voff, lds_tile + (uint32_t)((wv * kInstr + x) * kRowsPerInstr * L::kRowBytes));
        }
        return;
    }
    const int last = nvalid - 1;
    const uint64_t gbase = uniform_u64((uint64_t)(uintptr_t)g_row0);
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
        const int xrow0 = (wv * kInstr + x) * kRowsPerInstr;
        const int xsrc0 = xrow0 < last ? xrow0 : last;  // scalar
        const int row = xrow0 + q;
        const int d = (row < last ? row : last) - xsrc0;  // 0 .. kRowsPerInstr - 1
        const int r16 = (x * kRowsPerInstr + q) & 15;
        const int c = (lane % L::kChunks) ^ tile_swizzle<D, SWZ>(r16);
        const uint32_t voff = (uint32_t)d * (uint32_t)row_bytes + (uint32_t)(c * 16);
        const uint64_t xbase = gbase + (uint64_t)((int64_t)xsrc0 * row_bytes);
        copy16_to_lds_u(xbase, voff, lds_tile + (uint32_t)(xrow0 * L::kRowBytes));
    }
}

template <int D, int SWZ, int ROWS>
__device__ inline void issue_tile_to_lds(elem_t *lds_tile, const elem_t *g_row0, int64_t row_stride,
                                         int nvalid = ROWS) {
    issue_tile_to_lds_at<D, SWZ, ROWS>(lds_addr(lds_tile), g_row0, row_stride, nvalid);
}

// N int32 values, N/4 per wave (wave w copies entries w N/4 .. (w+1) N/4 - 1);
// entries at or past nvalid repeat entry nvalid - 1 (which exists).
template <int N = kTile>
__device__ inline void issue_ints_to_lds(int32_t *lds, const int32_t *g, int nvalid = N) {
    constexpr int kPer = N / 4;
    const int wv = wave_id(), lane = threadIdx.x & 63;
    const int e = wv * kPer + lane;
    if (lane < kPer) copy4_to_lds(g + (e < nvalid ? e : nvalid - 1), lds_addr(lds + wv * kPer));
}

// Same with the LDS destination given as a byte address.
template <int N>
__device__ inline void issue_ints_to_lds_at(uint32_t lds, const int32_t *g, int nvalid = N) {
    constexpr int kPer = N / 4;
    const int wv = wave_id(), lane = threadIdx.x & 63;
    const int e = wv * kPer + lane;
    if (lane < kPer) copy4_to_lds(g + (e < nvalid ? e : nvalid - 1), lds + 4 * wv * kPer);
}

// Load of a T from an LDS byte address.
template <typename T>
__device__ inline T lds_load(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T *>((uintptr_t)addr);
}

// Store of a T to an LDS byte address.
template <typename T>
__device__ inline void lds_store(uint32_t addr, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T *>((uintptr_t)addr) = v;
}

// Atomic add of v to the float at an LDS byte address (ds_add_f32, no
// return value).
__device__ inline void lds_add(uint32_t addr, float v) {
    __hip_atomic_fetch_add(reinterpret_cast<__attribute__((address_space(3))) float *>((uintptr_t)addr), v,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Same for N 4-byte words of any type.
template <int N>
__device__ inline void issue_words_to_lds(void *lds, const void *g) {
    issue_ints_to_lds<N>(static_cast<int32_t *>(lds), static_cast<const int32_t *>(g));
}

// s_waitcnt on vmcnt only (gfx9 encoding; expcnt and lgkmcnt left at max).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ inline i16x4 ds_read_tr16(const elem_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ inline i16x4 ds_read_tr16_at(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)((uintptr_t)addr));
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

// Per-lane LDS byte offsets of matrix-core operands read from a tile stored
// with the fkv swizzle (read both ways).  Both patterns are XOR-structured,
// so one base per pattern is kept and each operand's offset is derived where
// it is used (row-block offsets are added as immediates):
//   row read (A operand [32 rows][16 columns], lane = row):
//       row ^ (st << 5)                           st = 16-column step
//   transposing read (A operand [32 columns][16 rows] of the tile transposed):
//       (tr ^ (db << 6) ^ (u << 5)) + 8 u rows    db = 32-column block,
//                                                 u = rows +0..3 / +8..11 of a 16-row group
struct KvOffsets {
    int row;
    int tr;
};

template <int D>
__device__ inline void kv_offsets(KvOffsets &off) {
    using L = TileLayout<D>;
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, hl = lane >> 5;
    // chunk (2 st + hl) ^ fkv(n) = (2 st) ^ (hl ^ fkv(n)): 2 st and hl occupy
    // different bits; n * kRowBytes is a multiple of 128.
    off.row = n * L::kRowBytes + ((hl ^ L::fkv(n)) << 4);
    // ds_read_tr16_b64: lane j of a 16-lane group G supplies the address of
    // row R0 + j/4, columns c0 + 4 (j%4) .. +3; lane i then receives rows
    // R0..R0+3 of column c0 + i.  c0 = 32 db + 16 (G%2), R0 = 4 (G/2) (+8
    // for u = 1) inside each 16-row group.  The column block adds 4 db to the
    // chunk index (an XOR, as the chunk's own low bits stay below bit 2), and
    // the 8 extra rows of u = 1 flip bit 1 of fkv.
    const int G = lane >> 4, j = lane & 15;
    const int r = 4 * (G >> 1) + (j >> 2);
    const int c = 2 * (G & 1) + ((j & 3) >> 1);
    off.tr = r * L::kRowBytes + ((c ^ L::fkv(r)) << 4) + ((j & 1) << 3);
}

// A operand [32 rows][16 columns] at row block rb, column step st of an fkv
// tile at LDS byte address `tile` (lane = row, 8 consecutive columns).
template <int D>
__device__ inline elem8 read_rows_operand(uint32_t tile, const KvOffsets &off, int rb, int st) {
    return lds_load<elem8>(tile + rb * 32 * TileLayout<D>::kRowBytes + (off.row ^ (st << 5)));
}

// A operand [32 columns][16 rows] of an fkv tile transposed: columns
// 32 db + lane%32, rows 16 g16 + {4 hl..4 hl+3, 8+4 hl..8+4 hl+3} with hl the
// lane half (the k-slot order of a 32x32 score block's registers).
template <int D>
__device__ inline elem8 read_cols_operand(uint32_t tile, const KvOffsets &off, int g16, int db) {
    const uint32_t base = tile + g16 * 16 * TileLayout<D>::kRowBytes;
    const i16x4 lo = ds_read_tr16_at(base + (off.tr ^ (db << 6)));
    const i16x4 hi = ds_read_tr16_at(base + 8 * TileLayout<D>::kRowBytes + (off.tr ^ ((db << 6) | 32)));
    return __builtin_bit_cast(elem8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
__device__ inline void store_transposed_4x8(elem_t *dst, int ld, int r0, int c0, const u32x4 (&v)[4]) {
    const int slot = vt_slot(r0);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        u32x2 w;
        w.x = u16_at(v[0], dd) | (u16_at(v[1], dd) << 16);
        w.y = u16_at(v[2], dd) | (u16_at(v[3], dd) << 16);
        *reinterpret_cast<u32x2 *>(&dst[(c0 + dd) * ld + slot]) = w;
    }
}

// ---------------------------------------------------------------------------
// How partial tiles are masked (chosen once per workgroup):
//   kPlain  -- visible keys of a query form one interval [lo, hi]
//              (causal, window and, with contiguous documents, the document);
//   kSinks  -- plus the sink interval [slo, shi];
//   kGather -- document ids are not contiguous runs: interval terms without
//              the document, then a per-key document id compare;
//   kTable  -- a composed mask: the five terms of every score index its
//              truth table; [lo, hi] holds the keys that exist.
enum MaskMode { kPlain = 0, kSinks = 1, kGather = 2, kTable = 3 };

struct RowMask {
    int32_t lo, hi;     // main visible interval of keys (inclusive)
    int32_t slo, shi;   // sink interval (empty when slo > shi)
    int32_t docq;       // document id of the query (kGather, kTable)
    // kTable only: key bounds of the terms -- causal key <= qpos, window
    // key >= wlo, sink key < sinks, prefix key < prefix (0: term off) -- and
    // the truth table (bit C + 2 Dc + 4 W + 8 S + 16 P)
    int32_t qpos, wlo, sinks, prefix;
    uint32_t table;
};

// Row view of a composed mask.  A lane's 32 keys of a step are kbase + c,
// c = 32 kb + 8 g + e (e < 4), numbered j = 16 kb + 4 g + e; each term, as
// a function of the key, is a threshold, so over the lane's keys it is a
// 32-bit mask with bit j for key j.  The truth table then combines the five
// masks bitwise (a tree of 31 two-way selects), and a score is kept or set
// to -inf by its bit.
//
// Number of the lane's offsets c below t (t clamped to [0, 64]).
__device__ inline int owned_below(int t) {
    t = min(max(t, 0), 64);
    return 4 * (t >> 3) + min(t & 7, 4);
}

// Bits j of the lane's keys with offset c < t.
__device__ inline uint32_t bits_below(int t) {
    const int n = owned_below(t);
    return n >= 32 ? ~0u : (1u << n) - 1u;
}

// (sel & a) | (~sel & b), bit by bit.
__device__ inline uint32_t bit_select(uint32_t sel, uint32_t a, uint32_t b) { return (sel & a) | (~sel & b); }

// The truth table (bit C + 2 Dc + 4 W + 8 S + 16 P) applied bitwise to the
// term masks.
__device__ inline uint32_t table_combine(uint32_t table, uint32_t c, uint32_t d, uint32_t w, uint32_t s,
                                         uint32_t p) {
    uint32_t l1[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t t0 = ((table >> (2 * k)) & 1u) ? ~0u : 0u;
        const uint32_t t1 = ((table >> (2 * k + 1)) & 1u) ? ~0u : 0u;
        l1[k] = bit_select(c, t1, t0);
    }
    uint32_t l2[8], l3[4], l4[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) l2[k] = bit_select(d, l1[2 * k + 1], l1[2 * k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) l3[k] = bit_select(w, l2[2 * k + 1], l2[2 * k]);
#pragma unroll
    for (int k = 0; k < 2; ++k) l4[k] = bit_select(s, l3[2 * k + 1], l3[2 * k]);
    return bit_select(p, l4[1], l4[0]);
}

// Visible keys of the lane for the step starting at key0, as bits j; sdoc
// is the LDS byte address of the step's key document ids, read when docs.
__device__ inline uint32_t table_row_bits(const RowMask &rm, uint32_t sdoc, int key0, bool docs) {
    const int hl = (threadIdx.x & 63) >> 5;
    const int kbase = key0 + hl * 4;
    const uint32_t c = bits_below(rm.qpos + 1 - kbase);  // key <= qpos
    const uint32_t w = ~bits_below(rm.wlo - kbase);      // key >= wlo
    const uint32_t s = bits_below(rm.sinks - kbase);     // key < sinks
    const uint32_t p = bits_below(rm.prefix - kbase);    // key < prefix
    const uint32_t v = bits_below(rm.hi + 1 - kbase);    // the key exists
    uint32_t d = 0;
    if (docs) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const i32x4 dk = lds_load<i32x4>(sdoc + 4 * (kb * 32 + g * 8 + hl * 4));
                const int j = kb * 16 + g * 4;
                d |= (dk.x == rm.docq ? 1u : 0u) << j;
                d |= (dk.y == rm.docq ? 2u : 0u) << j;
                d |= (dk.z == rm.docq ? 4u : 0u) << j;
                d |= (dk.w == rm.docq ? 8u : 0u) << j;
            }
    }
    return table_combine(rm.table, c, d, w, s, p) & v;
}

// Score kept when bit j of bits is set, -inf otherwise (a sign-extended bit
// field as the select mask).
__device__ inline float keep_if_bit(float x, uint32_t bits, int j) {
    const uint32_t m = (uint32_t)((int32_t)(bits << (31 - j)) >> 31);
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & m) | (~m & 0xff800000u));
}

// Stores a wave's 32 x D block of fp32 accumulators as bf16 rows, times mul
// (per lane, i.e. per row).  Accumulator layout: lane (row n, half hl) holds
// for column block db the columns 32 db + 8 g + 4 hl + e in register 4 g + e.
// The block passes through this wave's own 32 x 2D-byte LDS slice at
// `stage` (16-byte chunks of a row XOR-swizzled by the row, so neither side
// conflicts), then each store writes 16 bytes per lane and whole 2D-byte
// rows, instead of 16-byte pieces of 32 rows.  The exchange stays inside the
// wave, whose LDS accesses execute in order; the caller makes sure no other
// wave uses the slice.  dst is row 0 of the block, ld its row stride; only
// rows below nrows are stored (the block may run past the end of a length
// that is not a multiple of 128).
template <int D>
__device__ __attribute__((always_inline)) inline void store_rows_staged(elem_t *dst, int64_t ld,
                                                                        const f32x16 (&acc)[D / 32], float mul,
                                                                        uint32_t stage, int nrows = 32) {
    constexpr int kRowBytes = 2 * D, kChunks = kRowBytes / 16, kRowsPerRead = 64 / kChunks;
    const int lane = threadIdx.x & 63, n = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;  // columns 32 db + 8 g + 4 hl + 0..3: chunk 4 db + g, half hl
            w.x = pack_elem2(acc[db][g * 4 + 0] * mul, acc[db][g * 4 + 1] * mul);
            w.y = pack_elem2(acc[db][g * 4 + 2] * mul, acc[db][g * 4 + 3] * mul);
            lds_store<u32x2>(stage + n * kRowBytes + (((db * 4 + g) ^ (n % kChunks)) * 16) + hl * 8, w);
        }
    }
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerRead; ++i) {
        const int r = i * kRowsPerRead + lane / kChunks, c = lane % kChunks;
        const u32x4 v = lds_load<u32x4>(stage + r * kRowBytes + ((c ^ (r % kChunks)) * 16));
        if (r < nrows) *reinterpret_cast<u32x4 *>(dst + (int64_t)r * ld + c * 8) = v;
    }
}

// Row view (lane = query, S^T = K Q^T layout: lane (query n, half hl) holds
// for key block kb the keys 32 kb + 8 (r/4) + 4 hl + r%4 of a 64-key step).
// Score modifications (to the log2 domain) and the mask for the step whose
// first key is key0; sdoc is the LDS byte address of the step's key document
// ids (gather mode).  Applied to every step: on a full tile every pair is
// visible, so the mask changes nothing there.
__device__ inline bool in_range(int c, int lo_t, int span) {
    return (uint32_t)(c - lo_t) <= (uint32_t)span;  // lo_t <= c <= lo_t + span, span >= 0
}

// Relative-position bias table (one scalar per clipped distance q - kv in
// [-R, R]) of a head, staged in LDS (stage_bias_load / stage_bias_store)
// already multiplied by the log2-domain factor of mod_k.
struct BiasLds {
    uint32_t tab;  // LDS byte address of entry 0 (distance -R)
    int R;
};

// Bias terms of one step of the row view: key kbase + c at the register
// offsets c <= 59, distance t - c with t = qpos - kbase.  When every
// distance of the wave's step lies inside [-R, R] each term is one LDS read
// at a fixed offset from a per-lane base (no clip); otherwise the distance
// is clipped per score.
constexpr int kRowMaxOffset = 59;  // 32 + 3 * 8 + 3

__device__ inline void row_bias(float (&bt)[2][16], int kbase, int qpos, const BiasLds &bl) {
    const int t = qpos - kbase;
    if (__all(t - kRowMaxOffset >= -bl.R && t <= bl.R)) {
        const uint32_t a0 = bl.tab + 4u * (uint32_t)(t - kRowMaxOffset + bl.R);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
                bt[kb][r] = lds_load<float>(a0 + 4u * (uint32_t)(kRowMaxOffset - c));
            }
    } else {
        const uint32_t a0 = bl.tab + 4u * (uint32_t)bl.R;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
                const int d = min(max(t - c, -bl.R), bl.R);
                bt[kb][r] = lds_load<float>(a0 + 4u * (uint32_t)d);  // d < 0 wraps back below a0
            }
    }
}

// Copies a head's 2R + 1 bias entries, times f, into LDS at `tab`: the
// loads happen here, the LDS writes in stage_bias_store after the caller's
// wait for its loads, so that no wait for them stalls the tile copies
// issued in between.  Up to kBiasPerThread entries per thread.
constexpr int kBiasMaxEntries = 2 * BSM_BIAS_MAX_RADIUS + 1;
constexpr int kBiasPerThread = (kBiasMaxEntries + 255) / 256;

__device__ inline void stage_bias_load(const float *row, int n, float (&v)[kBiasPerThread]) {
#pragma unroll
    for (int j = 0; j < kBiasPerThread; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        v[j] = i < n ? row[i] : 0.0f;
    }
}

__device__ inline void stage_bias_store(const float (&v)[kBiasPerThread], int n, float f, uint32_t tab) {
#pragma unroll
    for (int j = 0; j < kBiasPerThread; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        if (i < n) lds_store<float>(tab + 4u * (uint32_t)i, v[j] * f);
    }
}

// Score modifications alone (row view, step starting at key0): the scores
// leave in the log2 domain.  Without modifications nothing is done here; the
// scale is folded into the exponential instead.  The ALiBi term of the
// score at key offset c (key - key0 - 4 hl) is slope_f c + n with
// n = -slope_f (q - key0 - 4 hl); a bias table's term (BIAS) takes its place.
template <bool ALIBI, bool SOFTCAP, bool BIAS = false>
__device__ inline void row_mods(f32x16 (&s)[2], int key0, int qpos, const ModK &mk, const BiasLds &bl = {}) {
    static_assert(!(ALIBI && BIAS), "one additive term at a time");
    if (!(ALIBI || SOFTCAP || BIAS)) return;
    const int hl = (threadIdx.x & 63) >> 5;
    float n = 0.0f, sf = mk.slope_f;
    if (ALIBI) {
        n = -mk.slope_f * (float)(qpos - (key0 + hl * 4));
        asm volatile("" : "+v"(n), "+v"(sf));  // per step: keeps the per-register terms from being hoisted
    }
    float bt[2][16];
    if (BIAS) row_bias(bt, key0 + hl * 4, qpos, bl);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
            const float b = ALIBI ? __builtin_fmaf((float)c, sf, n) : BIAS ? bt[kb][r] : 0.0f;
            s[kb][r] = mod_apply<ALIBI || BIAS, SOFTCAP>(s[kb][r], b, mk);
        }
}

template <bool ALIBI, bool SOFTCAP, int MODE, bool BIAS = false>
__device__ inline void row_mod_mask(uint32_t sdoc, f32x16 (&s)[2], int key0, int qpos, const ModK &mk,
                                    const RowMask &rm, bool partial, bool table_docs = false,
                                    const BiasLds &bl = {}) {
    const int hl = (threadIdx.x & 63) >> 5;
    const int kbase = key0 + hl * 4;
    row_mods<ALIBI, SOFTCAP, BIAS>(s, key0, qpos, mk, bl);
    if (!partial) return;  // full tile: every pair is visible
    // Bounds relative to this step, kept opaque so that the compiler compares
    // them with the per-register key offsets instead of hoisting 64
    // loop-invariant thresholds into registers.  An empty interval is encoded
    // as a start beyond every key with span 0, which no offset matches.
    int lo_t = rm.hi >= rm.lo ? rm.lo - kbase : 1 << 30;
    const int span = rm.hi >= rm.lo ? rm.hi - rm.lo : 0;
    int slo_t = rm.shi >= rm.slo ? rm.slo - kbase : 1 << 30;
    const int sspan = rm.shi >= rm.slo ? rm.shi - rm.slo : 0;
    asm volatile("" : "+v"(lo_t), "+v"(slo_t));
    if (MODE == kTable) {
        const uint32_t bits = table_row_bits(rm, sdoc, key0, table_docs);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint32_t half = (bits >> (16 * kb)) & 0xffffu;
            if (__all(half == 0xffffu)) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = keep_if_bit(s[kb][r], bits, kb * 16 + r);
        }
        return;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        // The wave's 32 queries x these 32 keys: skip the elementwise test
        // when every query sees every key, fill with -inf when none sees any.
        const int kf = key0 + kb * 32, kl = kf + 31;
        const bool all_vis = MODE != kGather && rm.lo <= kf && rm.hi >= kl;
        const bool none_vis = (rm.hi < kf || rm.lo > kl || rm.hi < rm.lo) &&
                              (MODE == kPlain || rm.shi < kf || rm.slo > kl || rm.shi < rm.slo);
        if (__all(all_vis)) continue;
        if (__all(none_vis)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = -INFINITY;
            continue;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            i32x4 dk = {0, 0, 0, 0};
            if (MODE == kGather) dk = lds_load<i32x4>(sdoc + 4 * (kb * 32 + g * 8 + hl * 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int c = kb * 32 + g * 8 + e;  // key - kbase
                bool vis = in_range(c, lo_t, span);
                if (MODE != kPlain) vis = vis || in_range(c, slo_t, sspan);
                if (MODE == kGather) {
                    const int dkv = e == 0 ? dk.x : e == 1 ? dk.y : e == 2 ? dk.z : dk.w;
                    vis = vis && dkv == rm.docq;
                }
                s[kb][r] = vis ? s[kb][r] : -INFINITY;
            }
        }
    }
}

// Elementwise mask of a partial tile's step (row view), without branches:
// every score is tested, hidden ones become -inf.  sdoc is the LDS byte
// address of the step's key document ids (kGather only).
template <int MODE>
__device__ inline void row_mask_flat(uint32_t sdoc, f32x16 (&s)[2], int key0, const RowMask &rm,
                                     bool table_docs = false) {
    const int hl = (threadIdx.x & 63) >> 5;
    const int kbase = key0 + hl * 4;
    // Bounds relative to this lane's first key, opaque so that the compiler
    // compares them with the per-register key offsets instead of hoisting 64
    // loop-invariant thresholds.  An empty interval starts beyond every key.
    int lo_t = rm.hi >= rm.lo ? rm.lo - kbase : 1 << 30;
    const int span = rm.hi >= rm.lo ? rm.hi - rm.lo : 0;
    int slo_t = rm.shi >= rm.slo ? rm.slo - kbase : 1 << 30;
    const int sspan = rm.shi >= rm.slo ? rm.shi - rm.slo : 0;
    asm volatile("" : "+v"(lo_t), "+v"(slo_t));
    if (MODE == kTable) {
        const uint32_t bits = table_row_bits(rm, sdoc, key0, table_docs);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = keep_if_bit(s[kb][r], bits, kb * 16 + r);
        return;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            i32x4 dk = {0, 0, 0, 0};
            if (MODE == kGather) dk = lds_load<i32x4>(sdoc + 4 * (kb * 32 + g * 8 + hl * 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = g * 4 + e;
                const int c = kb * 32 + g * 8 + e;  // key - kbase
                bool vis = in_range(c, lo_t, span);
                if (MODE != kPlain) vis = vis || in_range(c, slo_t, sspan);
                if (MODE == kGather) {
                    const int dkv = e == 0 ? dk.x : e == 1 ? dk.y : e == 2 ? dk.z : dk.w;
                    vis = vis && dkv == rm.docq;
                }
                s[kb][r] = vis ? s[kb][r] : -INFINITY;
            }
        }
}

// Maximum over a row-view step (32 scores per lane, both lane halves of a
// query combined): four independent chains, then the lane-half exchange as
// one cross-lane swap (no LDS round trip).
// Maxima of scores, which are never NaN: fmaxf would first quiet inputs it
// cannot prove canonical (IEEE mode), up to three instructions for one
// two-input maximum, so the chains use v_max3_f32 / v_max_f32 from inline
// assembly.  The compiler inserts no hazard wait states before inline
// assembly, and the hardware does not interlock a vector read of a register
// that a matrix-core product is still writing.  So no inline-assembly
// instruction may read a product's result first.  Each chain therefore
// starts from ready(), a canonicalisation (one v_max_f32 x, x) the compiler
// emits itself and so waits for the product before.  The chain's
// inline-assembly steps depend on its result, and the chain's other scores
// come from the same product, complete by then.
__device__ inline float ready(float a) { return __builtin_canonicalizef(a); }

__device__ inline float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ inline float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ inline float row_max(const f32x16 (&s)[2]) {
    float c[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int kb = x >> 1, r0 = (x & 1) * 8;
        float v = max3(ready(s[kb][r0]), s[kb][r0 + 1], s[kb][r0 + 2]);
        v = max3(v, s[kb][r0 + 3], s[kb][r0 + 4]);
        v = max3(v, s[kb][r0 + 5], s[kb][r0 + 6]);
        c[x] = max2(v, s[kb][r0 + 7]);
    }
    const float mx = max2(max3(c[0], c[1], c[2]), c[3]);
    const uint32_t u = __builtin_bit_cast(uint32_t, mx);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // the swap's results, too, are first read by a compiled instruction
    return max2(ready(__builtin_bit_cast(float, (uint32_t)sw[0])), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// Row view of the mask for query qpos (mask batch row bm): visible keys form
// [lo, hi] plus, with sinks, [slo, shi] (empty when slo > shi).  With
// contiguous documents the document bounds come from the exported document
// range; a row whose documents are not contiguous is flagged (-1) there, and
// then the interval terms exclude the document and docq holds the query's id
// for a per-key compare.  Returns the mode the row needs.
// Composed mask: every key that exists, the term bounds and the truth table
// (window: the int32 scalar read at run time).
__device__ inline void make_table_mask(const AttnParams &p, int qpos, int window, int32_t docq, RowMask &rm) {
    rm.lo = 0;
    rm.hi = p.T - 1;
    rm.slo = 0;
    rm.shi = -1;
    rm.docq = docq;
    rm.qpos = qpos;
    int64_t wlo = (int64_t)qpos - (int64_t)window + 1;
    if (!(p.mask_flags & BSM_MASK_WINDOW)) wlo = (int64_t)1 << 30;  // no key is in an absent window
    rm.wlo = wlo < -(1 << 30) ? -(1 << 30) : (wlo > (1 << 30) ? (1 << 30) : (int)wlo);
    rm.sinks = (p.mask_flags & BSM_MASK_SINKS) ? min(max(p.sinks, 0), p.T) : 0;
    rm.prefix = p.prefix;
    rm.table = p.table;
}

__device__ inline int make_row_mask(const AttnParams &p, int bm, int qpos, RowMask &rm) {
    const bool doc_on = p.mask_flags & BSM_MASK_DOCUMENT;
    int ds = 0, de = p.T - 1;
    rm.docq = 0;
    bool gather = false;
    if (doc_on) {
        const int32_t *dr = p.doc_range + ((int64_t)bm * p.npos + qpos) * 2;
        ds = dr[0];
        de = dr[1];
        gather = ds < 0;  // the whole row is marked, so every lane agrees
        if (gather) {
            ds = 0;
            de = p.T - 1;
            rm.docq = p.doc_ids[(int64_t)bm * p.npos + qpos];
        }
    }
    const int hi = min(min((p.mask_flags & BSM_MASK_CAUSAL) ? max(qpos, p.prefix - 1) : p.T - 1, de), p.T - 1);
    int lo = ds;
    bool sinks = false;
    if (p.mask_flags & BSM_MASK_WINDOW) {
        const int64_t wlo = (int64_t)qpos - (int64_t)(*p.window) + 1;
        if (wlo > lo) lo = wlo > p.T ? p.T : (int)wlo;
        sinks = (p.mask_flags & BSM_MASK_SINKS) && p.sinks > 0;
    }
    rm.lo = lo;
    rm.hi = hi;
    rm.slo = ds;
    rm.shi = sinks ? min(p.sinks - 1, hi) : ds - 1;
    return gather ? kGather : sinks ? kSinks : kPlain;
}

// Whether no (query, key) pair of the wave's 32 queries and keys kf..kl is
// visible in the row view (wave-uniform).
template <int MODE>
__device__ inline bool block_none_visible(const RowMask &rm, int kf, int kl) {
    const bool none = (rm.hi < kf || rm.lo > kl || rm.hi < rm.lo) &&
                      (MODE == kPlain || rm.shi < kf || rm.slo > kl || rm.shi < rm.slo);
    return __all(none);
}

// Whether the row direction (forward, dQ) needs its general kernel: a key
// length off the 128-key grid (the last tile's copies are clamped; its
// second half may lie wholly past KV_LEN) or 64-key blocks.  The other
// kernel has whole 128-key tiles and two 64-key steps per tile compiled in.
inline bool kv_ragged(const AttnParams &p) { return p.T % kTile != 0 || p.kb != kTile; }

// ---------------------------------------------------------------- item order
// Both attention directions run one workgroup per item: a row (forward, dQ)
// or a column (dK/dV) of tiles of the block mask, for one head index.  The
// block mask's work orders list rows / columns longest first, as records
// that let a workgroup start with one scalar load.

// One work-order record: (flat row, full tiles, partial tiles, first tile).
struct WorkRec {
    int packed, nfull, npart, first;
};

__device__ inline WorkRec load_rec(const int32_t *order, int e) {
    const i32x4 r = *(const __attribute__((address_space(4))) i32x4 *)(order + 4 * (int64_t)e);
    return {r.x, r.y, r.z, r.w};
}

// Item order.  Item k is work-order entry e for head (and, with a shared
// mask, batch entry) rem.  Items come in chunks of 2^ord_chunk_log2
// consecutive entries of one head -- rows that mostly share key and value
// tiles -- dealt to the Q queues in rounds of Q chunks whose direction
// alternates (chunk Q r + j goes to queue j in even rounds r and to queue
// Q - 1 - j in odd ones): the work order runs from the longest rows down,
// so alternating evens out the queues' work.  Workgroup b takes the
// (b / Q)-th item of queue b % Q.  Workgroups are dispatched round-robin
// over the XCDs, so with Q = 8 each queue runs on one XCD and the rows
// running at the same time there share tiles through its L2; items leave
// each queue in work order.  The host picks the chunk so that every queue
// gets several chunks.
constexpr int kQueues = 8;

// Workgroups per CU that the row kernels (forward, dQ) are compiled for.
// Both fit 66 KB of LDS and 256 registers per lane at two per CU.  At D = 64
// without score modifications the loops fit 168 registers with no spill
// inside them, and the LDS (33 KB) allows three: 12 waves per CU instead of
// 8.  With score modifications at 168 registers the loops would spill.
// At D = 256 the K/V buffers alone take 128 KB: one per CU, with up to 512
// registers per lane.
template <int D, bool MODS>
constexpr int kWgPerCu = D == 256 ? 1 : (D == 64 && !MODS) ? 3 : 2;

// Quotient k / d for 0 <= k < 2^31 and d >= 1, with m = ceil(2^32 / d)
// computed on the host (d >= 2; d = 1 is passed through): the estimate is
// q or q + 1.
__device__ inline int div_by(int k, int d, uint32_t m) {
    if (d == 1) return k;
    int q = (int)(((uint64_t)(uint32_t)k * m) >> 32);
    if ((int64_t)q * d > k) --q;
    return q;
}

struct ItemOrder {
    int nitems;  // mask rows x head indices, within int32 (checked on the host)
    int Q, queue, cl;
    const AttnParams &p;

    __device__ ItemOrder(const AttnParams &p_, int G) : p(p_) {
        nitems = p.mask_b * p.nqt * p.ord_r;
        Q = G < kQueues ? G : kQueues;
        queue = blockIdx.x % Q;
        cl = p.ord_chunk_log2;
    }
    // Item of this queue's i-th grab (>= nitems: the queue is empty).
    __device__ int item(int i) const {
        const int r = i >> cl;
        const int pos = (r & 1) ? Q - 1 - queue : queue;  // this queue's chunk in round r
        const int64_t k = (((int64_t)pos + (int64_t)Q * r) << cl) + (i & ((1 << cl) - 1));
        return k < nitems ? (int)k : nitems;
    }
    // Blocks of 2^cl entries times R heads, head-major inside a block; the
    // last block holds the remaining P entries.
    __device__ void decode(int k, int &e, int &rem) const {
        const int cr = p.ord_r << cl;
        const int full_items = p.ord_nblk * cr;
        if (k < full_items) {
            const int blk = div_by(k, cr, p.ord_m_cr), w = k - blk * cr;
            rem = w >> cl;
            e = (blk << cl) + (w & ((1 << cl) - 1));
        } else {
            const int w = k - full_items;
            rem = div_by(w, p.ord_p, p.ord_m_p);
            e = (p.ord_nblk << cl) + (w - rem * p.ord_p);
        }
    }
};

// Batch and head of head index rem of an entry of mask batch bm (with one
// shared mask, rem runs over all batches and heads).
__device__ inline void head_of(const AttnParams &p, int rem, int bm, int &b, int &h) {
    b = p.mask_b == 1 ? rem / p.H : bm;
    h = p.mask_b == 1 ? rem % p.H : rem;
}

// ceil(2^32 / d) for d >= 2 (host side; d <= 1 passes k through).
inline uint32_t div_magic(int64_t d) {
    return d <= 1 ? 0xffffffffu : (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d);
}

// Fills q's item-order fields and returns the grid size: head indices per
// entry (every batch and head with one shared mask, the heads of the entry's
// batch otherwise), chunks of up to 16 entries, at least four per queue.
inline unsigned item_order(AttnParams &q) {
    q.ord_r = q.mask_b == 1 ? q.B * q.H : q.H;
    const int64_t nitems = (int64_t)q.mask_b * q.nqt * q.ord_r;
    int cl = 4;
    while (cl > 0 && ((int64_t)1 << cl) * 4 * kQueues > nitems) --cl;
    q.ord_chunk_log2 = cl;
    const int nrows = q.mask_b * q.nqt;
    q.ord_nblk = nrows >> cl;
    q.ord_p = nrows - (q.ord_nblk << cl);
    q.ord_m_cr = div_magic((int64_t)q.ord_r << cl);
    q.ord_m_p = div_magic(q.ord_p);
    const int64_t nchunks = (nitems + (1 << cl) - 1) >> cl;
    return (unsigned)((kQueues * ((nchunks + kQueues - 1) / kQueues)) << cl);
}

}  // namespace bsm
