// C ABI of the block-sparse masked attention library: host-side argument
// checks, workspace layout and kernel launches.  No call allocates memory or
// synchronises; every check runs before anything is enqueued.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "bsm_internal.hpp"

namespace {

thread_local std::string g_last_error;

bsm_status fail(bsm_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bsm_status ok() {
    g_last_error.clear();
    return BSM_OK;
}

constexpr int32_t kMaxT = 1 << 22;

// Head dimensions the kernels are built for.
bool built_head_dim(int32_t D) { return D == 64 || D == 128 || D == 256; }
constexpr uint32_t kMaskFlagsAll = BSM_MASK_CAUSAL | BSM_MASK_DOCUMENT | BSM_MASK_WINDOW | BSM_MASK_SINKS |
                                   BSM_MASK_PREFIX | BSM_MASK_TABLE;

// The prefix bound kv < prefix the kernels use, at most KV_LEN: with the
// standard combination the widened causal bound (0 when the term is off: no
// PREFIX, or no causal term for it to widen); with a truth table the prefix
// term's own bound (0 without PREFIX).
int32_t effective_prefix(const bsm_mask_spec *spec) {
    const bool table = spec->flags & BSM_MASK_TABLE;
    if (!(spec->flags & BSM_MASK_PREFIX) || (!table && !(spec->flags & BSM_MASK_CAUSAL))) return 0;
    return spec->prefix_len < spec->seq_len ? spec->prefix_len : spec->seq_len;
}

// Shape of a mask: keys, queries, query offset, document positions, tiles,
// and the key blocks of the row lists (kb keys each).
struct MaskDims {
    int32_t kv_len, q_len, q_off, npos, nqt, nkt, kb, nkb;
};

MaskDims mask_dims(const bsm_mask_spec *spec) {
    MaskDims m;
    m.kv_len = spec->seq_len;
    m.q_len = spec->q_len > 0 ? spec->q_len : spec->seq_len;
    m.q_off = spec->q_offset;
    m.npos = m.kv_len > m.q_off + m.q_len ? m.kv_len : m.q_off + m.q_len;
    m.nqt = (m.q_len + bsm::kTile - 1) / bsm::kTile;
    m.nkt = (m.kv_len + bsm::kTile - 1) / bsm::kTile;
    m.kb = spec->kv_block == 64 ? 64 : bsm::kTile;
    m.nkb = (m.kv_len + m.kb - 1) / m.kb;
    return m;
}
constexpr uint32_t kModFlagsAll = BSM_MOD_ALIBI | BSM_MOD_SOFTCAP | BSM_MOD_BIAS;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool bad_len(int64_t T) { return T <= 0 || T > kMaxT; }

int32_t n_chunks(int32_t n) { return (n + 255) / 256; }

// Blocks of a work order (kOrderBlock rows of one mask batch each) over
// `tiles` rows per mask batch.
int64_t order_blocks(int32_t tiles, int32_t mask_b) {
    return (int64_t)mask_b * ((tiles + bsm::kOrderBlock - 1) / bsm::kOrderBlock);
}

int64_t order_ws_ints(const MaskDims &m, int32_t mask_b) {
    const int64_t r = order_blocks(m.nqt, mask_b), c = order_blocks(m.nkt, mask_b);
    return r > c ? r : c;
}

bsm_status check_spec(const bsm_mask_spec *spec) {
    if (!spec) return fail(BSM_E_INVALID, "mask spec is NULL");
    if (spec->flags & ~kMaskFlagsAll) return fail(BSM_E_INVALID, "unknown mask flag bits 0x%x", spec->flags);
    if (bad_len(spec->seq_len))
        return fail(BSM_E_INVALID, "seq_len %d must be in [1, %d]", spec->seq_len, kMaxT);
    if (spec->q_len < 0 || spec->q_len > kMaxT)
        return fail(BSM_E_INVALID, "q_len %d must be in [0, %d] (0: seq_len)", spec->q_len, kMaxT);
    if (spec->q_offset < 0 || (int64_t)spec->q_offset + (spec->q_len ? spec->q_len : spec->seq_len) > kMaxT)
        return fail(BSM_E_INVALID, "q_offset %d must be >= 0 with q_offset + Q_LEN <= %d", spec->q_offset, kMaxT);
    if (spec->mask_b < 1) return fail(BSM_E_INVALID, "mask_b %d must be >= 1", spec->mask_b);
    if ((spec->flags & BSM_MASK_DOCUMENT) && !spec->doc_ids)
        return fail(BSM_E_INVALID, "DOCUMENT mask without doc_ids");
    if ((spec->flags & BSM_MASK_WINDOW) && !spec->window)
        return fail(BSM_E_INVALID, "WINDOW mask without a window pointer");
    if ((spec->flags & BSM_MASK_SINKS) && spec->num_sinks < 0)
        return fail(BSM_E_INVALID, "num_sinks %d must be >= 0", spec->num_sinks);
    if ((spec->flags & BSM_MASK_PREFIX) && spec->prefix_len < 0)
        return fail(BSM_E_INVALID, "prefix_len %d must be >= 0", spec->prefix_len);
    if (spec->kv_block != 0 && spec->kv_block != 64 && spec->kv_block != bsm::kTile)
        return fail(BSM_E_INVALID, "kv_block %d must be 0, 64 or 128", spec->kv_block);
    return BSM_OK;
}

bsm_status check_block_mask(const bsm_block_mask *bm, bool need_transposed, const bsm_mask_spec *spec) {
    if (!bm) return fail(BSM_E_INVALID, "block mask is NULL");
    if ((spec->flags & BSM_MASK_DOCUMENT) && !bm->doc_range)
        return fail(BSM_E_INVALID, "DOCUMENT mask needs the block mask's doc_range array");
    if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices ||
        !bm->kv_order)
        return fail(BSM_E_INVALID, "block mask row arrays must be non-NULL");
    if (reinterpret_cast<uintptr_t>(bm->kv_order) % 16 != 0 ||
        (need_transposed && reinterpret_cast<uintptr_t>(bm->q_order) % 16 != 0))
        return fail(BSM_E_INVALID, "block mask work orders must be 16-byte aligned");
    if (need_transposed && (!bm->q_num_blocks || !bm->q_indices || !bm->full_q_num_blocks ||
                            !bm->full_q_indices || !bm->q_order))
        return fail(BSM_E_INVALID, "block mask column arrays must be non-NULL");
    return BSM_OK;
}

bsm_status check_tensor(const bsm_tensor *t, const char *name) {
    if (!t || !t->ptr) return fail(BSM_E_INVALID, "tensor %s is NULL", name);
    if (t->dtype != BSM_DTYPE_BF16 && t->dtype != BSM_DTYPE_F16)
        return fail(BSM_E_INVALID, "tensor %s has unknown dtype %d", name, t->dtype);
    if (reinterpret_cast<uintptr_t>(t->ptr) % 16 != 0)
        return fail(BSM_E_INVALID, "tensor %s must be 16-byte aligned", name);
    if (t->stride_b % 8 || t->stride_h % 8 || t->stride_t % 8)
        return fail(BSM_E_INVALID, "tensor %s strides must be multiples of 8 elements", name);
    if (t->stride_b < 0 || t->stride_h < 0 || t->stride_t < 0)
        return fail(BSM_E_INVALID, "tensor %s strides must be non-negative", name);
    return BSM_OK;
}

bsm_status check_mod(const bsm_score_mod *mod) {
    if (!mod) return BSM_OK;
    if (mod->flags & ~kModFlagsAll) return fail(BSM_E_INVALID, "unknown score-mod flag bits 0x%x", mod->flags);
    if ((mod->flags & BSM_MOD_ALIBI) && !mod->alibi_slopes)
        return fail(BSM_E_INVALID, "ALIBI without slopes");
    if ((mod->flags & BSM_MOD_SOFTCAP) && !(mod->softcap > 0.0f && std::isfinite(mod->softcap)))
        return fail(BSM_E_INVALID, "SOFTCAP needs a finite cap > 0");
    if (mod->alibi_slopes_grad && !(mod->flags & BSM_MOD_ALIBI))
        return fail(BSM_E_INVALID, "alibi_slopes_grad given without ALIBI");
    if (mod->flags & BSM_MOD_BIAS) {
        if (!mod->bias) return fail(BSM_E_INVALID, "BIAS without a table");
        if (mod->bias_radius < 0 || mod->bias_radius > BSM_BIAS_MAX_RADIUS)
            return fail(BSM_E_UNSUPPORTED, "bias radius %d must be in [0, %d]", mod->bias_radius,
                        BSM_BIAS_MAX_RADIUS);
        if (mod->flags & BSM_MOD_ALIBI)
            return fail(BSM_E_UNSUPPORTED, "ALIBI and BIAS together are not built (put the slope into the table)");
    } else if (mod->bias_grad) {
        return fail(BSM_E_INVALID, "bias_grad given without BIAS");
    }
    return BSM_OK;
}

bsm_status check_attn_common(int32_t B, int32_t H, int32_t T, int32_t D, const bsm_mask_spec *spec,
                             const bsm_score_mod *mod) {
    if (B < 1 || H < 1) return fail(BSM_E_INVALID, "B=%d and H=%d must be >= 1", B, H);
    if (bad_len(T)) return fail(BSM_E_INVALID, "T %d must be in [1, %d]", T, kMaxT);
    if (!built_head_dim(D)) return fail(BSM_E_UNSUPPORTED, "head dim %d: only 64, 128 and 256 are built", D);
    bsm_status st = check_spec(spec);
    if (st != BSM_OK) return st;
    if (spec->seq_len != T) return fail(BSM_E_INVALID, "mask seq_len %d != T %d", spec->seq_len, T);
    if (spec->mask_b != 1 && spec->mask_b != B)
        return fail(BSM_E_INVALID, "mask_b %d must be 1 or B=%d", spec->mask_b, B);
    const MaskDims m = mask_dims(spec);
    // the D = 256 backward runs two workgroups per key tile, and a chunked
    // dK/dV grid is rounded up to 128 workgroups
    if ((int64_t)B * H * (m.nqt > m.nkt ? m.nqt : m.nkt) > (INT32_MAX - 1024) / 2)
        return fail(BSM_E_INVALID, "grid too large");
    return check_mod(mod);
}

// Every tensor of a call has the type of the first (already checked).
bsm_status check_same_dtype(std::initializer_list<const bsm_tensor *> ts) {
    const int32_t dt = (*ts.begin())->dtype;
    for (const bsm_tensor *t : ts)
        if (t->dtype != dt) return fail(BSM_E_INVALID, "tensors of one call must share one dtype");
    return BSM_OK;
}

using AttnLauncher = hipError_t (*)(const bsm::AttnParams &, hipStream_t);

AttnLauncher fwd_launcher(int D, int32_t dtype) {
    if (dtype == BSM_DTYPE_F16)
        return D == 64 ? bsm::launch_attn_fwd_d64_f16 : D == 256 ? bsm::launch_attn_fwd_d256_f16
                                                               : bsm::launch_attn_fwd_d128_f16;
    return D == 64 ? bsm::launch_attn_fwd_d64_bf16 : D == 256 ? bsm::launch_attn_fwd_d256_bf16
                                                            : bsm::launch_attn_fwd_d128_bf16;
}

AttnLauncher bwd_launcher(int D, int32_t dtype) {
    if (dtype == BSM_DTYPE_F16)
        return D == 64 ? bsm::launch_attn_bwd_d64_f16 : D == 256 ? bsm::launch_attn_bwd_d256_f16
                                                               : bsm::launch_attn_bwd_d128_f16;
    return D == 64 ? bsm::launch_attn_bwd_d64_bf16 : D == 256 ? bsm::launch_attn_bwd_d256_bf16
                                                            : bsm::launch_attn_bwd_d128_bf16;
}

hipError_t launch_decode(const bsm::DecodeLaunch &d, float *part, hipStream_t stream) {
    return d.dtype == BSM_DTYPE_F16 ? bsm::launch_attn_decode_f16(d, part, stream)
                                    : bsm::launch_attn_decode_bf16(d, part, stream);
}

void fill_tensor(const bsm_tensor *t, const void *&ptr, int64_t &sb, int64_t &sh, int64_t &st) {
    ptr = t->ptr;
    sb = t->stride_b;
    sh = t->stride_h;
    st = t->stride_t;
}

void fill_bias(bsm::AttnParams &p, const bsm_score_mod *mod) {
    const bool on = mod && (mod->flags & BSM_MOD_BIAS);
    p.bias = on ? mod->bias : nullptr;
    p.bias_r = on ? mod->bias_radius : 0;
    p.dbias_part = nullptr;  // set by the backward only
    p.dbias = nullptr;
}

void fill_common(bsm::AttnParams &p, int32_t B, int32_t H, int32_t T, int32_t D,
                 const bsm_block_mask *bm, const bsm_mask_spec *spec, const bsm_score_mod *mod,
                 float scale) {
    p = bsm::AttnParams{};
    const MaskDims m = mask_dims(spec);
    p.B = B;
    p.H = H;
    p.T = T;
    p.nt = m.nkt;
    p.kb = m.kb;
    p.nkb = m.nkb;
    p.q_len = m.q_len;
    p.nqt = m.nqt;
    p.q_off = m.q_off;
    p.npos = m.npos;
    p.table = spec->table;
    p.mask_b = spec->mask_b;
    p.mask_flags = spec->flags;
    p.sinks = spec->num_sinks;
    p.prefix = effective_prefix(spec);
    p.doc_ids = spec->doc_ids;
    p.window = spec->window;
    p.mod_flags = mod ? mod->flags : 0u;
    p.alibi_slopes = mod ? mod->alibi_slopes : nullptr;
    fill_bias(p, mod);
    p.dslopes = nullptr;  // set by the backward only
    p.dslope_part = nullptr;
    p.softcap = (mod && (mod->flags & BSM_MOD_SOFTCAP)) ? mod->softcap : 0.0f;
    p.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
    p.kv_num = bm->kv_num_blocks;
    p.kv_idx = bm->kv_indices;
    p.full_kv_num = bm->full_kv_num_blocks;
    p.full_kv_idx = bm->full_kv_indices;
    p.q_num = bm->q_num_blocks;
    p.q_idx = bm->q_indices;
    p.full_q_num = bm->full_q_num_blocks;
    p.full_q_idx = bm->full_q_indices;
    p.doc_range = (spec->flags & BSM_MASK_DOCUMENT) ? bm->doc_range : nullptr;
    p.kv_order = bm->kv_order;
    p.q_order = bm->q_order;
}

bsm_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(BSM_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

size_t decode_part_bytes(int32_t B, int32_t H, int32_t capacity, int32_t D) {
    return align256((size_t)B * H * bsm::decode_slots(capacity) * (D + 2) * sizeof(float));
}

// Host checks and parameter block of a decoding step (both decode entry
// points).  The cache holds `capacity` positions; kv_len is a device value.
bsm_status prepare_decode(int32_t B, int32_t H, int32_t capacity, int32_t D, const int32_t *kv_len,
                          int32_t kv_len_stride, const bsm_tensor *q, const bsm_tensor *k, const bsm_tensor *v,
                          const bsm_mask_spec *spec, const bsm_block_mask *bm, const bsm_score_mod *mod,
                          float scale, const bsm_tensor *out, float *lse, bsm::DecodeLaunch &d) {
    if (B < 1 || H < 1) return fail(BSM_E_INVALID, "B=%d and H=%d must be >= 1", B, H);
    if (capacity < 1 || capacity > kMaxT)
        return fail(BSM_E_INVALID, "capacity %d must be in [1, %d]", capacity, kMaxT);
    if (!built_head_dim(D)) return fail(BSM_E_UNSUPPORTED, "head dim %d: only 64, 128 and 256 are built", D);
    if (!spec) return fail(BSM_E_INVALID, "mask spec is NULL");
    if (spec->seq_len != capacity)
        return fail(BSM_E_INVALID, "mask seq_len %d != cache capacity %d", spec->seq_len, capacity);
    if ((spec->q_len != 0 && spec->q_len != capacity) || spec->q_offset != 0)
        return fail(BSM_E_INVALID, "a decoding step's mask is square over the cache (q_len 0, q_offset 0)");
    if (bm) {  // a block mask is built for the whole capacity, square
        bsm_status st = check_spec(spec);
        if (st != BSM_OK) return st;
        if (capacity % bsm::kTile != 0)
            return fail(BSM_E_INVALID, "with a block mask the capacity %d must be a multiple of 128", capacity);
        if (spec->kv_block == 64)
            return fail(BSM_E_UNSUPPORTED, "the decoding step reads block masks of 128-key blocks only");
        if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices)
            return fail(BSM_E_INVALID, "block mask row arrays must be non-NULL");
    } else {
        if (spec->flags & ~kMaskFlagsAll) return fail(BSM_E_INVALID, "unknown mask flag bits 0x%x", spec->flags);
        if (spec->mask_b < 1) return fail(BSM_E_INVALID, "mask_b %d must be >= 1", spec->mask_b);
        if ((spec->flags & BSM_MASK_DOCUMENT) && !spec->doc_ids)
            return fail(BSM_E_INVALID, "DOCUMENT mask without doc_ids");
        if ((spec->flags & BSM_MASK_WINDOW) && !spec->window)
            return fail(BSM_E_INVALID, "WINDOW mask without a window pointer");
        if ((spec->flags & BSM_MASK_SINKS) && spec->num_sinks < 0)
            return fail(BSM_E_INVALID, "num_sinks %d must be >= 0", spec->num_sinks);
        if ((spec->flags & BSM_MASK_PREFIX) && spec->prefix_len < 0)
            return fail(BSM_E_INVALID, "prefix_len %d must be >= 0", spec->prefix_len);
    }
    if (spec->mask_b != 1 && spec->mask_b != B)
        return fail(BSM_E_INVALID, "mask_b %d must be 1 or B=%d", spec->mask_b, B);
    if (!kv_len) return fail(BSM_E_INVALID, "kv_len is NULL");
    if (kv_len_stride != 0 && kv_len_stride != 1)
        return fail(BSM_E_INVALID, "kv_len_stride %d must be 0 or 1", kv_len_stride);
    bsm_status st = check_mod(mod);
    if (st != BSM_OK) return st;
    if (mod && mod->alibi_slopes_grad) return fail(BSM_E_INVALID, "alibi_slopes_grad is a backward output");
    if (mod && mod->bias_grad) return fail(BSM_E_INVALID, "bias_grad is a backward output");
    if ((st = check_tensor(q, "q")) != BSM_OK) return st;
    if ((st = check_tensor(k, "k")) != BSM_OK) return st;
    if ((st = check_tensor(v, "v")) != BSM_OK) return st;
    if ((st = check_tensor(out, "out")) != BSM_OK) return st;
    if ((st = check_same_dtype({q, k, v, out})) != BSM_OK) return st;
    if (!lse) return fail(BSM_E_INVALID, "lse is NULL");
    if (!std::isfinite(scale)) return fail(BSM_E_INVALID, "scale must be finite");
    d.dtype = q->dtype;
    bsm::AttnParams &p = d.a;
    p = bsm::AttnParams{};
    p.B = B;
    p.H = H;
    p.T = capacity;
    p.nt = (capacity + bsm::kTile - 1) / bsm::kTile;
    p.kb = bsm::kTile;
    p.nkb = p.nt;
    p.q_len = capacity;
    p.nqt = p.nt;
    p.npos = capacity;
    p.table = spec->table;
    p.mask_b = spec->mask_b;
    p.mask_flags = spec->flags;
    p.sinks = spec->num_sinks;
    p.prefix = effective_prefix(spec);
    p.doc_ids = spec->doc_ids;
    p.window = spec->window;
    p.mod_flags = mod ? mod->flags : 0u;
    p.alibi_slopes = mod ? mod->alibi_slopes : nullptr;
    fill_bias(p, mod);
    p.softcap = (mod && (mod->flags & BSM_MOD_SOFTCAP)) ? mod->softcap : 0.0f;
    p.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
    if (bm) {
        p.kv_num = bm->kv_num_blocks;
        p.kv_idx = bm->kv_indices;
        p.full_kv_num = bm->full_kv_num_blocks;
        p.full_kv_idx = bm->full_kv_indices;
    }
    fill_tensor(q, p.q, p.q_sb, p.q_sh, p.q_st);
    fill_tensor(k, p.k, p.k_sb, p.k_sh, p.k_st);
    fill_tensor(v, p.v, p.v_sb, p.v_sh, p.v_st);
    const void *optr;
    fill_tensor(out, optr, p.o_sb, p.o_sh, p.o_st);
    p.o = const_cast<void *>(optr);
    p.lse = lse;
    d.D = D;
    d.kv_len = kv_len;
    d.kv_len_stride = kv_len_stride;
    d.block_table = nullptr;  // contiguous cache (the paged entry point sets these)
    d.table_stride = 0;
    d.page_size = 0;
    d.num_pages = 0;
    return BSM_OK;
}

// ------------------------------------------------------------ static scratch
// Device memory of the allocation-free decoding entry point: one array per
// GPU, in the library's code object, held until the process ends.  Host code
// never uses the array's name as an address: the address on each device comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Address of this device's scratch array (the current device, which must be
// the stream's), looked up on the first call on the device.
bsm_status scratch_address(void *stream, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BSM_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(BSM_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return fail(BSM_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev) return fail(BSM_E_INVALID, "stream is on device %d, current device is %d", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(BSM_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BSM_OK;
}

}  // namespace

extern "C" {

size_t bsm_block_mask_workspace_bytes(const bsm_mask_spec *spec) {
    if (check_spec(spec) != BSM_OK) return 0;
    const MaskDims m = mask_dims(spec);
    return align256((size_t)spec->mask_b * n_chunks(m.npos) * sizeof(int32_t)) +
           align256((size_t)spec->mask_b * m.nqt * m.nkb) +
           2 * align256((size_t)order_ws_ints(m, spec->mask_b) * sizeof(int32_t));
}

bsm_status bsm_build_block_mask(const bsm_mask_spec *spec, const bsm_block_mask *out,
                                void *workspace, size_t workspace_bytes, void *stream) {
    bsm_status st = check_spec(spec);
    if (st != BSM_OK) return st;
    st = check_block_mask(out, true, spec);
    if (st != BSM_OK) return st;
    const MaskDims m = mask_dims(spec);
    if ((int64_t)spec->mask_b * (m.nqt > m.nkt ? m.nqt : m.nkt) > INT32_MAX ||
        (int64_t)spec->mask_b * m.npos > INT32_MAX)
        return fail(BSM_E_INVALID, "mask_b x tiles exceeds the int32 work-order range");
    const size_t need = bsm_block_mask_workspace_bytes(spec);
    if (!workspace || workspace_bytes < need)
        return fail(BSM_E_WORKSPACE, "block-mask workspace needs %zu bytes, got %zu%s", need,
                    workspace_bytes, workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(BSM_E_WORKSPACE, "workspace must be 256-byte aligned");
    bsm::MaskBuildParams p{};
    p.flags = spec->flags;
    p.T = m.kv_len;
    p.q_len = m.q_len;
    p.q_off = m.q_off;
    p.npos = m.npos;
    p.nqt = m.nqt;
    p.nkt = m.nkt;
    p.kb = m.kb;
    p.nkb = m.nkb;
    p.mask_b = spec->mask_b;
    p.nchunks = n_chunks(m.npos);
    p.sinks = spec->num_sinks;
    p.prefix = effective_prefix(spec);
    p.table = spec->table;
    p.doc_ids = spec->doc_ids;
    p.window = spec->window;
    p.out = *out;
    char *ws = static_cast<char *>(workspace);
    p.nonmono = reinterpret_cast<int32_t *>(ws);
    const size_t off_cls = align256((size_t)p.mask_b * p.nchunks * sizeof(int32_t));
    p.cls = reinterpret_cast<uint8_t *>(ws + off_cls);
    const size_t off_order = off_cls + align256((size_t)p.mask_b * p.nqt * p.nkb);
    p.order_ws = reinterpret_cast<int32_t *>(ws + off_order);
    p.order_ws_stride = (int32_t)(align256((size_t)order_ws_ints(m, spec->mask_b) * sizeof(int32_t)) / sizeof(int32_t));
    return hip_status(bsm::launch_build_block_mask(p, static_cast<hipStream_t>(stream)),
                      "bsm_build_block_mask launch");
}

bsm_status bsm_flex_attention_fwd(int32_t B, int32_t H, int32_t T, int32_t D, const bsm_tensor *q,
                                  const bsm_tensor *k, const bsm_tensor *v, const bsm_block_mask *bm,
                                  const bsm_mask_spec *spec, const bsm_score_mod *mod, float scale,
                                  const bsm_tensor *out, float *lse, void *stream) {
    bsm_status st = check_attn_common(B, H, T, D, spec, mod);
    if (st != BSM_OK) return st;
    if ((st = check_block_mask(bm, false, spec)) != BSM_OK) return st;
    if ((st = check_tensor(q, "q")) != BSM_OK) return st;
    if ((st = check_tensor(k, "k")) != BSM_OK) return st;
    if ((st = check_tensor(v, "v")) != BSM_OK) return st;
    if ((st = check_tensor(out, "out")) != BSM_OK) return st;
    if ((st = check_same_dtype({q, k, v, out})) != BSM_OK) return st;
    if (!lse) return fail(BSM_E_INVALID, "lse is NULL");
    if (!std::isfinite(scale)) return fail(BSM_E_INVALID, "scale must be finite");
    bsm::AttnParams p;
    fill_common(p, B, H, T, D, bm, spec, mod, scale);
    fill_tensor(q, p.q, p.q_sb, p.q_sh, p.q_st);
    fill_tensor(k, p.k, p.k_sb, p.k_sh, p.k_st);
    fill_tensor(v, p.v, p.v_sb, p.v_sh, p.v_st);
    const void *optr;
    fill_tensor(out, optr, p.o_sb, p.o_sh, p.o_st);
    p.o = const_cast<void *>(optr);
    p.lse = lse;
    return hip_status(fwd_launcher(D, q->dtype)(p, static_cast<hipStream_t>(stream)),
                      "bsm_flex_attention_fwd launch");
}

size_t bsm_bwd_workspace_bytes(int32_t B, int32_t H, int32_t Q, int32_t D) {
    if (B < 1 || H < 1 || bad_len(Q) || !built_head_dim(D)) return 0;
    return 2 * align256((size_t)B * H * Q * sizeof(float)) +
           align256((size_t)B * H * ((Q + bsm::kTile - 1) / bsm::kTile) * sizeof(float));
}

static size_t bias_part_bytes(int32_t B, int32_t H, int32_t Q, const bsm_score_mod *mod) {
    if (!mod || !(mod->flags & BSM_MOD_BIAS)) return 0;
    return align256((size_t)B * H * ((Q + bsm::kTile - 1) / bsm::kTile) * (2 * (size_t)mod->bias_radius + 1) *
                    sizeof(float));
}

size_t bsm_bwd_workspace_bytes_mod(int32_t B, int32_t H, int32_t Q, int32_t D, const bsm_score_mod *mod) {
    const size_t base = bsm_bwd_workspace_bytes(B, H, Q, D);
    if (base == 0 || check_mod(mod) != BSM_OK) return 0;
    return base + bias_part_bytes(B, H, Q, mod);
}

bsm_status bsm_flex_attention_bwd(int32_t B, int32_t H, int32_t T, int32_t D, const bsm_tensor *q,
                                  const bsm_tensor *k, const bsm_tensor *v, const bsm_tensor *out,
                                  const float *lse, const bsm_tensor *dout, const bsm_block_mask *bm,
                                  const bsm_mask_spec *spec, const bsm_score_mod *mod, float scale,
                                  const bsm_tensor *dq, const bsm_tensor *dk, const bsm_tensor *dv,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    bsm_status st = check_attn_common(B, H, T, D, spec, mod);
    if (st != BSM_OK) return st;
    if (D == 256 && mod && (mod->flags & BSM_MOD_BIAS))
        return fail(BSM_E_UNSUPPORTED, "a bias table's backward is built for head dims 64 and 128");
    if ((st = check_block_mask(bm, true, spec)) != BSM_OK) return st;
    if ((st = check_tensor(q, "q")) != BSM_OK) return st;
    if ((st = check_tensor(k, "k")) != BSM_OK) return st;
    if ((st = check_tensor(v, "v")) != BSM_OK) return st;
    if ((st = check_tensor(out, "out")) != BSM_OK) return st;
    if ((st = check_tensor(dout, "dout")) != BSM_OK) return st;
    if ((st = check_tensor(dq, "dq")) != BSM_OK) return st;
    if ((st = check_tensor(dk, "dk")) != BSM_OK) return st;
    if ((st = check_tensor(dv, "dv")) != BSM_OK) return st;
    if ((st = check_same_dtype({q, k, v, out, dout, dq, dk, dv})) != BSM_OK) return st;
    if (!lse) return fail(BSM_E_INVALID, "lse is NULL");
    if (!std::isfinite(scale)) return fail(BSM_E_INVALID, "scale must be finite");
    const int32_t Q = mask_dims(spec).q_len;
    const size_t need = bsm_bwd_workspace_bytes_mod(B, H, Q, D, mod);
    if (!workspace || workspace_bytes < need)
        return fail(BSM_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu%s", need,
                    workspace_bytes, workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(BSM_E_WORKSPACE, "workspace must be 256-byte aligned");
    bsm::AttnParams p;
    fill_common(p, B, H, T, D, bm, spec, mod, scale);
    fill_tensor(q, p.q, p.q_sb, p.q_sh, p.q_st);
    fill_tensor(k, p.k, p.k_sb, p.k_sh, p.k_st);
    fill_tensor(v, p.v, p.v_sb, p.v_sh, p.v_st);
    const void *ptr;
    fill_tensor(out, ptr, p.o_sb, p.o_sh, p.o_st);
    p.o = const_cast<void *>(ptr);
    fill_tensor(dout, p.dout, p.do_sb, p.do_sh, p.do_st);
    fill_tensor(dq, ptr, p.dq_sb, p.dq_sh, p.dq_st);
    p.dq = const_cast<void *>(ptr);
    fill_tensor(dk, ptr, p.dk_sb, p.dk_sh, p.dk_st);
    p.dk = const_cast<void *>(ptr);
    fill_tensor(dv, ptr, p.dv_sb, p.dv_sh, p.dv_st);
    p.dv = const_cast<void *>(ptr);
    p.lse = const_cast<float *>(lse);
    p.delta = static_cast<float *>(workspace);
    p.lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + align256((size_t)B * H * Q * sizeof(float)));
    p.dslope_part = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                              2 * align256((size_t)B * H * Q * sizeof(float)));
    p.dslopes = (mod && (mod->flags & BSM_MOD_ALIBI)) ? mod->alibi_slopes_grad : nullptr;
    if (p.bias) {
        p.dbias_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + bsm_bwd_workspace_bytes(B, H, Q, D));
        p.dbias = mod->bias_grad;
    }
    return hip_status(bwd_launcher(D, q->dtype)(p, static_cast<hipStream_t>(stream)),
                      "bsm_flex_attention_bwd launch");
}

size_t bsm_decode_workspace_bytes(int32_t B, int32_t H, int32_t capacity, int32_t D) {
    if (B < 1 || H < 1 || capacity < 1 || capacity > kMaxT || !built_head_dim(D)) return 0;
    return decode_part_bytes(B, H, capacity, D);
}

bsm_status bsm_flex_attention_decode(int32_t B, int32_t H, int32_t capacity, int32_t D, const int32_t *kv_len,
                                     int32_t kv_len_stride, const bsm_tensor *q, const bsm_tensor *k,
                                     const bsm_tensor *v, const bsm_mask_spec *spec, const bsm_block_mask *bm,
                                     const bsm_score_mod *mod, float scale, const bsm_tensor *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    bsm::DecodeLaunch d;
    bsm_status st = prepare_decode(B, H, capacity, D, kv_len, kv_len_stride, q, k, v, spec, bm, mod, scale, out,
                                   lse, d);
    if (st != BSM_OK) return st;
    const size_t need = decode_part_bytes(B, H, capacity, D);
    if (!workspace || workspace_bytes < need)
        return fail(BSM_E_WORKSPACE, "decode workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(BSM_E_WORKSPACE, "workspace must be 256-byte aligned");
    return hip_status(launch_decode(d, static_cast<float *>(workspace), static_cast<hipStream_t>(stream)),
                      "bsm_flex_attention_decode launch");
}

bsm_status bsm_flex_attention_decode_paged(int32_t B, int32_t H, int32_t D, int32_t page_size, int32_t num_pages,
                                           const int32_t *block_table, int32_t table_stride, const int32_t *kv_len,
                                           int32_t kv_len_stride, const bsm_tensor *q, const bsm_tensor *k_pages,
                                           const bsm_tensor *v_pages, const bsm_mask_spec *spec,
                                           const bsm_block_mask *bm, const bsm_score_mod *mod, float scale,
                                           const bsm_tensor *out, float *lse, void *workspace, size_t workspace_bytes,
                                           void *stream) {
    if (page_size < 64 || page_size % 64 != 0)
        return fail(BSM_E_INVALID, "page_size %d must be a positive multiple of 64", page_size);
    if (num_pages < 1) return fail(BSM_E_INVALID, "num_pages %d must be >= 1", num_pages);
    if (!block_table) return fail(BSM_E_INVALID, "block_table is NULL");
    if (table_stride < 1 || (int64_t)table_stride * page_size > kMaxT)
        return fail(BSM_E_INVALID, "table_stride %d x page_size %d must give a capacity in [1, %d]", table_stride,
                    page_size, kMaxT);
    const int32_t capacity = table_stride * page_size;
    bsm::DecodeLaunch d;
    bsm_status st = prepare_decode(B, H, capacity, D, kv_len, kv_len_stride, q, k_pages, v_pages, spec, bm, mod,
                                   scale, out, lse, d);
    if (st != BSM_OK) return st;
    const size_t need = decode_part_bytes(B, H, capacity, D);
    if (!workspace || workspace_bytes < need)
        return fail(BSM_E_WORKSPACE, "decode workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(BSM_E_WORKSPACE, "workspace must be 256-byte aligned");
    d.block_table = block_table;
    d.table_stride = table_stride;
    d.page_size = page_size;
    d.num_pages = num_pages;
    return hip_status(launch_decode(d, static_cast<float *>(workspace), static_cast<hipStream_t>(stream)),
                      "bsm_flex_attention_decode_paged launch");
}

bsm_status bsm_gather_kv_pages(int32_t B, int32_t H, int32_t D, int32_t page_size, int32_t num_pages,
                               const int32_t *block_table, int32_t table_stride, int32_t n_keys,
                               const bsm_tensor *k_pages, const bsm_tensor *v_pages, const bsm_tensor *k_out,
                               const bsm_tensor *v_out, void *stream) {
    if (B < 1 || H < 1) return fail(BSM_E_INVALID, "B=%d and H=%d must be >= 1", B, H);
    if ((int64_t)B * H > INT32_MAX) return fail(BSM_E_INVALID, "grid too large");
    if (!built_head_dim(D)) return fail(BSM_E_UNSUPPORTED, "head dim %d: only 64, 128 and 256 are built", D);
    if (page_size < 64 || page_size % 64 != 0)
        return fail(BSM_E_INVALID, "page_size %d must be a positive multiple of 64", page_size);
    if (num_pages < 1) return fail(BSM_E_INVALID, "num_pages %d must be >= 1", num_pages);
    if (!block_table) return fail(BSM_E_INVALID, "block_table is NULL");
    if (table_stride < 1 || (int64_t)table_stride * page_size > kMaxT)
        return fail(BSM_E_INVALID, "table_stride %d x page_size %d must give a capacity in [1, %d]", table_stride,
                    page_size, kMaxT);
    if (n_keys < 1 || n_keys > table_stride * page_size)
        return fail(BSM_E_INVALID, "n_keys %d must be in [1, %d]", n_keys, table_stride * page_size);
    bsm_status st;
    if ((st = check_tensor(k_pages, "k_pages")) != BSM_OK) return st;
    if ((st = check_tensor(v_pages, "v_pages")) != BSM_OK) return st;
    if ((st = check_tensor(k_out, "k_out")) != BSM_OK) return st;
    if ((st = check_tensor(v_out, "v_out")) != BSM_OK) return st;
    if ((st = check_same_dtype({k_pages, v_pages, k_out, v_out})) != BSM_OK) return st;
    constexpr int64_t kElem = 2;  // bf16 and fp16
    bsm::GatherLaunch g;
    g.B = B;
    g.H = H;
    g.row_bytes = D * (int32_t)kElem;
    g.page_size = page_size;
    g.num_pages = num_pages;
    g.table_stride = table_stride;
    g.n_keys = n_keys;
    g.table = block_table;
    g.k_src = static_cast<const char *>(k_pages->ptr);
    g.v_src = static_cast<const char *>(v_pages->ptr);
    g.ks_b = k_pages->stride_b * kElem, g.ks_h = k_pages->stride_h * kElem, g.ks_t = k_pages->stride_t * kElem;
    g.vs_b = v_pages->stride_b * kElem, g.vs_h = v_pages->stride_h * kElem, g.vs_t = v_pages->stride_t * kElem;
    g.k_dst = static_cast<char *>(const_cast<void *>(k_out->ptr));
    g.v_dst = static_cast<char *>(const_cast<void *>(v_out->ptr));
    g.kd_b = k_out->stride_b * kElem, g.kd_h = k_out->stride_h * kElem, g.kd_t = k_out->stride_t * kElem;
    g.vd_b = v_out->stride_b * kElem, g.vd_h = v_out->stride_h * kElem, g.vd_t = v_out->stride_t * kElem;
    return hip_status(bsm::launch_gather_pages(g, static_cast<hipStream_t>(stream)), "bsm_gather_kv_pages launch");
}

size_t bsm_decode_static_max_bytes(void) { return kScratchBytes; }

bsm_status bsm_flex_attention_decode_static(int32_t B, int32_t H, int32_t capacity, int32_t D,
                                            const int32_t *kv_len, int32_t kv_len_stride, const bsm_tensor *q,
                                            const bsm_tensor *k, const bsm_tensor *v, const bsm_mask_spec *spec,
                                            const bsm_block_mask *bm, const bsm_score_mod *mod, float scale,
                                            const bsm_tensor *out, float *lse, void *stream) {
    bsm::DecodeLaunch d;
    bsm_status st = prepare_decode(B, H, capacity, D, kv_len, kv_len_stride, q, k, v, spec, bm, mod, scale, out,
                                   lse, d);
    if (st != BSM_OK) return st;
    const size_t need = decode_part_bytes(B, H, capacity, D);
    if (need > kScratchBytes)
        return fail(BSM_E_WORKSPACE,
                    "decode partials need %zu bytes, beyond the %zu-byte static scratch (B * H * ceil(capacity / "
                    "1024) * (D + 2) * 4 bytes); use bsm_flex_attention_decode with a workspace",
                    need, kScratchBytes);
    void *ptr = nullptr;
    if ((st = scratch_address(stream, &ptr)) != BSM_OK) return st;
    // Every slot of the partials is written before the combine reads it, so
    // nothing in the scratch needs clearing.
    return hip_status(launch_decode(d, static_cast<float *>(ptr), static_cast<hipStream_t>(stream)),
                      "bsm_flex_attention_decode_static launch");
}

const char *bsm_last_error(void) { return g_last_error.c_str(); }

const char *bsm_version(void) { return "bsm 0.1.0 gfx950"; }

}  // extern "C"
