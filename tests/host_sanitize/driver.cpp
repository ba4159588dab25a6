// Host-side driver of the C ABI shim (bsm_api.cpp) for the sanitizer build:
// every entry point with rejected and accepted arguments, the launchers
// replaced by stand-ins that record what the shim built.  Checks that each
// rejection returns its status with a message, that accepted calls reach one
// launcher, and that the workspace parts the shim carves out lie inside the
// caller's workspace without overlapping.  No device memory is touched: the
// shim only checks and forwards pointers, so host buffers stand in for them.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "stub_launchers.hpp"

static int g_failures = 0;

#define CHECK(cond)                                                                          \
    do {                                                                                     \
        if (!(cond)) {                                                                       \
            std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__,     \
                         __LINE__, #cond, bsm_last_error());                                 \
            ++g_failures;                                                                    \
        }                                                                                    \
    } while (0)

// A rejected call: the status and a non-empty message, no launch.
#define REJECT(call, code)                                          \
    do {                                                            \
        const int before = stub::calls;                             \
        const bsm_status st_ = (call);                              \
        CHECK(st_ == (code));                                       \
        CHECK(std::strlen(bsm_last_error()) > 0);                   \
        CHECK(stub::calls == before);                               \
    } while (0)

// An accepted call: BSM_OK and exactly one more launch.
#define ACCEPT(call)                                                \
    do {                                                            \
        const int before = stub::calls;                             \
        const bsm_status st_ = (call);                              \
        CHECK(st_ == BSM_OK);                                       \
        CHECK(stub::calls >= before + 1);                           \
    } while (0)

// Host memory standing in for device buffers (never dereferenced by the shim).
static std::vector<char> g_arena(64 << 20);

static char *arena(size_t offset) {
    return reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(g_arena.data()) + 4095) & ~uintptr_t(4095)) + offset;
}

static bool inside(const void *p, size_t bytes, const void *lo, size_t span) {
    const char *a = static_cast<const char *>(p), *b = static_cast<const char *>(lo);
    return a >= b && a + bytes <= b + span;
}

static bsm_mask_spec spec_of(int32_t T, uint32_t flags = BSM_MASK_CAUSAL) {
    bsm_mask_spec s;
    std::memset(&s, 0, sizeof(s));
    s.flags = flags;
    s.seq_len = T;
    s.mask_b = 1;
    return s;
}

static bsm_block_mask block_mask_of(char *base) {
    bsm_block_mask bm;
    int32_t **f = reinterpret_cast<int32_t **>(&bm);
    for (size_t i = 0; i < sizeof(bm) / sizeof(int32_t *); ++i) f[i] = reinterpret_cast<int32_t *>(base + 4096 * i);
    return bm;
}

static bsm_tensor tensor_of(char *p, int32_t H, int32_t T, int32_t D, int32_t dtype = BSM_DTYPE_BF16) {
    bsm_tensor t;
    t.ptr = p;
    t.stride_t = D;
    t.stride_h = (int64_t)T * D;
    t.stride_b = (int64_t)H * T * D;
    t.dtype = dtype;
    return t;
}

static void block_mask_build() {
    bsm_mask_spec s = spec_of(65536, BSM_MASK_CAUSAL | BSM_MASK_DOCUMENT | BSM_MASK_WINDOW);
    int32_t *docs = reinterpret_cast<int32_t *>(arena(1 << 20));
    int32_t *win = reinterpret_cast<int32_t *>(arena(2 << 20));
    s.doc_ids = docs;
    s.window = win;
    const size_t need = bsm_block_mask_workspace_bytes(&s);
    CHECK(need > 0);
    CHECK(bsm_block_mask_workspace_bytes(nullptr) == 0);
    bsm_block_mask bm = block_mask_of(arena(4 << 20));
    char *ws = arena(8 << 20);
    REJECT(bsm_build_block_mask(nullptr, &bm, ws, need, nullptr), BSM_E_INVALID);
    REJECT(bsm_build_block_mask(&s, nullptr, ws, need, nullptr), BSM_E_INVALID);
    REJECT(bsm_build_block_mask(&s, &bm, ws, need - 1, nullptr), BSM_E_WORKSPACE);
    REJECT(bsm_build_block_mask(&s, &bm, ws + 16, need, nullptr), BSM_E_WORKSPACE);
    REJECT(bsm_build_block_mask(&s, &bm, nullptr, need, nullptr), BSM_E_WORKSPACE);
    bsm_mask_spec bad = s;
    bad.doc_ids = nullptr;
    REJECT(bsm_build_block_mask(&bad, &bm, ws, need, nullptr), BSM_E_INVALID);
    bad = s;
    bad.kv_block = 32;
    REJECT(bsm_build_block_mask(&bad, &bm, ws, need, nullptr), BSM_E_INVALID);
    bad = s;
    bad.flags |= 1u << 10;
    REJECT(bsm_build_block_mask(&bad, &bm, ws, need, nullptr), BSM_E_INVALID);
    ACCEPT(bsm_build_block_mask(&s, &bm, ws, need, nullptr));
    // the class matrix, monotonicity flags and order scratch lie inside the workspace
    const bsm::MaskBuildParams &p = stub::last_build;
    CHECK(inside(p.cls, (size_t)p.mask_b * p.nqt * p.nkb, ws, need));
    CHECK(inside(p.nonmono, (size_t)p.mask_b * p.nchunks * 4, ws, need));
    CHECK(inside(p.order_ws, (size_t)2 * p.order_ws_stride * 4, ws, need));
    // rectangular, 64-key blocks and composed masks
    bsm_mask_spec r = spec_of(1000, BSM_MASK_CAUSAL | BSM_MASK_TABLE);
    r.q_len = 300;
    r.q_offset = 700;
    r.kv_block = 64;
    r.table = 0xAAAAAAAAu;
    const size_t need_r = bsm_block_mask_workspace_bytes(&r);
    CHECK(need_r > 0);
    ACCEPT(bsm_build_block_mask(&r, &bm, ws, need_r, nullptr));
    CHECK(stub::last_build.nqt == 3 && stub::last_build.nkb == 16 && stub::last_build.q_off == 700);
}

static void attention() {
    const int32_t B = 2, H = 3, T = 1000, D = 128;
    bsm_mask_spec s = spec_of(T);
    bsm_block_mask bm = block_mask_of(arena(4 << 20));
    bsm_tensor q = tensor_of(arena(16 << 20), H, T, D), k = q, v = q, o = q;
    float *lse = reinterpret_cast<float *>(arena(12 << 20));
    // forward
    REJECT(bsm_flex_attention_fwd(B, H, T, 96, &q, &k, &v, &bm, &s, nullptr, 0.0f, &o, lse, nullptr),
           BSM_E_UNSUPPORTED);
    REJECT(bsm_flex_attention_fwd(B, H, T + 1, D, &q, &k, &v, &bm, &s, nullptr, 0.0f, &o, lse, nullptr),
           BSM_E_INVALID);
    bsm_tensor bad = q;
    bad.stride_t = 60;
    REJECT(bsm_flex_attention_fwd(B, H, T, D, &q, &bad, &v, &bm, &s, nullptr, 0.0f, &o, lse, nullptr), BSM_E_INVALID);
    bad = q;
    bad.dtype = BSM_DTYPE_F16;
    REJECT(bsm_flex_attention_fwd(B, H, T, D, &q, &bad, &v, &bm, &s, nullptr, 0.0f, &o, lse, nullptr), BSM_E_INVALID);
    REJECT(bsm_flex_attention_fwd(B, H, T, D, &q, &k, &v, &bm, &s, nullptr, 0.0f, &o, nullptr, nullptr),
           BSM_E_INVALID);
    ACCEPT(bsm_flex_attention_fwd(B, H, T, D, &q, &k, &v, &bm, &s, nullptr, 0.0f, &o, lse, nullptr));
    CHECK(stub::last_attn.nt == 8 && stub::last_attn.q_len == T && stub::last_attn.bias == nullptr);
    // score modifications
    float *table = reinterpret_cast<float *>(arena(20 << 20));
    bsm_score_mod mod;
    std::memset(&mod, 0, sizeof(mod));
    mod.flags = BSM_MOD_BIAS | BSM_MOD_SOFTCAP;
    mod.softcap = 30.0f;
    mod.bias = table;
    mod.bias_radius = 1024;
    ACCEPT(bsm_flex_attention_fwd(B, H, T, D, &q, &k, &v, &bm, &s, &mod, 0.0f, &o, lse, nullptr));
    CHECK(stub::last_attn.bias == table && stub::last_attn.bias_r == 1024);
    bsm_score_mod m2 = mod;
    m2.bias_radius = 1025;
    REJECT(bsm_flex_attention_fwd(B, H, T, D, &q, &k, &v, &bm, &s, &m2, 0.0f, &o, lse, nullptr), BSM_E_UNSUPPORTED);
    m2 = mod;
    m2.flags |= BSM_MOD_ALIBI;
    m2.alibi_slopes = table;
    REJECT(bsm_flex_attention_fwd(B, H, T, D, &q, &k, &v, &bm, &s, &m2, 0.0f, &o, lse, nullptr), BSM_E_UNSUPPORTED);
    // backward: the workspace parts of Delta, lse log2 e, slope and bias partials
    const size_t base = bsm_bwd_workspace_bytes(B, H, T, D);
    const size_t need = bsm_bwd_workspace_bytes_mod(B, H, T, D, &mod);
    CHECK(base > 0 && need > base);
    char *ws = arena(40 << 20);
    mod.bias_grad = reinterpret_cast<float *>(arena(24 << 20));
    REJECT(bsm_flex_attention_bwd(B, H, T, D, &q, &k, &v, &o, lse, &q, &bm, &s, &mod, 0.0f, &q, &k, &v, ws, need - 1,
                                  nullptr),
           BSM_E_WORKSPACE);
    ACCEPT(bsm_flex_attention_bwd(B, H, T, D, &q, &k, &v, &o, lse, &q, &bm, &s, &mod, 0.0f, &q, &k, &v, ws, need,
                                  nullptr));
    const bsm::AttnParams &p = stub::last_attn;
    const size_t rows = (size_t)B * H * T * 4, part = (size_t)B * H * p.nqt * (2 * 1024 + 1) * 4;
    CHECK(inside(p.delta, rows, ws, need));
    CHECK(inside(p.lse2, rows, ws, need));
    CHECK(inside(p.dslope_part, (size_t)B * H * p.nqt * 4, ws, need));
    CHECK(inside(p.dbias_part, part, ws, need));
    CHECK(reinterpret_cast<char *>(p.lse2) >= reinterpret_cast<char *>(p.delta) + rows);
    CHECK(reinterpret_cast<char *>(p.dbias_part) >= reinterpret_cast<char *>(p.dslope_part) + B * H * p.nqt * 4);
    CHECK(p.dbias == mod.bias_grad);
    bsm_score_mod m3;
    std::memset(&m3, 0, sizeof(m3));
    m3.bias_grad = mod.bias_grad;  // a gradient output without the table
    REJECT(bsm_flex_attention_bwd(B, H, T, D, &q, &k, &v, &o, lse, &q, &bm, &s, &m3, 0.0f, &q, &k, &v, ws, need,
                                  nullptr),
           BSM_E_INVALID);
}

static void decoding() {
    const int32_t B = 2, H = 4, C = 4096, D = 128;
    bsm_mask_spec s = spec_of(C);
    bsm_tensor q = tensor_of(arena(16 << 20), H, 1, D), k = tensor_of(arena(18 << 20), H, C, D), v = k, o = q;
    int32_t *kv_len = reinterpret_cast<int32_t *>(arena(2 << 20));
    float *lse = reinterpret_cast<float *>(arena(12 << 20));
    const size_t need = bsm_decode_workspace_bytes(B, H, C, D);
    char *ws = arena(40 << 20);
    REJECT(bsm_flex_attention_decode(B, H, C, D, nullptr, 0, &q, &k, &v, &s, nullptr, nullptr, 0.0f, &o, lse, ws,
                                     need, nullptr),
           BSM_E_INVALID);
    REJECT(bsm_flex_attention_decode(B, H, C, D, kv_len, 2, &q, &k, &v, &s, nullptr, nullptr, 0.0f, &o, lse, ws, need,
                                     nullptr),
           BSM_E_INVALID);
    REJECT(bsm_flex_attention_decode(B, H, C, D, kv_len, 0, &q, &k, &v, &s, nullptr, nullptr, 0.0f, &o, lse, ws,
                                     need - 4, nullptr),
           BSM_E_WORKSPACE);
    ACCEPT(bsm_flex_attention_decode(B, H, C, D, kv_len, 1, &q, &k, &v, &s, nullptr, nullptr, 0.0f, &o, lse, ws, need,
                                     nullptr));
    CHECK(stub::last_decode_part == reinterpret_cast<float *>(ws));
    CHECK(stub::last_decode.kv_len_stride == 1 && stub::last_decode.D == D);
    CHECK(stub::last_decode.block_table == nullptr);
    // paged: 16 logical pages of 256 keys over a pool of 40
    int32_t *table = reinterpret_cast<int32_t *>(arena(1 << 20));
    bsm_tensor kp = tensor_of(arena(20 << 20), H, 256, D);
    REJECT(bsm_flex_attention_decode_paged(B, H, D, 96, 40, table, 16, kv_len, 1, &q, &kp, &kp, &s, nullptr, nullptr,
                                           0.0f, &o, lse, ws, need, nullptr),
           BSM_E_INVALID);
    REJECT(bsm_flex_attention_decode_paged(B, H, D, 256, 40, nullptr, 16, kv_len, 1, &q, &kp, &kp, &s, nullptr,
                                           nullptr, 0.0f, &o, lse, ws, need, nullptr),
           BSM_E_INVALID);
    REJECT(bsm_flex_attention_decode_paged(B, H, D, 256, 40, table, 8, kv_len, 1, &q, &kp, &kp, &s, nullptr, nullptr,
                                           0.0f, &o, lse, ws, need, nullptr),
           BSM_E_INVALID);  // 8 x 256 != the mask's 4096
    ACCEPT(bsm_flex_attention_decode_paged(B, H, D, 256, 40, table, 16, kv_len, 1, &q, &kp, &kp, &s, nullptr, nullptr,
                                           0.0f, &o, lse, ws, need, nullptr));
    CHECK(stub::last_decode.block_table == table && stub::last_decode.table_stride == 16);
    CHECK(stub::last_decode.page_size == 256 && stub::last_decode.num_pages == 40);
    CHECK(stub::last_decode.a.k_sb == kp.stride_b);
    // gathering the live keys of the pages into contiguous rows
    bsm_tensor kc = tensor_of(arena(24 << 20), H, 1000, D);
    REJECT(bsm_gather_kv_pages(B, H, D, 256, 40, table, 16, 0, &kp, &kp, &kc, &kc, nullptr), BSM_E_INVALID);
    REJECT(bsm_gather_kv_pages(B, H, D, 256, 40, table, 16, 4097, &kp, &kp, &kc, &kc, nullptr), BSM_E_INVALID);
    REJECT(bsm_gather_kv_pages(B, H, 96, 256, 40, table, 16, 1000, &kp, &kp, &kc, &kc, nullptr), BSM_E_UNSUPPORTED);
    ACCEPT(bsm_gather_kv_pages(B, H, D, 256, 40, table, 16, 1000, &kp, &kp, &kc, &kc, nullptr));
    CHECK(stub::last_gather.n_keys == 1000 && stub::last_gather.row_bytes == 2 * D);
    CHECK(stub::last_gather.ks_b == 2 * kp.stride_b && stub::last_gather.kd_t == 2 * kc.stride_t);
    // the allocation-free variant looks up its static array on the current
    // device first: with no device that is a HIP error, never a launch
    const int before = stub::calls;
    const bsm_status st = bsm_flex_attention_decode_static(B, H, C, D, kv_len, 0, &q, &k, &v, &s, nullptr, nullptr,
                                                           0.0f, &o, lse, nullptr);
    CHECK(st == BSM_OK || st == BSM_E_HIP);
    CHECK(st != BSM_E_HIP || stub::calls == before);
    CHECK(bsm_decode_static_max_bytes() == (size_t)16 << 20);
}

int main() {
    CHECK(std::strlen(bsm_version()) > 0);
    block_mask_build();
    attention();
    decoding();
    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host driver: all checks passed (%d launches recorded)\n", stub::calls);
    return 0;
}
