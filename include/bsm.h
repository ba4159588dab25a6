/*
 * bsm.h -- block-sparse masked attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over three operations:
 *
 *   bsm_build_block_mask    mask predicate -> per-tile classes -> tile lists
 *   bsm_flex_attention_fwd  exact softmax attention over the listed tiles
 *   bsm_flex_attention_bwd  dQ, dK, dV over the same tile lists
 *
 * The operations follow the FlexAttention method as described on three web
 * pages: speedrun notes "FlexAttention" (sbabichenko.com), the paper record
 * "FlexAttention: A Programming Model for Generating Optimized Attention
 * Kernels", and the tutorial "FlexAttention in PyTorch" (intellisensei.com).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing and keeps no pointer after a call returns.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    null stream) and returns without synchronising.  Nothing that lives in
 *    device memory (document ids, the window value) is read by the host.
 *  - Errors: a call returns a bsm_status.  Argument checks run on the host
 *    before anything is enqueued; on failure nothing is launched and
 *    bsm_last_error() gives a message (thread-local, valid until the next
 *    call on the same thread).  BSM_E_HIP reports a launch failure.
 *  - Sizes: a mask has KV_LEN keys (bsm_mask_spec.seq_len) and Q_LEN queries
 *    (q_len; 0 means Q_LEN = KV_LEN), each from 1 to 4,194,304, not
 *    necessarily multiples of 128.  Query i sits at absolute position
 *    q_offset + i (0 by default), so queries can be the last positions of a
 *    cache.  Tiles are 128 x 128: QT = ceil(Q_LEN / 128) query tiles and
 *    KT = ceil(KV_LEN / 128) key tiles; a tile cut short by a length that is
 *    not a multiple of 128 is never full.
 *  - Tensors are [B, H, T, D] of bf16 or fp16 elements (bsm_tensor.dtype;
 *    every tensor of one call has the same type) with the last dimension
 *    contiguous and the other three strides given in elements.  Base
 *    pointers must be 16-byte aligned and strides multiples of 8 elements.
 *    The matrix-core products take their operands in the tensors' type
 *    (including the probabilities and score gradients formed on the way)
 *    and accumulate in fp32 (tutorial "FlexAttention in PyTorch", "What to
 *    expect, and the sharp edges": bf16 and fp16 inputs).
 */
#ifndef BSM_H
#define BSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSM_OK = 0,
    BSM_E_INVALID = 1,     /* bad argument: null pointer, bad size or stride */
    BSM_E_UNSUPPORTED = 2, /* valid request outside what the library covers  */
    BSM_E_WORKSPACE = 3,   /* workspace missing or too small                 */
    BSM_E_HIP = 4          /* HIP runtime reported an error at launch        */
} bsm_status;

/* Mask predicate terms (bsm_mask_spec.flags).  With q the query's absolute
 * position, a (q, kv) pair is visible iff
 *   (!CAUSAL   || q >= kv || (PREFIX && kv < prefix_len))
 * && (!DOCUMENT || doc_ids[b][q] == doc_ids[b][kv])
 * && (!WINDOW   || q - kv < *window || (SINKS && kv < num_sinks))
 * Causal, same-document and window terms: speedrun notes "FlexAttention",
 * code listing; sinks OR-ed with the window: tutorial "FlexAttention in
 * PyTorch", Pattern 2; a prefix every query sees (prefix-LM masking, named
 * in that tutorial's introduction) OR-ed with the causal term.  SINKS
 * without WINDOW and PREFIX without CAUSAL have no effect.
 * TABLE replaces that combination by any and / or / not composition of the
 * five terms (that tutorial, Pattern 3: compose masks with and_masks /
 * or_masks): the pair is visible iff bit (C + 2 Dc + 4 W + 8 S + 16 P) of
 * bsm_mask_spec.table is set, where C = (q >= kv), Dc = same document,
 * W = (q - kv < *window), S = (kv < num_sinks), P = (kv < prefix_len); a
 * term whose flag (DOCUMENT, WINDOW, SINKS, PREFIX) is not set is 0.  CAUSAL
 * is not needed for C. */
enum {
    BSM_MASK_CAUSAL = 1u,
    BSM_MASK_DOCUMENT = 2u,
    BSM_MASK_WINDOW = 4u,
    BSM_MASK_SINKS = 8u,
    BSM_MASK_PREFIX = 16u,
    BSM_MASK_TABLE = 32u
};

/* Score modifications (bsm_score_mod.flags), applied to s = scale * q.k in
 * this order (tutorial "FlexAttention in PyTorch", Pattern 3):
 *   ALIBI:   s <- s - alibi_slopes[h] * (q - kv)     (absolute positions)
 *   BIAS:    s <- s + bias[h][R + clip(q - kv, -R, R)]
 *   SOFTCAP: s <- softcap * tanh(s / softcap)
 * BIAS is a learned relative-position bias (named in the same section): one
 * scalar per head and query-key distance, distances beyond R sharing the
 * end entries (clipped relative positions).  ALIBI and BIAS together are
 * BSM_E_UNSUPPORTED (within R a slope is a special table).               */
enum {
    BSM_MOD_ALIBI = 1u,
    BSM_MOD_SOFTCAP = 2u,
    BSM_MOD_BIAS = 4u
};

/* Largest bias radius R: the kernels keep the head's 2R + 1 entries (and
 * the backward its per-wave gradient sums) in LDS. */
#define BSM_BIAS_MAX_RADIUS 1024

typedef struct {
    uint32_t flags;          /* BSM_MASK_* bits                                    */
    int32_t seq_len;         /* KV_LEN: keys 0 .. seq_len - 1                      */
    int32_t mask_b;          /* 1: one mask shared by the whole batch; else = B    */
    const int32_t *doc_ids;  /* DOCUMENT: device int32 [mask_b, P], P = the number
                                of positions, max(KV_LEN, q_offset + Q_LEN),
                                indexed by absolute position for queries and keys;
                                any values; non-decreasing rows take the fast path */
    const int32_t *window;   /* WINDOW: device int32 scalar, read by the kernels at
                                run time (may change between calls, no rebuild of
                                anything but the block mask)                       */
    int32_t num_sinks;       /* SINKS: keys kv < num_sinks widen the window        */
    int32_t prefix_len;      /* PREFIX: keys kv < prefix_len widen the causal term
                                (host value, >= 0; values above KV_LEN act as
                                KV_LEN)                                            */
    int32_t q_len;           /* Q_LEN; 0: equal to seq_len                         */
    int32_t q_offset;        /* absolute position of query 0 (>= 0)                */
    uint32_t table;          /* TABLE: truth table over the five terms             */
    int32_t kv_block;        /* key-block width of the row lists: 128 (0 means
                                128) or 64, i.e. blocks of 128 queries x 64 keys
                                (tutorial "FlexAttention in PyTorch", "What to
                                expect, and the sharp edges", item 4: the block
                                size is a tunable; smaller blocks capture more
                                sparsity).  The forward and dQ then visit only
                                the listed 64-key blocks; the column lists stay
                                128 x 128.                                    */
} bsm_mask_spec;

/* A block mask: the tile-level summary of a mask predicate (speedrun notes
 * "FlexAttention", tile-summary paragraph: per row of query tiles, the number
 * of tiles that are not fully masked and their column indices; tutorial,
 * "The two hooks": blocks are empty, partial or full).
 * Layout, all device int32, head dimension 1 (shared by every head); KB =
 * ceil(KV_LEN / kv_block) key blocks (KB = KT for 128-key blocks):
 *   kv_num_blocks       [mask_b, 1, QT]      partial blocks per query-tile row
 *   kv_indices          [mask_b, 1, QT, KB]  their key-block indices, ascending,
 *                                            slots >= count hold -1
 *   full_kv_num_blocks  [mask_b, 1, QT]      full blocks per row
 *   full_kv_indices     [mask_b, 1, QT, KB]
 *   q_num_blocks        [mask_b, 1, KT]      transposed view (per key tile,
 *   q_indices           [mask_b, 1, KT, QT]   the query tiles), used by the
 *   full_q_num_blocks   [mask_b, 1, KT]       backward pass
 *   full_q_indices      [mask_b, 1, KT, QT]
 *   doc_range           [mask_b, P, 2]       DOCUMENT only (else may be NULL):
 *                                            first and last position of the
 *                                            document holding t when the row's
 *                                            ids are non-decreasing (documents
 *                                            are contiguous runs, as for the
 *                                            running count of end-of-text flags,
 *                                            speedrun notes code listing);
 *                                            (-1, -1) for every t of a row whose
 *                                            ids are not, which makes the
 *                                            attention kernels compare ids key
 *                                            by key instead
 *   kv_order            [mask_b * QT, 4]     (16-byte aligned) work order of the
 *                                            query-tile rows:
 *                                            entry e describes the row (bm, i)
 *                                            with the e-th largest
 *                                            min(kv_num + full_kv_num, 8191),
 *                                            ties in ascending bm * QT + i, as
 *                                            (bm * QT + i, full_kv_num,
 *                                            kv_num, first listed key block:
 *                                            the first full one if any, else
 *                                            the first partial one, else 0)
 *   q_order             [mask_b * KT, 4]     the same for the key-tile columns
 *                                            (q_num + full_q_num; first listed
 *                                            query tile)
 * The work orders are a schedule, not part of the mask: the attention
 * kernels start the rows (columns) with the most tiles first, so that the
 * short ones fill the end of the launch.
 * bsm_build_block_mask writes all eleven; the forward reads the kv_* five
 * and doc_range, the backward reads all eleven. */
typedef struct {
    int32_t *kv_num_blocks;
    int32_t *kv_indices;
    int32_t *full_kv_num_blocks;
    int32_t *full_kv_indices;
    int32_t *q_num_blocks;
    int32_t *q_indices;
    int32_t *full_q_num_blocks;
    int32_t *full_q_indices;
    int32_t *doc_range;
    int32_t *kv_order;
    int32_t *q_order;
} bsm_block_mask;

typedef struct {
    uint32_t flags;              /* BSM_MOD_* bits                   */
    const float *alibi_slopes;   /* ALIBI: device float32 [H]         */
    float softcap;               /* SOFTCAP: cap value c > 0          */
    float *alibi_slopes_grad;    /* ALIBI, backward only: NULL, or device
                                    float32 [H] that bsm_flex_attention_bwd
                                    overwrites with dL/dslope[h], summed over
                                    the batch (a learned bias trains through the
                                    fused backward: tutorial "FlexAttention in
                                    PyTorch", Pattern 3).  Non-NULL without
                                    ALIBI is BSM_E_INVALID; the forward
                                    ignores it.                        */
    const float *bias;           /* BIAS: device float32 [H, 2 bias_radius + 1],
                                    rows contiguous; entry R + d holds the bias
                                    of distance q - kv = d                */
    int32_t bias_radius;         /* BIAS: R, 0 <= R <= BSM_BIAS_MAX_RADIUS  */
    float *bias_grad;            /* BIAS, backward only: NULL, or device
                                    float32 [H, 2R + 1] that
                                    bsm_flex_attention_bwd overwrites with
                                    dL/dbias summed over the batch (the sums
                                    are formed in a fixed order: repeated
                                    calls give identical bits).  Non-NULL
                                    without BIAS is BSM_E_INVALID; the forward
                                    ignores it, a decoding step rejects it. */
} bsm_score_mod;

/* Element types of bsm_tensor.dtype (0, the zero-initialised value, is
 * bf16). */
enum {
    BSM_DTYPE_BF16 = 0,
    BSM_DTYPE_F16 = 1
};

/* Tensor [B, H, T, D]; element (b,h,t,d) lives at
 * ptr + b*stride_b + h*stride_h + t*stride_t + d  (strides in elements). */
typedef struct {
    void *ptr;
    int64_t stride_b;
    int64_t stride_h;
    int64_t stride_t;
    int32_t dtype;           /* BSM_DTYPE_*                                        */
} bsm_tensor;

/* Bytes of device workspace bsm_build_block_mask needs for `spec` (per-tile
 * class bytes, per-chunk monotonicity flags, work-order blocks); 0 for an
 * invalid spec. */
size_t bsm_block_mask_workspace_bytes(const bsm_mask_spec *spec);

/* Build the block mask of `spec` (speedrun notes "FlexAttention",
 * tile-summary paragraph; tutorial "FlexAttention in PyTorch", "The two
 * hooks").  Every tile's class comes from the exact number of visible pairs
 * in it: 0 -> empty (not listed), 128*128 -> full, otherwise partial.
 * The tutorial's advice holds: build once per mask and reuse it across
 * forward calls; rebuild only when the window or documents change.
 * workspace: device, >= bsm_block_mask_workspace_bytes(), 256-byte aligned,
 * contents need not be initialised.  Errors: BSM_E_INVALID (null spec/out
 * pointers, bad T or mask_b, DOCUMENT without doc_ids, WINDOW without
 * window), BSM_E_WORKSPACE, BSM_E_HIP. */
bsm_status bsm_build_block_mask(const bsm_mask_spec *spec, const bsm_block_mask *out,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Forward attention (speedrun notes "FlexAttention", Context: the two
 * matmuls and the softmax fused in one tiled kernel that never writes the
 * Q_LEN x KV_LEN scores; the kernel visits only listed tiles, applies the
 * elementwise mask only to partial tiles and the score modifications to
 * every score).
 *   out[b,h,i,:] = sum_{kv visible} softmax_kv(s)[kv] * v[b,h,kv,:]
 *   lse[b,h,i]   = log sum_{kv visible} exp(s[kv])   (natural log; -inf and
 *                  out = 0 for a query with no visible key)
 * q, out: [B, H, Q_LEN, D]; k, v: [B, H, KV_LEN, D] (T = KV_LEN =
 * spec->seq_len, Q_LEN from spec->q_len).  D in {64, 128, 256} (that
 * tutorial's sharp edges: head dims that are multiples of 64).  scale <= 0
 * selects 1/sqrt(D).  mod may be NULL.  ALiBi uses absolute positions.
 * bm must be the block mask of `spec` (as built by bsm_build_block_mask);
 * the mask batch index is b when spec->mask_b == B, else 0.
 * lse: device float32 [B, H, Q_LEN], contiguous.
 * Errors: BSM_E_INVALID, BSM_E_UNSUPPORTED (D not 64/128/256), BSM_E_HIP. */
bsm_status bsm_flex_attention_fwd(int32_t B, int32_t H, int32_t T, int32_t D,
                                  const bsm_tensor *q, const bsm_tensor *k,
                                  const bsm_tensor *v, const bsm_block_mask *bm,
                                  const bsm_mask_spec *spec, const bsm_score_mod *mod,
                                  float scale, const bsm_tensor *out, float *lse,
                                  void *stream);

/* Bytes of device workspace bsm_flex_attention_bwd needs: Delta and
 * lse log2(e) per query (2 x B*H*Q_LEN floats) and one slope-gradient partial
 * per (batch, head, query tile), each part rounded up to 256 bytes.  Q is
 * Q_LEN (the square case: T). */
size_t bsm_bwd_workspace_bytes(int32_t B, int32_t H, int32_t Q, int32_t D);

/* The same for a call with score modifications `mod` (may be NULL): with
 * BIAS it adds one bias-gradient partial row of 2R + 1 floats per (batch,
 * head, query tile), B*H*ceil(Q/128)*(2R + 1)*4 bytes rounded up to 256.
 * Returns 0 for arguments the backward would reject. */
size_t bsm_bwd_workspace_bytes_mod(int32_t B, int32_t H, int32_t Q, int32_t D, const bsm_score_mod *mod);

/* Backward attention: gradients of sum(out * dout) with respect to q, k, v
 * through the softmax, the mask and the score modifications (tutorial
 * "FlexAttention in PyTorch", Pattern 3: differentiable score mods with a
 * fused backward).  Visits exactly the tiles the block mask lists.
 * out and lse are the forward's outputs for the same inputs.
 * dq: bf16 [B, H, Q_LEN, D]; dk, dv: bf16 [B, H, KV_LEN, D]; fully
 * overwritten.
 * mod->alibi_slopes_grad (optional, ALIBI): dL/dslope[h] = sum over the batch
 * and the visible pairs of g_qk (k - q), with g the gradient with respect to
 * the score the ALiBi term is added to; deterministic (fixed-order sums).
 * mod->bias_grad (optional, BIAS): dL/dbias[h][R + r] = sum over the batch
 * and the visible pairs with clip(q - kv, -R, R) = r of g_qk, the same g;
 * deterministic as well.  With BIAS the kernels form these sums whether or
 * not bias_grad is given.
 * workspace: device, >= bsm_bwd_workspace_bytes_mod(B, H, Q_LEN, D, mod),
 * 256-byte aligned.  With BIAS, D in {64, 128} (BSM_E_UNSUPPORTED at 256).
 * Errors: as the forward, plus BSM_E_WORKSPACE. */
bsm_status bsm_flex_attention_bwd(int32_t B, int32_t H, int32_t T, int32_t D,
                                  const bsm_tensor *q, const bsm_tensor *k,
                                  const bsm_tensor *v, const bsm_tensor *out,
                                  const float *lse, const bsm_tensor *dout,
                                  const bsm_block_mask *bm, const bsm_mask_spec *spec,
                                  const bsm_score_mod *mod, float scale,
                                  const bsm_tensor *dq, const bsm_tensor *dk,
                                  const bsm_tensor *dv, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Bytes of device workspace bsm_flex_attention_decode needs: per (batch,
 * head) and slot of eight 128-key tiles of the capacity, D + 2 floats (the
 * slot's unnormalised output, running maximum and sum). */
size_t bsm_decode_workspace_bytes(int32_t B, int32_t H, int32_t capacity, int32_t D);

/* Decoding step (tutorial "FlexAttention in PyTorch", section "Decoding and
 * paged KV caches": one query per step against a cache that grows; the
 * allocation is bucketed and the mask follows the current length).
 * The cache k, v is [B, H, capacity, D] (any capacity >= 1); its live length
 * is a DEVICE int32 value read by the kernels -- kv_len[0] for every batch
 * element (kv_len_stride 0) or kv_len[b] (kv_len_stride 1) -- so a step
 * needs no host value and one launch configuration serves a whole bucket.
 * Values are clamped to [0, capacity]; 0 gives out = 0, lse = -inf.
 * The query of batch element b (q: [B, H, 1, D], stride_t unused) sits at
 * position kv_len[b] - 1 and sees key kv < kv_len[b] when the mask predicate
 * of spec (seq_len == capacity, doc_ids [mask_b, capacity]) holds for
 * (kv_len[b] - 1, kv); its scores take the score modifications of the
 * forward.
 * bm (optional, may be NULL): the block mask of spec built once for the
 * whole capacity (so capacity is then a multiple of 128, and kv_block 128:
 * 64-key blocks are BSM_E_UNSUPPORTED here).  The step reads
 * only the key tiles listed in the row of query tiles holding the query
 * (every tile some query of that row sees), so a document-masked step reads
 * its document's tiles only; the mask stays valid while the cache grows
 * within the capacity.  Without it every key below the live length is
 * visited, except 1024-key chunks wholly before the window.
 * out: [B, H, 1, D] of q's type (stride_t unused); lse: fp32 [B, H],
 * natural log.
 * workspace: device, >= bsm_decode_workspace_bytes(), 256-byte aligned.
 * Errors: BSM_E_INVALID, BSM_E_UNSUPPORTED (D), BSM_E_WORKSPACE, BSM_E_HIP. */
bsm_status bsm_flex_attention_decode(int32_t B, int32_t H, int32_t capacity, int32_t D,
                                     const int32_t *kv_len, int32_t kv_len_stride,
                                     const bsm_tensor *q, const bsm_tensor *k, const bsm_tensor *v,
                                     const bsm_mask_spec *spec, const bsm_block_mask *bm,
                                     const bsm_score_mod *mod, float scale,
                                     const bsm_tensor *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The decoding step over a paged key/value cache (tutorial "FlexAttention in
 * PyTorch", "Decoding and paged KV caches": the cache is held in fixed-size
 * pages that a block table maps to each sequence's logical key blocks).
 * k_pages, v_pages: pools of num_pages pages, each [H, page_size, D]; the
 * tensors' stride_b is the page stride, stride_h and stride_t as usual.
 * block_table: device int32 [B, table_stride]: key kv of batch element b
 * sits at row kv % page_size of page block_table[b][kv / page_size].  The
 * logical capacity is table_stride * page_size (spec->seq_len and any block
 * mask are for it); entries for pages at or past the live length are never
 * read; entries outside [0, num_pages) are clamped into it (a wrong page,
 * never a read outside the pools).  page_size: a positive multiple of 64.
 * Otherwise as bsm_flex_attention_decode, whose workspace size it shares
 * (bsm_decode_workspace_bytes(B, H, table_stride * page_size, D)); the
 * results equal those of that call on the gathered contiguous cache bit for
 * bit.  The pools, the table and every output stay the caller's; the table
 * is read by the kernels on `stream`, so it may change between steps (and
 * between replays of a captured graph) like kv_len.
 * Errors: BSM_E_INVALID for page_size < 64 or not a multiple of 64,
 * num_pages < 1, a NULL block_table, table_stride < 1 or a logical capacity
 * past 2^22, and then every error of bsm_flex_attention_decode for the
 * logical capacity (BSM_E_INVALID, BSM_E_UNSUPPORTED for D, BSM_E_WORKSPACE,
 * BSM_E_HIP on a failed launch). */
bsm_status bsm_flex_attention_decode_paged(int32_t B, int32_t H, int32_t D, int32_t page_size,
                                           int32_t num_pages, const int32_t *block_table,
                                           int32_t table_stride, const int32_t *kv_len,
                                           int32_t kv_len_stride, const bsm_tensor *q,
                                           const bsm_tensor *k_pages, const bsm_tensor *v_pages,
                                           const bsm_mask_spec *spec, const bsm_block_mask *bm,
                                           const bsm_score_mod *mod, float scale,
                                           const bsm_tensor *out, float *lse, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* Copies the first n_keys keys and values of every sequence of a paged
 * cache into contiguous rows (tutorial "FlexAttention in PyTorch",
 * "Decoding and paged KV caches"), for the calls that take contiguous K and
 * V: a block of several new queries runs the rectangular forward over them.
 * k_pages, v_pages, block_table, table_stride, page_size, num_pages: as in
 * bsm_flex_attention_decode_paged.  k_out, v_out: device tensors
 * [B, H, n_keys, D] of the pools' element type, written (key kv of batch
 * element b, head h at k_out + b stride_b + h stride_h + kv stride_t).
 * Table entries outside [0, num_pages) are clamped into it.  Enqueued on
 * `stream`; nothing is allocated.  Errors: BSM_E_INVALID for B or H < 1,
 * page_size not a positive multiple of 64, num_pages < 1, a NULL table,
 * table_stride < 1, n_keys outside [1, table_stride * page_size], or a bad
 * tensor (NULL, unaligned, mixed element types); BSM_E_UNSUPPORTED for D
 * outside {64, 128, 256}; BSM_E_HIP on a failed launch. */
bsm_status bsm_gather_kv_pages(int32_t B, int32_t H, int32_t D, int32_t page_size, int32_t num_pages,
                               const int32_t *block_table, int32_t table_stride, int32_t n_keys,
                               const bsm_tensor *k_pages, const bsm_tensor *v_pages,
                               const bsm_tensor *k_out, const bsm_tensor *v_out, void *stream);

/* Allocation-free decoding step, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same step as bsm_flex_attention_decode, with the
 * partials kept in a static device array of bsm_decode_static_max_bytes()
 * (16 MiB) that the library holds on each GPU it runs on until the process
 * ends, instead of a caller workspace.  Requests whose partials,
 * B * H * ceil(capacity / 1024) * (D + 2) * 4 bytes, exceed it return
 * BSM_E_WORKSPACE.  The call allocates nothing; stream must belong to the
 * current device (BSM_E_INVALID otherwise).  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (different streams, or host
 * threads) race and give wrong results; calls ordered on one stream are
 * safe.  Errors: as bsm_flex_attention_decode. */
size_t bsm_decode_static_max_bytes(void);
bsm_status bsm_flex_attention_decode_static(int32_t B, int32_t H, int32_t capacity, int32_t D,
                                            const int32_t *kv_len, int32_t kv_len_stride,
                                            const bsm_tensor *q, const bsm_tensor *k, const bsm_tensor *v,
                                            const bsm_mask_spec *spec, const bsm_block_mask *bm,
                                            const bsm_score_mod *mod, float scale,
                                            const bsm_tensor *out, float *lse, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *bsm_last_error(void);

/* Library version string. */
const char *bsm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSM_H */
