/*
 * Oracle (test infrastructure only): brute-force count of visible (q, kv)
 * pairs in every tile_q x tile_k block of the attention grid (128 x 128 by
 * default; the tutorial's sharp edges call the block size a tunable that
 * captures more sparsity when smaller).
 *
 * Definition followed: a tile's class is decided by how many of its scores
 * the mask predicate lets through -- none (empty), all 128 x 128 (full) or
 * some (partial).  Tutorial "FlexAttention in PyTorch", section "The two
 * hooks" (BlockMask of empty / partially masked / full blocks); speedrun
 * notes "FlexAttention", tile-summary paragraph (128 x 128 tiles, a tile with
 * one visible score costs a full tile).  A tile at the end of a length that
 * is not a multiple of 128 holds fewer than 128 x 128 pairs, so it is never
 * full.
 *
 * The predicate is evaluated for every single pair, exactly as written on the
 * pages: causal (q >= kv), same document (docs[q] == docs[kv]), window
 * (q - kv < window), sinks (kv < SINKS) OR-ed with the window
 * (speedrun notes, code listing; tutorial, Patterns 1 and 2), prefix
 * (kv < PREFIX) OR-ed with the causal term (prefix-LM masking, named in the
 * tutorial's introduction) -- or, for a composed mask (tutorial, Pattern 3:
 * and_masks / or_masks), any boolean function of those five terms given as
 * its truth table.  Queries sit at absolute positions q_offset + i.
 *
 * No shortcut, no interval reasoning, no pruning: O(Q_LEN * KV_LEN) work per
 * mask.  Only tests/, the smoke check and the benchmark's CPU baseline use
 * this.
 */
#include <stdint.h>
#include <string.h>

/* flags: bit0 causal, bit1 document, bit2 window, bit3 sinks, bit4 prefix,
 * bit5 truth table (table bit C + 2 Dc + 4 W + 8 S + 16 P) */
static inline int visible_pair(int64_t q, int64_t kv, int flags,
                               const int32_t *docs, int64_t window,
                               int64_t sinks, int64_t prefix, uint32_t table)
{
    const int c = q >= kv;
    const int d = (flags & 2) ? docs[q] == docs[kv] : 0;
    const int w = (flags & 4) ? (q - kv) < window : 0;
    const int s = (flags & 8) ? kv < sinks : 0;
    const int p = (flags & 16) ? kv < prefix : 0;
    if (flags & 32)
        return (int)((table >> (c + 2 * d + 4 * w + 8 * s + 16 * p)) & 1u);
    int ok = 1;
    if (flags & 1)
        ok = ok && (c || p);
    if (flags & 2)
        ok = ok && d;
    if (flags & 4)
        ok = ok && (w || s);
    return ok;
}

/*
 * counts: int32 [mask_b, ceil(q_len/tile_q), ceil(kv_len/tile_k)];
 * counts[b][i][j] = number of visible pairs with query index qi in
 * [tile_q i, min(tile_q (i + 1), q_len) - 1] (absolute position
 * q_offset + qi) and kv in [tile_k j, min(tile_k (j + 1), kv_len) - 1].
 * docs: int32 [mask_b, positions] (may be NULL when bit1 is clear), indexed by
 * absolute position; positions >= max(kv_len, q_offset + q_len).
 * Returns 0 on success, -1 on a bad size.
 */
int oracle_tile_counts(int64_t kv_len, int64_t q_len, int64_t q_offset, int mask_b, int flags,
                       const int32_t *docs, int64_t positions, int64_t window, int64_t sinks,
                       int64_t prefix, uint32_t table, int64_t tile_q, int64_t tile_k, int32_t *counts)
{
    if (kv_len <= 0 || q_len <= 0 || q_offset < 0 || mask_b <= 0 || tile_q <= 0 || tile_k <= 0)
        return -1;
    if ((flags & 2) && positions < (kv_len > q_offset + q_len ? kv_len : q_offset + q_len))
        return -1;
    const int64_t nq = (q_len + tile_q - 1) / tile_q;
    const int64_t nk = (kv_len + tile_k - 1) / tile_k;
    for (int b = 0; b < mask_b; ++b) {
        const int32_t *d = docs ? docs + (int64_t)b * positions : NULL;
        int32_t *c = counts + (int64_t)b * nq * nk;
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < nq; ++i) {
            const int64_t q1 = (i + 1) * tile_q < q_len ? (i + 1) * tile_q : q_len;
            for (int64_t j = 0; j < nk; ++j) {
                const int64_t k1 = (j + 1) * tile_k < kv_len ? (j + 1) * tile_k : kv_len;
                int32_t n = 0;
                for (int64_t qi = i * tile_q; qi < q1; ++qi)
                    for (int64_t kv = j * tile_k; kv < k1; ++kv)
                        n += visible_pair(q_offset + qi, kv, flags, d, window, sinks, prefix, table);
                c[i * nk + j] = n;
            }
        }
    }
    return 0;
}
