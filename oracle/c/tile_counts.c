/*
 * Oracle (test infrastructure only): brute-force count of visible (q, kv)
 * pairs in every 128 x 128 tile of the attention grid.
 *
 * Definition followed: a tile's class is decided by how many of its scores
 * the mask predicate lets through -- none (empty), all (full) or some
 * (partial).  Tutorial "FlexAttention in PyTorch", section "The two hooks"
 * (BlockMask of empty / partially masked / full blocks); speedrun notes
 * "FlexAttention", tile-summary paragraph (128 x 128 tiles, a tile with one
 * visible score costs a full tile).
 *
 * The predicate is evaluated for every single pair, exactly as written on the
 * pages: causal (q >= kv), same document (docs[q] == docs[kv]), window
 * (q - kv < window), sinks (kv < SINKS) OR-ed with the window
 * (speedrun notes, code listing; tutorial, Patterns 1 and 2), prefix
 * (kv < PREFIX) OR-ed with the causal term (prefix-LM masking, named in the
 * tutorial's introduction).
 *
 * No shortcut, no interval reasoning, no pruning: O(T^2) work per mask.
 * Only tests/, the smoke check and the benchmark's CPU baseline use this.
 */
#include <stdint.h>
#include <string.h>

#define ORACLE_TILE 128

/* flags: bit0 causal, bit1 document, bit2 window, bit3 sinks, bit4 prefix */
static inline int visible_pair(int64_t q, int64_t kv, int flags,
                               const int32_t *docs, int64_t window,
                               int64_t sinks, int64_t prefix)
{
    int ok = 1;
    if (flags & 1) {
        int c = q >= kv;
        if (flags & 16)
            c = c || (kv < prefix);
        ok = ok && c;
    }
    if (flags & 2)
        ok = ok && (docs[q] == docs[kv]);
    if (flags & 4) {
        int w = (q - kv) < window;
        if (flags & 8)
            w = w || (kv < sinks);
        ok = ok && w;
    }
    return ok;
}

/*
 * counts: int32 [mask_b, T/128, T/128]; counts[b][i][j] = number of visible
 * pairs with q in [128 i, 128 i + 127] and kv in [128 j, 128 j + 127].
 * docs: int32 [mask_b, T] (may be NULL when bit1 is clear).
 * Returns 0 on success, -1 if T is not a positive multiple of 128.
 */
int oracle_tile_counts(int64_t T, int mask_b, int flags, const int32_t *docs,
                       int64_t window, int64_t sinks, int64_t prefix,
                       int32_t *counts)
{
    if (T <= 0 || T % ORACLE_TILE != 0 || mask_b <= 0)
        return -1;
    const int64_t nt = T / ORACLE_TILE;
    for (int b = 0; b < mask_b; ++b) {
        const int32_t *d = docs ? docs + (int64_t)b * T : NULL;
        int32_t *c = counts + (int64_t)b * nt * nt;
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < nt; ++i) {
            for (int64_t j = 0; j < nt; ++j) {
                int32_t n = 0;
                for (int64_t q = i * ORACLE_TILE; q < (i + 1) * ORACLE_TILE; ++q)
                    for (int64_t kv = j * ORACLE_TILE; kv < (j + 1) * ORACLE_TILE; ++kv)
                        n += visible_pair(q, kv, flags, d, window, sinks, prefix);
                c[i * nt + j] = n;
            }
        }
    }
    return 0;
}
