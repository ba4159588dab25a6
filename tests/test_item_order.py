"""Host emulation of the attention kernels' item order (CPU only): the grid
size, the queue / grab arithmetic (chunks dealt to the queues in rounds of
alternating direction) and the decode of an item into (work-order entry,
head index), written out exactly as the forward and dQ kernels compute them (including the division by magic numbers), one item per
workgroup.  For many shapes every item must be taken exactly once, and every
index the kernels form from it -- the record they load, the batch and head --
must lie inside its array.  The emulation also takes several consecutive
grabs of a queue per workgroup (items_per_wg > 1), the order a workgroup that
runs several items back to back would follow; that arrangement was built,
measured slower and dropped, and these cases keep its index arithmetic
checked."""
import itertools

import pytest

QUEUES = 8
ORDER_BLOCK_CAP = 16


def div_magic(d):
    return 0xFFFFFFFF if d <= 1 else ((1 << 32) + d - 1) // d


def div_by(k, d, m):
    if d == 1:
        return k
    q = (k * m) >> 32
    if q * d > k:
        q -= 1
    return q


def item_order(mask_b, nt, B, H):
    """Host side: the fields the launcher fills and the grid for one item
    per workgroup."""
    r = B * H if mask_b == 1 else H
    nitems = mask_b * nt * r
    cl = 4
    while cl > 0 and (1 << cl) * 4 * QUEUES > nitems:
        cl -= 1
    nrows = mask_b * nt
    nblk = nrows >> cl
    p = nrows - (nblk << cl)
    f = dict(r=r, cl=cl, nblk=nblk, p=p, m_cr=div_magic(r << cl), m_p=div_magic(p), nitems=nitems)
    nchunks = (nitems + (1 << cl) - 1) >> cl
    grid1 = (QUEUES * ((nchunks + QUEUES - 1) // QUEUES)) << cl
    return f, grid1


def item(f, queue, i):
    cl = f["cl"]
    r = i >> cl
    pos = QUEUES - 1 - queue if r & 1 else queue
    k = ((pos + QUEUES * r) << cl) + (i & ((1 << cl) - 1))
    return k if k < f["nitems"] else f["nitems"]


def decode(f, k):
    cl = f["cl"]
    cr = f["r"] << cl
    full = f["nblk"] * cr
    if k < full:
        blk = div_by(k, cr, f["m_cr"])
        w = k - blk * cr
        return (blk << cl) + (w & ((1 << cl) - 1)), w >> cl
    w = k - full
    rem = div_by(w, f["p"], f["m_p"])
    return (f["nblk"] << cl) + (w - rem * f["p"]), rem


def emulate(mask_b, nt, B, H, items_per_wg):
    f, grid1 = item_order(mask_b, nt, B, H)
    per_queue = grid1 // QUEUES
    grid = QUEUES * ((per_queue + items_per_wg - 1) // items_per_wg)
    seen = {}
    for wg in range(grid):
        queue = wg % QUEUES
        g0 = (wg // QUEUES) * items_per_wg
        for j in range(items_per_wg):
            k = item(f, queue, g0 + j)
            if k >= f["nitems"]:
                continue  # the kernel loads nothing for it
            e, rem = decode(f, k)
            assert 0 <= e < mask_b * nt, (k, e)
            assert 0 <= rem < f["r"], (k, rem)
            bm_row = e  # the record's flat row index is a permutation of this range
            b = rem // H if mask_b == 1 else bm_row // nt
            h = rem % H if mask_b == 1 else rem
            assert 0 <= b < B and 0 <= h < H
            assert (e, rem) not in seen, ("item taken twice", k)
            seen[(e, rem)] = (wg, j)
    assert len(seen) == f["nitems"], (len(seen), f["nitems"])
    return grid


SHAPES = [
    # (mask_b, nt, B, H)
    (1, 4, 2, 2),        # B2 H2 T512: the random case that faulted a two-head design
    (1, 1, 1, 1), (1, 2, 1, 1), (1, 3, 1, 3), (2, 4, 2, 2), (2, 3, 2, 5),
    (1, 8, 1, 2),        # workload 1
    (1, 512, 1, 6),      # 64K workloads
    (1, 64, 4, 16),      # dense causal 8K
    (1, 256, 1, 16),     # sinks 32K
    (2, 128, 2, 16),     # documents per batch, 16K
    (1030, 8, 1030, 1),  # many mask batches
    (1, 2048, 1, 1),     # 262,144 tokens
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("items_per_wg", [1, 2, 3, 4])
def test_every_item_once_in_range(shape, items_per_wg):
    emulate(*shape, items_per_wg)


def test_random_small_shapes():
    for mask_b, nt, B, H in itertools.product([1, 2, 3], [1, 2, 3, 5, 17], [1, 2, 3], [1, 2, 7]):
        if mask_b != 1 and mask_b != B:
            continue
        for ipw in (1, 2):
            emulate(mask_b, nt, B, H, ipw)


# dK/dV workgroup placement (the backward's column kernels), written out as
# the launcher and kernels compute it.
COL_CHUNK = 16


def xcd_remap(L, N):
    per, rem = N // 8, N % 8
    x, slot = L % 8, L // 8
    return x * (per + 1) + slot if x < rem else rem * (per + 1) + (x - rem) * per + slot


def col_grid(n):
    r = 8 * COL_CHUNK
    return (n + r - 1) // r * r


def col_remap(L):
    x, s = L % 8, L // 8
    rnd = s // COL_CHUNK
    pos = 7 - x if rnd & 1 else x
    return (8 * rnd + pos) * COL_CHUNK + s % COL_CHUNK


def dkdv_grid_of(B, H, per_head, plain_causal):
    n = B * H * per_head
    chunked = plain_causal and n % (8 * per_head) != 0
    return (col_grid(n) if chunked else n), chunked


def _placement(B, H, per_head, plain_causal):
    n = B * H * per_head
    grid, chunked = dkdv_grid_of(B, H, per_head, plain_causal)
    wgs = [col_remap(L) if chunked else xcd_remap(L, grid) for L in range(grid)]
    return n, grid, chunked, wgs


@pytest.mark.parametrize("B,H,nt", [(1, 1, 1), (1, 1, 7), (1, 6, 512), (1, 1, 512), (2, 3, 129), (3, 5, 64),
                                    (4, 16, 64), (1, 16, 256), (2, 16, 128)])
@pytest.mark.parametrize("per_tile", [1, 2])  # D = 256 runs two workgroups per key tile
@pytest.mark.parametrize("plain_causal", [False, True])
def test_dkdv_placement_covers_every_tile_once(B, H, nt, per_tile, plain_causal):
    n, grid, chunked, wgs = _placement(B, H, nt * per_tile, plain_causal)
    assert sorted(wgs) == list(range(grid))        # a bijection of the grid
    assert sorted(w for w in wgs if w < n) == list(range(n))  # every tile once; the rest exit
    assert grid - n < 8 * COL_CHUNK


@pytest.mark.parametrize("B,H,nt", [(1, 6, 512), (1, 1, 512), (1, 3, 256), (2, 3, 129), (1, 6, 128)])
def test_dkdv_placement_balances_causal_work_over_xcds(B, H, nt):
    """Under a causal mask key tile j of a head has nt - j query tiles.  The
    placement used for a plain causal mask gives the XCDs equal work when a
    head's tiles fill whole chunks, and within 25% otherwise, where
    contiguous ranges differed by 1.6x and more."""
    n, grid, chunked, wgs = _placement(B, H, nt, True)
    assert chunked
    work = [0] * 8
    for L, w in enumerate(wgs):
        if w < n:
            work[L % 8] += nt - w % nt
    ranges = [0] * 8
    for L in range(n):
        ranges[L % 8] += nt - xcd_remap(L, n) % nt
    assert max(work) / min(work) < (1.0001 if nt % COL_CHUNK == 0 else 1.25), work
    assert max(ranges) / min(ranges) > 1.6, ranges


def _queue_tiles(nt, R, counts_by_entry):
    """Visible tiles each queue (XCD) runs for one mask batch whose work-order
    entry e has counts_by_entry[e] tiles, R heads."""
    f, grid = item_order(1, nt, 1, R)
    work = [0] * QUEUES
    for wg in range(grid):
        k = item(f, wg % QUEUES, wg // QUEUES)
        if k < f["nitems"]:
            e, _ = decode(f, k)
            work[wg % QUEUES] += counts_by_entry[e]
    return work


@pytest.mark.parametrize("nt,R", [(512, 6), (512, 1), (128, 3), (64, 64)])
def test_queues_share_causal_rows_evenly(nt, R):
    """Causal rows sorted longest first (entry e has nt - e tiles): the
    alternating rounds give every queue the same tiles within 1%; dealing
    every round in the same direction gave the first queue up to 1.56x the
    last one's."""
    work = _queue_tiles(nt, R, [nt - e for e in range(nt)])
    assert max(work) / min(work) < 1.01, work
