"""Host emulation of the attention kernels' item order (CPU only): the grid
size, the queue / grab arithmetic and the decode of an item into (work-order
entry, head index), written out exactly as the forward and dQ kernels
compute them (including the division by magic numbers), one item per
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
    k = ((queue + QUEUES * (i >> cl)) << cl) + (i & ((1 << cl) - 1))
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
