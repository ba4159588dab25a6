"""Property checks of the scheduling data the block-mask builder exports
beside the tile lists.  These arrays are a design choice of the HIP path, not
part of the method, so the oracle does not produce them; the tests check them
against their definitions, computed from the GPU's own tile lists (which are
themselves compared bit for bit with the oracle).

Work orders (kv_order over query-tile rows, q_order over key-tile columns):
  * records (row, full count, partial count, first listed tile), one per row
    of every mask batch, the rows a permutation of 0 .. mask_b * n - 1;
  * rows come in blocks of BLOCK consecutive rows of one mask batch (the last
    block of a batch may be shorter), each block one run, ascending inside;
  * the block key min(visible tiles of the block, KEY_CAP) never increases
    along the order, and equal keys keep ascending block order;
  * each record's counts and first tile equal the row's lists (first full
    tile if any, else first partial tile, else 0).

Document ranges: for a batch row of non-decreasing ids, entry t holds the
first and last position whose id equals id[t]; every entry of any other row
is (-1, -1).
"""
import numpy as np

BLOCK = 16
KEY_CAP = 8191


def check_work_order(order, num, idx, fnum, fidx, ctx=""):
    """order [mask_b * n, 4]; num / fnum [mask_b, 1, n]; idx / fidx
    [mask_b, 1, n, m] -- the GPU's partial and full lists for the same
    direction.  Raises AssertionError naming the first property that fails."""
    order = np.asarray(order)
    mask_b, n = num.shape[0], num.shape[-1]
    num = np.asarray(num).reshape(mask_b * n)
    fnum = np.asarray(fnum).reshape(mask_b * n)
    idx = np.asarray(idx).reshape(mask_b * n, -1)
    fidx = np.asarray(fidx).reshape(mask_b * n, -1)
    rows = order[:, 0].astype(np.int64)
    assert order.shape == (mask_b * n, 4), (ctx, order.shape)
    assert np.array_equal(np.sort(rows), np.arange(mask_b * n)), f"{ctx}: rows are not a permutation"
    bpb = (n + BLOCK - 1) // BLOCK
    blk = (rows // n) * bpb + (rows % n) // BLOCK
    # each block is one run of ascending consecutive rows covering the block
    starts = np.concatenate([[0], np.nonzero(blk[1:] != blk[:-1])[0] + 1])
    run_blocks = blk[starts]
    assert len(set(run_blocks.tolist())) == len(run_blocks), f"{ctx}: a block is split"
    for s, e in zip(starts, np.concatenate([starts[1:], [len(rows)]])):
        r = rows[s:e]
        b = blk[s]
        first = (b // bpb) * n + (b % bpb) * BLOCK
        size = min(BLOCK, n - (b % bpb) * BLOCK)
        assert np.array_equal(r, np.arange(first, first + size)), f"{ctx}: block {b} rows {r[:4]}.."
    tiles = num + fnum
    keys = np.array([min(int(tiles[rows[s:e]].sum()), KEY_CAP)
                     for s, e in zip(starts, np.concatenate([starts[1:], [len(rows)]]))])
    assert np.all(keys[:-1] >= keys[1:]), f"{ctx}: block keys increase"
    ties = keys[:-1] == keys[1:]
    assert np.all(run_blocks[:-1][ties] < run_blocks[1:][ties]), f"{ctx}: equal keys out of block order"
    assert np.array_equal(order[:, 1], fnum[rows]), f"{ctx}: full counts"
    assert np.array_equal(order[:, 2], num[rows]), f"{ctx}: partial counts"
    first = np.where(fnum[rows] > 0, fidx[rows, 0], np.where(num[rows] > 0, idx[rows, 0], 0))
    assert np.array_equal(order[:, 3], first), f"{ctx}: first listed tile"


def check_doc_range(doc_range, doc_ids, ctx=""):
    """doc_range [mask_b, N, 2] against doc_ids [mask_b, N]."""
    doc_range = np.asarray(doc_range)
    doc_ids = np.asarray(doc_ids, dtype=np.int64)
    assert doc_range.shape == doc_ids.shape + (2,), (ctx, doc_range.shape, doc_ids.shape)
    for b in range(doc_ids.shape[0]):
        d = doc_ids[b]
        if np.any(d[1:] < d[:-1]):
            assert np.all(doc_range[b] == -1), f"{ctx}: batch row {b} is not monotone but not flagged"
            continue
        # runs of equal ids: first and last position of each run
        t = np.arange(len(d))
        change = np.concatenate([[True], d[1:] != d[:-1]])
        run_id = np.cumsum(change) - 1
        run_first = t[change]
        run_last = np.concatenate([run_first[1:] - 1, [len(d) - 1]])
        assert np.array_equal(doc_range[b, :, 0], run_first[run_id]), f"{ctx}: batch row {b} starts"
        assert np.array_equal(doc_range[b, :, 1], run_last[run_id]), f"{ctx}: batch row {b} ends"


def check_schedule(gpu, doc_ids=None, ctx=""):
    """Both work orders and (with documents) the document ranges of one GPU
    block mask given as a dict of numpy arrays."""
    check_work_order(gpu["kv_order"], gpu["kv_num_blocks"], gpu["kv_indices"], gpu["full_kv_num_blocks"],
                     gpu["full_kv_indices"], f"{ctx} kv_order")
    check_work_order(gpu["q_order"], gpu["q_num_blocks"], gpu["q_indices"], gpu["full_q_num_blocks"],
                     gpu["full_q_indices"], f"{ctx} q_order")
    if doc_ids is not None and "doc_range" in gpu:
        check_doc_range(gpu["doc_range"], doc_ids, f"{ctx} doc_range")
