"""The property checks of the exported scheduling data (work orders and
document ranges) accept hand-worked examples and reject planted mistakes
(CPU only)."""
import numpy as np
import pytest

import oracle
from schedule_checks import check_doc_range, check_work_order
from workloads import MaskSpecData, doc_ids_chunks


def _lists(spec):
    bm = oracle.block_mask_lists(oracle.tile_counts(spec))
    return bm


def test_causal_512_hand_worked():
    """Causal T = 512: rows hold 1, 2, 3, 4 tiles (one block, kept in
    order), columns 4, 3, 2, 1 (one block)."""
    bm = _lists(MaskSpecData(512, causal=True))
    kv = np.array([[0, 0, 1, 0], [1, 1, 1, 0], [2, 2, 1, 0], [3, 3, 1, 0]])
    q = np.array([[0, 3, 1, 1], [1, 2, 1, 2], [2, 1, 1, 3], [3, 0, 1, 3]])
    check_work_order(kv, bm["kv_num_blocks"], bm["kv_indices"], bm["full_kv_num_blocks"], bm["full_kv_indices"])
    check_work_order(q, bm["q_num_blocks"], bm["q_indices"], bm["full_q_num_blocks"], bm["full_q_indices"])


def _synthetic(tiles):
    """Lists with `tiles[r]` partial tiles 0..tiles[r]-1 in row r, no full."""
    tiles = np.asarray(tiles)
    n = tiles.size
    m = int(tiles.max())
    num = tiles.reshape(1, 1, n).astype(np.int32)
    idx = np.full((1, 1, n, max(m, 1)), -1, dtype=np.int32)
    for r, t in enumerate(tiles):
        idx[0, 0, r, :t] = np.arange(t)
    fnum = np.zeros_like(num)
    fidx = np.full_like(idx, -1)
    return num, idx, fnum, fidx


def _records(rows, tiles):
    return np.array([[r, 0, tiles[r], 0] for r in rows])


def test_blocks_ranked_longest_first():
    """40 rows: blocks 0-15 (16 tiles), 16-31 (32) and 32-39 (40, the short
    last block) go last, second and first."""
    tiles = [1] * 16 + [2] * 16 + [5] * 8
    lists = _synthetic(tiles)
    good = list(range(32, 40)) + list(range(16, 32)) + list(range(16))
    check_work_order(_records(good, tiles), *lists)


@pytest.mark.parametrize("mutation", ["swap_in_block", "swap_blocks", "count", "first", "duplicate"])
def test_planted_mistakes_are_rejected(mutation):
    tiles = [1] * 16 + [2] * 16 + [5] * 8
    lists = _synthetic(tiles)
    rows = list(range(32, 40)) + list(range(16, 32)) + list(range(16))
    rec = _records(rows, tiles)
    if mutation == "swap_in_block":
        rec[[0, 1]] = rec[[1, 0]]
    elif mutation == "swap_blocks":
        rec = np.concatenate([rec[8:24], rec[:8], rec[24:]])
    elif mutation == "count":
        rec[3, 2] += 1
    elif mutation == "first":
        rec[3, 3] = 1
    elif mutation == "duplicate":
        rec[5, 0] = rec[4, 0]
    with pytest.raises(AssertionError):
        check_work_order(rec, *lists)


def test_equal_keys_keep_block_order():
    tiles = [1] * 16 + [1] * 16
    lists = _synthetic(tiles)
    check_work_order(_records(list(range(32)), tiles), *lists)
    with pytest.raises(AssertionError):
        check_work_order(_records(list(range(16, 32)) + list(range(16)), tiles), *lists)


def test_doc_range_definition():
    """Fixed 1000-token chunks: position t lies in [1000 floor(t/1000),
    min(1000 floor(t/1000) + 999, T - 1)]; ids that go down mark every
    position of their batch row with (-1, -1)."""
    T = 2560
    docs = doc_ids_chunks(T, 1000)
    ids = np.stack([docs, docs[::-1].copy()])
    t = np.arange(T)
    start = 1000 * (t // 1000)
    good = np.full((2, T, 2), -1, dtype=np.int32)
    good[0, :, 0] = start
    good[0, :, 1] = np.minimum(start + 999, T - 1)
    check_doc_range(good, ids)
    bad = good.copy()
    bad[0, 1500, 1] -= 1
    with pytest.raises(AssertionError):
        check_doc_range(bad, ids)
    bad = good.copy()
    bad[1, 7] = (0, 5)
    with pytest.raises(AssertionError):
        check_doc_range(bad, ids)
