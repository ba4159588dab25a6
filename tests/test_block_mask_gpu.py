"""GPU parity of the block-mask builder: all eight integer arrays must equal
the oracle's bit for bit (counts, ascending indices, -1 padding)."""
import numpy as np
import pytest

from parity_utils import (assert_block_masks_equal, gpu_block_mask, log, needs_gpu,
                          oracle_block_mask)
from workloads import MaskSpecData, doc_ids_chunks, make_config

pytestmark = [pytest.mark.gpu, needs_gpu]


def _check(spec, ctx):
    log(f"[block-mask] {ctx} T={spec.T} mask_b={spec.mask_b}")
    _, _, g = gpu_block_mask(spec)
    assert_block_masks_equal(g, oracle_block_mask(spec), ctx, spec)
    return g


def _random_spec(rng, T):
    causal = bool(rng.integers(0, 4) > 0)
    docs = None
    if rng.integers(0, 3) > 0:
        mb = int(rng.integers(1, 3))
        if rng.integers(0, 4) == 0:  # arbitrary (non-monotone) ids: general path
            docs = rng.integers(0, 4, size=(mb, T)).astype(np.int32)
        else:
            docs = np.stack([np.cumsum(rng.random(T) < 1.0 / rng.integers(4, 400)).astype(np.int32)
                             for _ in range(mb)])
    window, sinks = None, 0
    if rng.integers(0, 3) > 0:
        window = int(rng.choice([-5, 0, 1, 2, 63, 64, 127, 128, 129, 255, 256, 300, 1000, 100000]))
        if rng.integers(0, 2):
            sinks = int(rng.choice([1, 4, 127, 128, 129, 500]))
    return MaskSpecData(T, causal=causal, document=docs is not None, doc_ids=docs,
                        window=window, sinks=sinks)


def test_random_small_specs():
    rng = np.random.default_rng(1234)
    for it in range(40):
        T = int(rng.choice([128, 256, 384, 1024, 1280, 2048]))
        _check(_random_spec(rng, T), f"random#{it}")


def test_many_mask_batches():
    """1030 mask batches of T = 1024 (one row block each): more blocks than
    the work-order kernel ranks directly, so its counting-sort path runs."""
    rng = np.random.default_rng(77)
    T, mb = 1024, 1030
    docs = np.stack([np.cumsum(rng.random(T) < 1.0 / rng.integers(4, 600)).astype(np.int32)
                     for _ in range(mb)])
    _check(MaskSpecData(T, causal=True, document=True, doc_ids=docs), "1030 batches")


def test_config1_tiny():
    _check(make_config(1).spec, "config 1")


def test_config2_and_variants_64k():
    g = _check(make_config(2).spec, "config 2")
    vis = int(g["kv_num_blocks"].sum() + g["full_kv_num_blocks"].sum())
    log(f"  config 2 visible tiles {vis}")
    expected = {"2-causal": 131328, "2-window": 4572, "2-chunks": 2304}
    for key, n in expected.items():
        g = _check(make_config(key).spec, f"config {key}")
        assert int(g["kv_num_blocks"].sum() + g["full_kv_num_blocks"].sum()) == n


def test_config3_window_sweep_all_28():
    """Window in device memory, rebuilt at each of the 28 steps 64..1792."""
    from block_sparse_masked_build_amd import api
    w = make_config(3)
    spec_dev = api.from_spec_data(w.spec)
    bm = api.empty_block_mask(w.T, 1)
    ws = api.block_mask_workspace(spec_dev)
    import torch
    for win in w.windows:
        spec_dev.set_window(win)
        api.build_block_mask(spec_dev, out=bm, workspace=ws)
        torch.cuda.synchronize()
        g = {n: getattr(bm, n).cpu().numpy() for n in bm._fields}
        s = MaskSpecData(w.T, causal=True, document=True, doc_ids=w.spec.doc_ids, window=win)
        if win != w.windows[0]:
            g.pop("doc_range")  # checked once; it does not depend on the window
        log(f"[block-mask] config 3 window {win}")
        assert_block_masks_equal(g, oracle_block_mask(s), f"window {win}", s)


def test_config4_and_5():
    _check(make_config("4a").spec, "config 4a")
    _check(make_config("4b").spec, "config 4b")
    _check(make_config(5).spec, "config 5 (mask_b = 2)")


def test_max_tile_grid_property():
    """Largest grid exercised: T = 262,144 (2048 x 2048 tiles), chunks of
    1000 (not aligned to tiles) plus a window; checked against the
    brute-force oracle on the row and column totals and on sampled rows."""
    T = 262144
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=doc_ids_chunks(T, 1000)[None],
                        window=3000)
    log(f"[block-mask] max grid T={T}")
    _, _, g = gpu_block_mask(spec)
    ref = oracle_block_mask(spec)
    assert_block_masks_equal(g, ref, "T=262144", spec)
