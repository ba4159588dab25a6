"""Tile classification and tile lists.  Oracle; test infrastructure only.

Follows:
  * speedrun notes "FlexAttention", tile-summary paragraph: the mask is
    summarised at 128 x 128 tiles; for every row of query tiles the summary
    holds how many tiles are not fully masked and their column indices;
  * tutorial "FlexAttention in PyTorch", section "The two hooks": each block
    is entirely empty, partially masked or full; empty blocks are never
    scheduled, only partial blocks need the elementwise mask.

  * same tutorial, "What to expect, and the sharp edges", item 4: the block
    size is a tunable (128 x 128 by default); smaller blocks capture more
    sparsity.  Here the key-block width of the row lists may be 64 (blocks
    of 128 queries x 64 keys).

Readings taken where the pages are silent:
  * classes come from the exact number of visible pairs in the block
    (0 -> empty, all of its tile_q x tile_k pairs -> full, otherwise
    partial), so a block at the end of a length that is not a multiple of
    its size is never full;
  * with 64-key blocks the row lists (what the forward visits) are at
    128 x 64; the column lists stay at 128 x 128 tiles;
  * partial and full tiles are listed separately, each in ascending column
    order, padded with -1 after the count; counts are int32;
  * for the backward pass the same lists are also given per key tile
    (ascending query-tile order), the transposed view of the same classes.

The counts come from the brute-force C counter in c/tile_counts.c (every pair
evaluated); tile_counts_dense_numpy is an independent numpy path over a dense
[T, T] boolean mask for small T.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .predicate import visible

TILE = 128
EMPTY, PARTIAL, FULL = 0, 1, 2


def kv_block(spec) -> int:
    """Key-block width of the spec's row lists (128 by default)."""
    return int(getattr(spec, "kv_block", TILE) or TILE)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "c", "liboracle_tiles.so")
_lib = None


def build_c(force: bool = False) -> str:
    """Compile the brute-force counter (gcc, OpenMP)."""
    import subprocess
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["make", "-B" if force else "-s", "-C", os.path.join(_HERE, "c")],
                       check=True, stdout=subprocess.DEVNULL)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        src = os.path.join(os.path.dirname(_LIB_PATH), "tile_counts.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            build_c(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_tile_counts.restype = ctypes.c_int
        lib.oracle_tile_counts.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        _lib = lib
    return _lib


def _flags(spec) -> int:
    f = 0
    if spec.causal:
        f |= 1
    if spec.document:
        f |= 2
    if spec.window is not None:
        f |= 4
    if spec.sinks:
        f |= 8
    if getattr(spec, "prefix", 0):
        f |= 16
    if getattr(spec, "table", None) is not None:
        f |= 32
    return f


def _q_len(spec):
    q = getattr(spec, "q_len", None)
    return spec.T if q is None else int(q)


def tile_counts(spec, tile_q: int = TILE, tile_k: int = TILE) -> np.ndarray:
    """int32 [mask_b, ceil(Q_LEN/tile_q), ceil(KV_LEN/tile_k)]: visible pairs
    per block (brute force)."""
    kv_len, q_len, q_off = spec.T, _q_len(spec), int(getattr(spec, "q_offset", 0))
    mb = spec.mask_b
    nq, nk = -(-q_len // tile_q), -(-kv_len // tile_k)
    out = np.zeros((mb, nq, nk), dtype=np.int32)
    docs, npos = None, max(kv_len, q_off + q_len)
    if spec.document:
        docs = np.ascontiguousarray(spec.doc_ids, dtype=np.int32)
        if docs.shape[1] < npos:
            raise ValueError(f"doc_ids cover {docs.shape[1]} positions, need {npos}")
        npos = docs.shape[1]
    rc = _load().oracle_tile_counts(
        kv_len, q_len, q_off, mb, _flags(spec),
        docs.ctypes.data if docs is not None else None, npos,
        int(spec.window) if spec.window is not None else 0,
        int(spec.sinks), int(getattr(spec, "prefix", 0)),
        int(getattr(spec, "table", None) or 0) & 0xFFFFFFFF, int(tile_q), int(tile_k), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_tile_counts rejected the spec")
    return out


def tile_counts_dense_numpy(spec, tile_q: int = TILE, tile_k: int = TILE) -> np.ndarray:
    """Same counts from a dense [Q_LEN, KV_LEN] boolean mask, padded with
    False to whole blocks (small sizes only)."""
    kv_len, q_len = spec.T, _q_len(spec)
    nq, nk = -(-q_len // tile_q), -(-kv_len // tile_k)
    res = []
    for b in range(spec.mask_b):
        m = np.zeros((nq * tile_q, nk * tile_k), dtype=bool)
        m[:q_len, :kv_len] = visible(spec, b, np.arange(q_len)[:, None], np.arange(kv_len)[None, :])
        res.append(m.reshape(nq, tile_q, nk, tile_k).sum(axis=(1, 3)).astype(np.int32))
    return np.stack(res)


def classify(counts: np.ndarray, tile_q: int = TILE, tile_k: int = TILE) -> np.ndarray:
    """uint8 class per block of tile_q x tile_k pairs: 0 empty, 1 partial,
    2 full."""
    cls = np.full(counts.shape, PARTIAL, dtype=np.uint8)
    cls[counts == 0] = EMPTY
    cls[counts == tile_q * tile_k] = FULL
    return cls


def _lists(cls2d: np.ndarray, want: int):
    """Per row of cls2d: count of tiles of class `want` and their ascending
    column indices, padded with -1."""
    n_rows, n_cols = cls2d.shape
    num = np.zeros(n_rows, dtype=np.int32)
    idx = np.full((n_rows, n_cols), -1, dtype=np.int32)
    for r in range(n_rows):
        cols = np.nonzero(cls2d[r] == want)[0]
        num[r] = len(cols)
        idx[r, :len(cols)] = cols
    return num, idx


def block_mask_lists(counts: np.ndarray, row_counts: np.ndarray = None, row_tile_k: int = TILE) -> dict:
    """The eight tile-list arrays of a block mask, shaped [mask_b, 1, ...]
    (head dim 1: one mask shared by all heads).  counts: 128 x 128 tile
    counts; row_counts (optional): counts at 128 x row_tile_k blocks for the
    row lists (the column lists always come from counts)."""
    cls = classify(counts)
    row_cls = cls if row_counts is None else classify(row_counts, TILE, row_tile_k)
    names = {}
    out = {k: [] for k in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                           "full_kv_indices", "q_num_blocks", "q_indices",
                           "full_q_num_blocks", "full_q_indices")}
    for b in range(cls.shape[0]):
        c = cls[b]
        n, i = _lists(row_cls[b], PARTIAL)
        out["kv_num_blocks"].append(n)
        out["kv_indices"].append(i)
        n, i = _lists(row_cls[b], FULL)
        out["full_kv_num_blocks"].append(n)
        out["full_kv_indices"].append(i)
        n, i = _lists(c.T, PARTIAL)
        out["q_num_blocks"].append(n)
        out["q_indices"].append(i)
        n, i = _lists(c.T, FULL)
        out["full_q_num_blocks"].append(n)
        out["full_q_indices"].append(i)
    for k, v in out.items():
        names[k] = np.stack(v)[:, None]
    return names


def spec_block_mask_lists(spec) -> dict:
    """The eight arrays of the spec's block mask: row lists at the spec's
    key-block width, column lists at 128 x 128."""
    kb = kv_block(spec)
    counts = tile_counts(spec)
    if kb == TILE:
        return block_mask_lists(counts)
    return block_mask_lists(counts, tile_counts(spec, TILE, kb), kb)
