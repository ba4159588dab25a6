"""Tile classification and tile lists.  Oracle; test infrastructure only.

Follows:
  * speedrun notes "FlexAttention", tile-summary paragraph: the mask is
    summarised at 128 x 128 tiles; for every row of query tiles the summary
    holds how many tiles are not fully masked and their column indices;
  * tutorial "FlexAttention in PyTorch", section "The two hooks": each block
    is entirely empty, partially masked or full; empty blocks are never
    scheduled, only partial blocks need the elementwise mask.

Readings taken where the pages are silent:
  * classes come from the exact number of visible pairs in the tile
    (0 -> empty, 128*128 -> full, otherwise partial);
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
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
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
    if spec.causal and getattr(spec, "prefix", 0):
        f |= 16
    return f


def tile_counts(spec) -> np.ndarray:
    """int32 [mask_b, T/128, T/128]: visible pairs per tile (brute force)."""
    T = spec.T
    if T % TILE:
        raise ValueError("T must be a multiple of 128")
    mb = spec.mask_b
    nt = T // TILE
    out = np.zeros((mb, nt, nt), dtype=np.int32)
    docs = None
    if spec.document:
        docs = np.ascontiguousarray(spec.doc_ids, dtype=np.int32)
    rc = _load().oracle_tile_counts(
        T, mb, _flags(spec),
        docs.ctypes.data if docs is not None else None,
        int(spec.window) if spec.window is not None else 0,
        int(spec.sinks), int(getattr(spec, "prefix", 0)), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_tile_counts rejected the spec")
    return out


def tile_counts_dense_numpy(spec) -> np.ndarray:
    """Same counts from a dense [T, T] boolean mask (small T only)."""
    T = spec.T
    nt = T // TILE
    ar = np.arange(T)
    res = []
    for b in range(spec.mask_b):
        m = visible(spec, b, ar[:, None], ar[None, :])
        res.append(m.reshape(nt, TILE, nt, TILE).sum(axis=(1, 3)).astype(np.int32))
    return np.stack(res)


def classify(counts: np.ndarray) -> np.ndarray:
    """uint8 class per tile: 0 empty, 1 partial, 2 full."""
    cls = np.full(counts.shape, PARTIAL, dtype=np.uint8)
    cls[counts == 0] = EMPTY
    cls[counts == TILE * TILE] = FULL
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


def block_mask_lists(counts: np.ndarray) -> dict:
    """The eight tile-list arrays of a block mask, shaped [mask_b, 1, ...]
    (head dim 1: one mask shared by all heads)."""
    cls = classify(counts)
    names = {}
    out = {k: [] for k in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                           "full_kv_indices", "q_num_blocks", "q_indices",
                           "full_q_num_blocks", "full_q_indices")}
    for b in range(cls.shape[0]):
        c = cls[b]
        n, i = _lists(c, PARTIAL)
        out["kv_num_blocks"].append(n)
        out["kv_indices"].append(i)
        n, i = _lists(c, FULL)
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
