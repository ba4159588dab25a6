"""Python binding of the block-sparse masked attention library.

Argument marshalling only: every step runs in the HIP kernels of libbsm.so.
PyTorch provides device memory and the current stream.

    spec = mask_spec(T, causal=True, doc_ids=docs, window=1024)
    bm   = build_block_mask(spec)                     # once per mask
    out, lse = flex_attention_fwd(q, k, v, bm, spec, score_mod)
    dq, dk, dv = flex_attention_bwd(q, k, v, out, lse, dout, bm, spec, score_mod)
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import NamedTuple, Optional

import numpy as np
import torch

from . import _lib
from ._lib import (BsmBlockMask, BsmMaskSpec, BsmScoreMod, BsmTensor, check, lib,
                   BSM_MASK_CAUSAL, BSM_MASK_DOCUMENT, BSM_MASK_WINDOW, BSM_MASK_SINKS, BSM_MASK_PREFIX,
                   BSM_MOD_ALIBI, BSM_MOD_SOFTCAP)

TILE = 128


@dataclasses.dataclass
class MaskSpec:
    """Device-side mask description.  `window` is a device int32 tensor of
    one element so it can change between calls without touching the host."""
    T: int
    causal: bool = True
    doc_ids: Optional[torch.Tensor] = None   # int32 [mask_b, T] on the device
    window: Optional[torch.Tensor] = None    # int32 [1] on the device
    sinks: int = 0
    prefix: int = 0                          # prefix-LM: keys < prefix seen by every query

    @property
    def mask_b(self) -> int:
        return 1 if self.doc_ids is None else int(self.doc_ids.shape[0])

    @property
    def flags(self) -> int:
        f = BSM_MASK_CAUSAL if self.causal else 0
        if self.prefix:
            f |= BSM_MASK_PREFIX
        if self.doc_ids is not None:
            f |= BSM_MASK_DOCUMENT
        if self.window is not None:
            f |= BSM_MASK_WINDOW
            if self.sinks:
                f |= BSM_MASK_SINKS
        return f

    def c_struct(self) -> BsmMaskSpec:
        return BsmMaskSpec(self.flags, self.T, self.mask_b,
                           self.doc_ids.data_ptr() if self.doc_ids is not None else None,
                           self.window.data_ptr() if self.window is not None else None,
                           int(self.sinks), int(self.prefix))

    def set_window(self, w: int) -> None:
        """Writes a new window value on the device (stream-ordered)."""
        self.window.fill_(int(w))


@dataclasses.dataclass
class ScoreMod:
    alibi_slopes: Optional[torch.Tensor] = None  # float32 [H] on the device
    softcap: Optional[float] = None

    def c_struct(self) -> BsmScoreMod:
        f = 0
        if self.alibi_slopes is not None:
            f |= BSM_MOD_ALIBI
        if self.softcap is not None:
            f |= BSM_MOD_SOFTCAP
        return BsmScoreMod(f, self.alibi_slopes.data_ptr() if self.alibi_slopes is not None else None,
                           float(self.softcap) if self.softcap is not None else 0.0, None)


class BlockMask(NamedTuple):
    kv_num_blocks: torch.Tensor
    kv_indices: torch.Tensor
    full_kv_num_blocks: torch.Tensor
    full_kv_indices: torch.Tensor
    q_num_blocks: torch.Tensor
    q_indices: torch.Tensor
    full_q_num_blocks: torch.Tensor
    full_q_indices: torch.Tensor
    doc_range: torch.Tensor   # int32 [mask_b, T, 2]: (first, last) position of each position's document
    kv_order: torch.Tensor    # int32 [mask_b * QT, 4]: rows, most tiles first (row, full, partial, first tile)
    q_order: torch.Tensor     # int32 [mask_b * KT, 4]: columns, most tiles first (same layout)

    def c_struct(self) -> BsmBlockMask:
        return BsmBlockMask(*[t.data_ptr() for t in self])

    def visible_tiles(self) -> int:
        """Non-empty tiles (partial + full) over the mask batch."""
        return int(self.kv_num_blocks.sum().item() + self.full_kv_num_blocks.sum().item())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def mask_spec(T: int, causal: bool = True, doc_ids=None, window: Optional[int] = None,
              sinks: int = 0, device="cuda", prefix: int = 0) -> MaskSpec:
    """Device mask spec from host values (numpy / torch / int)."""
    d = None
    if doc_ids is not None:
        d = torch.as_tensor(np.asarray(doc_ids), dtype=torch.int32)
        if d.dim() == 1:
            d = d[None]
        d = d.to(device).contiguous()
    w = None
    if window is not None:
        w = torch.tensor([int(window)], dtype=torch.int32, device=device)
    return MaskSpec(int(T), bool(causal), d, w, int(sinks), int(prefix))


def from_spec_data(spec_data, device="cuda") -> MaskSpec:
    """Device mask spec from a workloads.MaskSpecData."""
    return mask_spec(spec_data.T, spec_data.causal,
                     spec_data.doc_ids if spec_data.document else None,
                     spec_data.window, spec_data.sinks, device, getattr(spec_data, "prefix", 0))


def score_mod(alibi_slopes=None, softcap: Optional[float] = None, device="cuda") -> ScoreMod:
    s = None
    if alibi_slopes is not None:
        s = torch.as_tensor(np.asarray(alibi_slopes), dtype=torch.float32).to(device).contiguous()
    return ScoreMod(s, softcap)


def empty_block_mask(T: int, mask_b: int, device="cuda") -> BlockMask:
    nt = T // TILE
    mk = lambda *s: torch.empty(s, dtype=torch.int32, device=device)
    return BlockMask(mk(mask_b, 1, nt), mk(mask_b, 1, nt, nt), mk(mask_b, 1, nt), mk(mask_b, 1, nt, nt),
                     mk(mask_b, 1, nt), mk(mask_b, 1, nt, nt), mk(mask_b, 1, nt), mk(mask_b, 1, nt, nt),
                     mk(mask_b, T, 2), mk(mask_b * nt, 4), mk(mask_b * nt, 4))


def block_mask_workspace(spec: MaskSpec) -> torch.Tensor:
    n = lib.bsm_block_mask_workspace_bytes(spec.T, spec.mask_b)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=spec.doc_ids.device
                       if spec.doc_ids is not None else "cuda")


def build_block_mask(spec: MaskSpec, out: Optional[BlockMask] = None,
                     workspace: Optional[torch.Tensor] = None) -> BlockMask:
    """Runs bsm_build_block_mask on the current stream."""
    if out is None:
        out = empty_block_mask(spec.T, spec.mask_b)
    if workspace is None:
        workspace = block_mask_workspace(spec)
    cs = spec.c_struct()
    cb = out.c_struct()
    check(lib.bsm_build_block_mask(ctypes.byref(cs), ctypes.byref(cb), workspace.data_ptr(),
                                   workspace.numel(), _stream()))
    return out


def _tensor(t: torch.Tensor, name: str) -> BsmTensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, T, D]")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    sb, sh, st, _ = t.stride()
    return BsmTensor(t.data_ptr(), sb, sh, st)


def flex_attention_fwd(q, k, v, block_mask: BlockMask, spec: MaskSpec,
                       mod: Optional[ScoreMod] = None, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Returns (out bf16 [B,H,T,D], lse float32 [B,H,T])."""
    B, H, T, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape [B, H, T, D]")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, T):
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    _check_mod(mod, H)
    tq, tk, tv, to = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v"), _tensor(out, "out")
    cb = block_mask.c_struct()
    cs = spec.c_struct()
    cm = mod.c_struct() if mod is not None else None
    check(lib.bsm_flex_attention_fwd(
        B, H, T, D, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(cb),
        ctypes.byref(cs), ctypes.byref(cm) if cm is not None else None,
        float(scale) if scale is not None else 0.0, ctypes.byref(to), lse.data_ptr(), _stream()))
    return out, lse


def bwd_workspace(B: int, H: int, T: int, D: int, device="cuda") -> torch.Tensor:
    n = lib.bsm_bwd_workspace_bytes(B, H, T, D)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def flex_attention_bwd(q, k, v, out, lse, dout, block_mask: BlockMask, spec: MaskSpec,
                       mod: Optional[ScoreMod] = None, scale: Optional[float] = None,
                       dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None,
                       dslopes: Optional[torch.Tensor] = None):
    """Returns (dq, dk, dv), bf16 [B,H,T,D].  With ALiBi, a float32 [H]
    device tensor passed as dslopes receives dL/dslope (summed over the
    batch)."""
    B, H, T, D = q.shape
    for name, x in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if x.shape != q.shape:
            raise ValueError(f"{name} {tuple(x.shape)} must have the shape of q {tuple(q.shape)}")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, T):
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    _check_mod(mod, H)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = bwd_workspace(B, H, T, D, q.device)
    ts = [_tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"),
                                     (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    cb = block_mask.c_struct()
    cs = spec.c_struct()
    cm = mod.c_struct() if mod is not None else None
    if dslopes is not None:
        if cm is None or mod.alibi_slopes is None:
            raise ValueError("dslopes needs a score_mod with ALiBi slopes")
        if dslopes.dtype != torch.float32 or dslopes.numel() != H or not dslopes.is_contiguous():
            raise ValueError("dslopes must be a contiguous float32 tensor of H elements")
        cm.alibi_slopes_grad = dslopes.data_ptr()
    check(lib.bsm_flex_attention_bwd(
        B, H, T, D, *[ctypes.byref(t) for t in ts[:4]], lse.data_ptr(), ctypes.byref(ts[4]),
        ctypes.byref(cb), ctypes.byref(cs), ctypes.byref(cm) if cm is not None else None,
        float(scale) if scale is not None else 0.0, *[ctypes.byref(t) for t in ts[5:]],
        workspace.data_ptr(), workspace.numel(), _stream()))
    return dq, dk, dv


def _check_mod(mod: Optional[ScoreMod], H: int) -> None:
    """The slopes tensor the kernels read H entries of."""
    if mod is not None and mod.alibi_slopes is not None:
        sl = mod.alibi_slopes
        if sl.dtype != torch.float32 or not sl.is_contiguous() or sl.numel() < H:
            raise ValueError(f"alibi_slopes must be a contiguous float32 tensor of at least H={H} elements")


def _kv_len_tensor(kv_len, B: int, capacity: int, device) -> tuple:
    """(device int32 tensor, stride): one live length for the batch or one per
    batch element."""
    if kv_len is None:
        kv_len = capacity
    if isinstance(kv_len, int):
        if not 0 <= kv_len <= capacity:
            raise ValueError(f"kv_len {kv_len} must be in [0, capacity={capacity}]")
        kv_len = torch.tensor([kv_len], dtype=torch.int32, device=device)
    if not isinstance(kv_len, torch.Tensor) or kv_len.dtype != torch.int32 or not kv_len.is_contiguous():
        raise ValueError("kv_len must be an int or a contiguous int32 device tensor")
    if kv_len.numel() == 1:
        return kv_len, 0
    if kv_len.numel() == B:
        return kv_len, 1
    raise ValueError(f"kv_len must hold 1 or B={B} values, got {kv_len.numel()}")


def decode_workspace(B: int, H: int, capacity: int, D: int, device="cuda") -> torch.Tensor:
    n = lib.bsm_decode_workspace_bytes(B, H, capacity, D)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def flex_attention_decode(q, k, v, spec: MaskSpec, mod: Optional[ScoreMod] = None,
                          scale: Optional[float] = None, kv_len=None,
                          block_mask: Optional[BlockMask] = None, out=None, lse=None,
                          workspace: Optional[torch.Tensor] = None):
    """One decoding step: q [B, H, 1, D] at position kv_len - 1 against the
    cache k, v [B, H, capacity, D] of which the first kv_len positions are
    live.  kv_len: an int, or a device int32 tensor of 1 or B values (read
    by the kernels, so a captured step replays as the cache grows); default
    the whole capacity.  block_mask: optional mask of spec built once for the
    capacity; the step then reads only the key tiles its row lists.
    Returns (out [B, H, 1, D] bf16, lse [B, H] float32)."""
    B, H, capacity, D = k.shape
    if v.shape != k.shape:
        raise ValueError(f"v {tuple(v.shape)} must have the shape of k {tuple(k.shape)}")
    if q.shape != (B, H, 1, D):
        raise ValueError(f"q must be [B, H, 1, D] = {(B, H, 1, D)}, got {tuple(q.shape)}")
    if spec.T != capacity:
        raise ValueError(f"mask spec length {spec.T} != cache capacity {capacity}")
    _check_mod(mod, H)
    out = torch.empty_like(q) if out is None else out
    if out.shape != (B, H, 1, D):
        raise ValueError(f"out must be [B, H, 1, D] = {(B, H, 1, D)}")
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H):
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    kvl, stride = _kv_len_tensor(kv_len, B, capacity, q.device)
    if workspace is None:
        workspace = decode_workspace(B, H, capacity, D, q.device)
    ts = [_tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
    cs = spec.c_struct()
    cb = block_mask.c_struct() if block_mask is not None else None
    cm = mod.c_struct() if mod is not None else None
    check(lib.bsm_flex_attention_decode(
        B, H, capacity, D, kvl.data_ptr(), stride, ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]),
        ctypes.byref(cs), ctypes.byref(cb) if cb is not None else None,
        ctypes.byref(cm) if cm is not None else None, float(scale) if scale is not None else 0.0,
        ctypes.byref(ts[3]), lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()))
    return out, lse


def flex_attention_decode_static(q, k, v, spec: MaskSpec, mod: Optional[ScoreMod], scale: Optional[float],
                                 kv_len: torch.Tensor, block_mask: Optional[BlockMask], out: torch.Tensor,
                                 lse: torch.Tensor):
    """The decoding step of flex_attention_decode through the allocation-free
    entry point: nothing is allocated, here or in the library (its partials
    live in the library's static device scratch).  Every buffer is the
    caller's: kv_len a device int32 tensor of 1 or B values, out [B, H, 1, D]
    bf16, lse [B, H] float32.  Calls that overlap on one GPU race."""
    B, H, capacity, D = k.shape
    if v.shape != k.shape:
        raise ValueError(f"v {tuple(v.shape)} must have the shape of k {tuple(k.shape)}")
    if q.shape != (B, H, 1, D) or out.shape != (B, H, 1, D):
        raise ValueError(f"q and out must be [B, H, 1, D] = {(B, H, 1, D)}")
    if spec.T != capacity:
        raise ValueError(f"mask spec length {spec.T} != cache capacity {capacity}")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H):
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    if not isinstance(kv_len, torch.Tensor):
        raise ValueError("kv_len must be a device int32 tensor (the static entry point allocates nothing)")
    _check_mod(mod, H)
    kvl, stride = _kv_len_tensor(kv_len, B, capacity, q.device)
    ts = [_tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
    cs = spec.c_struct()
    cb = block_mask.c_struct() if block_mask is not None else None
    cm = mod.c_struct() if mod is not None else None
    check(lib.bsm_flex_attention_decode_static(
        B, H, capacity, D, kvl.data_ptr(), stride, ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]),
        ctypes.byref(cs), ctypes.byref(cb) if cb is not None else None,
        ctypes.byref(cm) if cm is not None else None, float(scale) if scale is not None else 0.0,
        ctypes.byref(ts[3]), lse.data_ptr(), _stream()))
    return out, lse


__all__ = ["MaskSpec", "ScoreMod", "BlockMask", "mask_spec", "from_spec_data", "score_mod",
           "empty_block_mask", "build_block_mask", "flex_attention_fwd", "flex_attention_bwd",
           "flex_attention_decode", "decode_workspace", "flex_attention_decode_static",
           "bwd_workspace", "block_mask_workspace", "_lib"]
