"""Python binding of the block-sparse masked attention library.

Argument marshalling only: every step runs in the HIP kernels of libbsm.so.
PyTorch provides device memory and the current stream.

    spec = mask_spec(T, causal=True, doc_ids=docs, window=1024)
    bm   = build_block_mask(spec)                     # once per mask
    out, lse = flex_attention_fwd(q, k, v, bm, spec, score_mod)
    dq, dk, dv = flex_attention_bwd(q, k, v, out, lse, dout, bm, spec, score_mod)

Queries and keys may differ in number: mask_spec(KV_LEN, q_len=Q_LEN,
q_offset=o) puts query i at absolute position o + i (the last Q_LEN positions
of a cache when o = KV_LEN - Q_LEN).  Masks composed with and_masks /
or_masks / ~ over the terms CAUSAL, SAME_DOC, IN_WINDOW, SINK and PREFIX are
passed as mask_spec(..., composed=expr).
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
                   BSM_MASK_TABLE, BSM_MOD_ALIBI, BSM_MOD_SOFTCAP, BSM_MOD_BIAS)

TILE = 128


class MaskTerm:
    """A boolean function of the five mask terms -- causal (q >= kv), same
    document, in window (q - kv < window), sink (kv < sinks), prefix
    (kv < prefix) -- held as its 32-entry truth table: bit
    (C + 2 Dc + 4 W + 8 S + 16 P) is the value when those terms hold.
    Combined with & (and_masks), | (or_masks) and ~ (tutorial "FlexAttention
    in PyTorch", Pattern 3)."""

    __slots__ = ("table",)

    def __init__(self, table: int):
        self.table = int(table) & 0xFFFFFFFF

    def __and__(self, other: "MaskTerm") -> "MaskTerm":
        return MaskTerm(self.table & other.table)

    def __or__(self, other: "MaskTerm") -> "MaskTerm":
        return MaskTerm(self.table | other.table)

    def __invert__(self) -> "MaskTerm":
        return MaskTerm(~self.table)

    def __eq__(self, other) -> bool:
        return isinstance(other, MaskTerm) and other.table == self.table

    def __hash__(self) -> int:
        return hash(self.table)

    def __repr__(self) -> str:
        return f"MaskTerm(0x{self.table:08X})"


CAUSAL = MaskTerm(0xAAAAAAAA)
SAME_DOC = MaskTerm(0xCCCCCCCC)
IN_WINDOW = MaskTerm(0xF0F0F0F0)
SINK = MaskTerm(0xFF00FF00)
PREFIX = MaskTerm(0xFFFF0000)
ALL = MaskTerm(0xFFFFFFFF)
NONE = MaskTerm(0)


def and_masks(*terms: MaskTerm) -> MaskTerm:
    out = ALL
    for t in terms:
        out = out & t
    return out


def or_masks(*terms: MaskTerm) -> MaskTerm:
    out = NONE
    for t in terms:
        out = out | t
    return out


def _ptr(t: torch.Tensor, name: str) -> int:
    """Device address of a tensor the kernels read or write: it must live on
    the current GPU (a host or other-device address would be read by the
    kernels as if it were theirs)."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on the GPU, got "
                         f"{t.device if isinstance(t, torch.Tensor) else type(t).__name__}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


@dataclasses.dataclass
class MaskSpec:
    """Device-side mask description.  `window` is a device int32 tensor of
    one element so it can change between calls without touching the host.
    T is KV_LEN; Q_LEN = q_len (0: T) queries sit at absolute positions
    q_offset + i."""
    T: int
    causal: bool = True
    doc_ids: Optional[torch.Tensor] = None   # int32 [mask_b, positions] on the device
    window: Optional[torch.Tensor] = None    # int32 [1] on the device
    sinks: int = 0
    prefix: int = 0                          # prefix-LM: keys < prefix seen by every query
    q_len: int = 0
    q_offset: int = 0
    composed: Optional[MaskTerm] = None      # replaces the standard combination of the terms
    kv_block: int = 128                      # key-block width of the row lists: 128 or 64

    @property
    def Q(self) -> int:
        return self.q_len if self.q_len else self.T

    @property
    def positions(self) -> int:
        return max(self.T, self.q_offset + self.Q)

    @property
    def QT(self) -> int:
        return -(-self.Q // TILE)

    @property
    def KT(self) -> int:
        return -(-self.T // TILE)

    @property
    def KB(self) -> int:
        """Key blocks of the row lists."""
        return -(-self.T // self.kv_block)

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
        if self.sinks and (self.window is not None or self.composed is not None):
            f |= BSM_MASK_SINKS
        if self.composed is not None:
            f |= BSM_MASK_TABLE
        return f

    def c_struct(self) -> BsmMaskSpec:
        return BsmMaskSpec(self.flags, self.T, self.mask_b,
                           _ptr(self.doc_ids, "doc_ids") if self.doc_ids is not None else None,
                           _ptr(self.window, "window") if self.window is not None else None,
                           int(self.sinks), int(self.prefix), int(self.q_len), int(self.q_offset),
                           self.composed.table if self.composed is not None else 0, int(self.kv_block))

    def set_window(self, w: int) -> None:
        """Writes a new window value on the device (stream-ordered)."""
        self.window.fill_(int(w))


@dataclasses.dataclass
class ScoreMod:
    alibi_slopes: Optional[torch.Tensor] = None  # float32 [H] on the device
    softcap: Optional[float] = None
    bias: Optional[torch.Tensor] = None          # float32 [H, 2R + 1] on the device: relative-position bias

    @property
    def bias_radius(self) -> int:
        return (self.bias.shape[-1] - 1) // 2 if self.bias is not None else 0

    def c_struct(self) -> BsmScoreMod:
        f = 0
        if self.alibi_slopes is not None:
            f |= BSM_MOD_ALIBI
        if self.softcap is not None:
            f |= BSM_MOD_SOFTCAP
        if self.bias is not None:
            f |= BSM_MOD_BIAS
        return BsmScoreMod(f, _ptr(self.alibi_slopes, "alibi_slopes") if self.alibi_slopes is not None else None,
                           float(self.softcap) if self.softcap is not None else 0.0, None,
                           _ptr(self.bias, "bias") if self.bias is not None else None, self.bias_radius, None)


class BlockMask(NamedTuple):
    kv_num_blocks: torch.Tensor
    kv_indices: torch.Tensor
    full_kv_num_blocks: torch.Tensor
    full_kv_indices: torch.Tensor
    q_num_blocks: torch.Tensor
    q_indices: torch.Tensor
    full_q_num_blocks: torch.Tensor
    full_q_indices: torch.Tensor
    doc_range: torch.Tensor   # int32 [mask_b, positions, 2]: (first, last) position of each position's document
    kv_order: torch.Tensor    # int32 [mask_b * QT, 4]: rows, most tiles first (row, full, partial, first tile)
    q_order: torch.Tensor     # int32 [mask_b * KT, 4]: columns, most tiles first (same layout)

    def c_struct(self) -> BsmBlockMask:
        return BsmBlockMask(*[_ptr(t, n) for n, t in zip(self._fields, self)])

    def visible_tiles(self) -> int:
        """Non-empty tiles (partial + full) over the mask batch."""
        return int(self.kv_num_blocks.sum().item() + self.full_kv_num_blocks.sum().item())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def mask_spec(T: int, causal: bool = True, doc_ids=None, window: Optional[int] = None,
              sinks: int = 0, device="cuda", prefix: int = 0, q_len: int = 0, q_offset: int = 0,
              composed: Optional[MaskTerm] = None, kv_block: int = 128) -> MaskSpec:
    """Device mask spec from host values (numpy / torch / int).  T is KV_LEN;
    doc_ids has one id per absolute position (max(T, q_offset + Q_LEN))."""
    d = None
    if doc_ids is not None:
        d = torch.as_tensor(np.asarray(doc_ids), dtype=torch.int32)
        if d.dim() == 1:
            d = d[None]
        d = d.to(device).contiguous()
    w = None
    if window is not None:
        w = torch.tensor([int(window)], dtype=torch.int32, device=device)
    if composed is not None and not isinstance(composed, MaskTerm):
        composed = MaskTerm(composed)
    if kv_block not in (64, 128):
        raise ValueError(f"kv_block must be 64 or 128, got {kv_block}")
    return MaskSpec(int(T), bool(causal), d, w, int(sinks), int(prefix), int(q_len), int(q_offset), composed,
                    int(kv_block))


def from_spec_data(spec_data, device="cuda") -> MaskSpec:
    """Device mask spec from a workloads.MaskSpecData."""
    table = getattr(spec_data, "table", None)
    q_len = getattr(spec_data, "q_len", None)
    return mask_spec(spec_data.T, spec_data.causal,
                     spec_data.doc_ids if spec_data.document else None,
                     spec_data.window, spec_data.sinks, device, getattr(spec_data, "prefix", 0),
                     q_len=int(q_len) if q_len else 0, q_offset=int(getattr(spec_data, "q_offset", 0)),
                     composed=MaskTerm(table) if table is not None else None,
                     kv_block=int(getattr(spec_data, "kv_block", 128)))


def score_mod(alibi_slopes=None, softcap: Optional[float] = None, device="cuda", bias=None) -> ScoreMod:
    """Score modifications: ALiBi slopes [H], a soft-cap value, and a
    relative-position bias table [H, 2R + 1] (entry R + d for the distance
    q - kv = d, distances beyond R clipped)."""
    s = None
    if alibi_slopes is not None:
        s = torch.as_tensor(np.asarray(alibi_slopes), dtype=torch.float32).to(device).contiguous()
    t = None
    if bias is not None:
        t = torch.as_tensor(np.asarray(bias) if not isinstance(bias, torch.Tensor) else bias,
                            dtype=torch.float32).to(device).contiguous()
    return ScoreMod(s, softcap, t)


def empty_block_mask(spec, mask_b: Optional[int] = None, device="cuda") -> BlockMask:
    """Uninitialised block-mask arrays for a MaskSpec (or for a square mask
    of length T = spec and mask_b batch rows)."""
    if isinstance(spec, MaskSpec):
        Q, T, npos, kbw = spec.Q, spec.T, spec.positions, spec.kv_block
        mask_b = spec.mask_b if mask_b is None else mask_b
    else:
        Q = T = npos = int(spec)
        kbw = TILE
        mask_b = 1 if mask_b is None else mask_b
    qt, kt, nkb = -(-Q // TILE), -(-T // TILE), -(-T // kbw)
    mk = lambda *s: torch.empty(s, dtype=torch.int32, device=device)
    return BlockMask(mk(mask_b, 1, qt), mk(mask_b, 1, qt, nkb), mk(mask_b, 1, qt), mk(mask_b, 1, qt, nkb),
                     mk(mask_b, 1, kt), mk(mask_b, 1, kt, qt), mk(mask_b, 1, kt), mk(mask_b, 1, kt, qt),
                     mk(mask_b, npos, 2), mk(mask_b * qt, 4), mk(mask_b * kt, 4))


def block_mask_workspace(spec: MaskSpec) -> torch.Tensor:
    cs = spec.c_struct()
    n = lib.bsm_block_mask_workspace_bytes(ctypes.byref(cs))
    if n == 0:
        check(lib.bsm_build_block_mask(ctypes.byref(cs), None, None, 0, None))  # raises with the reason
    return torch.empty(max(n, 256), dtype=torch.uint8, device=spec.doc_ids.device
                       if spec.doc_ids is not None else "cuda")


def build_block_mask(spec: MaskSpec, out: Optional[BlockMask] = None,
                     workspace: Optional[torch.Tensor] = None) -> BlockMask:
    """Runs bsm_build_block_mask on the current stream."""
    if out is None:
        out = empty_block_mask(spec)
    if workspace is None:
        workspace = block_mask_workspace(spec)
    cs = spec.c_struct()
    cb = out.c_struct()
    check(lib.bsm_build_block_mask(ctypes.byref(cs), ctypes.byref(cb), _ptr(workspace, "workspace"),
                                   workspace.numel(), _stream()))
    return out


_DTYPES = {torch.bfloat16: _lib.BSM_DTYPE_BF16, torch.float16: _lib.BSM_DTYPE_F16}


def _tensor(t: torch.Tensor, name: str) -> BsmTensor:
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, T, D]")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    sb, sh, st, _ = t.stride()
    return BsmTensor(_ptr(t, name), sb, sh, st, _DTYPES[t.dtype])


def flex_attention_fwd(q, k, v, block_mask: BlockMask, spec: MaskSpec,
                       mod: Optional[ScoreMod] = None, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """q [B, H, Q_LEN, D], k and v [B, H, KV_LEN, D].  Returns (out bf16
    [B, H, Q_LEN, D], lse float32 [B, H, Q_LEN])."""
    B, H, Q, D, T = _shapes(q, k, v, spec)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape:
        raise ValueError(f"out {tuple(out.shape)} must have the shape of q {tuple(q.shape)}")
    if lse is None:
        lse = torch.empty((B, H, Q), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Q):
        raise ValueError("lse must be a contiguous float32 [B, H, Q_LEN] tensor")
    _check_mod(mod, H)
    tq, tk, tv, to = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v"), _tensor(out, "out")
    cb = block_mask.c_struct()
    cs = spec.c_struct()
    cm = mod.c_struct() if mod is not None else None
    check(lib.bsm_flex_attention_fwd(
        B, H, T, D, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(cb),
        ctypes.byref(cs), ctypes.byref(cm) if cm is not None else None,
        float(scale) if scale is not None else 0.0, ctypes.byref(to), _ptr(lse, "lse"), _stream()))
    return out, lse


def _shapes(q, k, v, spec: MaskSpec):
    """(B, H, Q_LEN, D, KV_LEN) after checking q against Q_LEN and k, v
    against KV_LEN."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, length, D]")
    B, H, Q, D = q.shape
    T = k.shape[2]
    if k.shape != (B, H, T, D) or v.shape != k.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must be [B, H, KV_LEN, D] with B, H, D of q")
    if T != spec.T or Q != spec.Q:
        raise ValueError(f"q has {Q} queries and k {T} keys; the mask spec has Q_LEN {spec.Q}, KV_LEN {spec.T}")
    return B, H, Q, D, T


def bwd_workspace(B: int, H: int, Q: int, D: int, device="cuda", mod: Optional[ScoreMod] = None) -> torch.Tensor:
    """Workspace of the backward for Q = Q_LEN queries (and the score
    modifications mod: a bias table adds its gradient partials)."""
    if mod is None:
        n = lib.bsm_bwd_workspace_bytes(B, H, Q, D)
    else:
        cm = mod.c_struct()
        n = lib.bsm_bwd_workspace_bytes_mod(B, H, Q, D, ctypes.byref(cm))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def flex_attention_bwd(q, k, v, out, lse, dout, block_mask: BlockMask, spec: MaskSpec,
                       mod: Optional[ScoreMod] = None, scale: Optional[float] = None,
                       dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None,
                       dslopes: Optional[torch.Tensor] = None, dbias: Optional[torch.Tensor] = None):
    """Returns (dq bf16 [B, H, Q_LEN, D], dk and dv bf16 [B, H, KV_LEN, D]).
    With ALiBi, a float32 [H] device tensor passed as dslopes receives
    dL/dslope (summed over the batch); with a bias table, a float32
    [H, 2R + 1] device tensor passed as dbias receives dL/dbias."""
    B, H, Q, D, T = _shapes(q, k, v, spec)
    for name, x in (("out", out), ("dout", dout)):
        if x.shape != q.shape:
            raise ValueError(f"{name} {tuple(x.shape)} must have the shape of q {tuple(q.shape)}")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Q):
        raise ValueError("lse must be a contiguous float32 [B, H, Q_LEN] tensor")
    _check_mod(mod, H)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, x, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if x.shape != ref.shape:
            raise ValueError(f"{name} {tuple(x.shape)} must be {tuple(ref.shape)}")
    if workspace is None:
        workspace = bwd_workspace(B, H, Q, D, q.device, mod)
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
        cm.alibi_slopes_grad = _ptr(dslopes, "dslopes")
    if dbias is not None:
        if cm is None or mod.bias is None:
            raise ValueError("dbias needs a score_mod with a bias table")
        if dbias.dtype != torch.float32 or dbias.shape != mod.bias.shape or not dbias.is_contiguous():
            raise ValueError("dbias must be a contiguous float32 tensor shaped like the bias table")
        cm.bias_grad = _ptr(dbias, "dbias")
    check(lib.bsm_flex_attention_bwd(
        B, H, T, D, *[ctypes.byref(t) for t in ts[:4]], _ptr(lse, "lse"), ctypes.byref(ts[4]),
        ctypes.byref(cb), ctypes.byref(cs), ctypes.byref(cm) if cm is not None else None,
        float(scale) if scale is not None else 0.0, *[ctypes.byref(t) for t in ts[5:]],
        _ptr(workspace, "workspace"), workspace.numel(), _stream()))
    return dq, dk, dv


def _check_mod(mod: Optional[ScoreMod], H: int) -> None:
    """The slopes tensor the kernels read H entries of, and the bias table
    they read H rows of 2R + 1 entries of."""
    if mod is not None and mod.alibi_slopes is not None:
        sl = mod.alibi_slopes
        if sl.dtype != torch.float32 or not sl.is_contiguous() or sl.numel() < H:
            raise ValueError(f"alibi_slopes must be a contiguous float32 tensor of at least H={H} elements")
    if mod is not None and mod.bias is not None:
        t = mod.bias
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 2 or t.shape[0] < H or t.shape[1] % 2 != 1:
            raise ValueError(f"bias must be a contiguous float32 [H={H}, 2R + 1] tensor")


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
        B, H, capacity, D, _ptr(kvl, "kv_len"), stride, ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]),
        ctypes.byref(cs), ctypes.byref(cb) if cb is not None else None,
        ctypes.byref(cm) if cm is not None else None, float(scale) if scale is not None else 0.0,
        ctypes.byref(ts[3]), _ptr(lse, "lse"), _ptr(workspace, "workspace"), workspace.numel(), _stream()))
    return out, lse


def flex_attention_decode_paged(q, k_pages, v_pages, block_table, spec: MaskSpec,
                                mod: Optional[ScoreMod] = None, scale: Optional[float] = None, kv_len=None,
                                block_mask: Optional[BlockMask] = None, out=None, lse=None,
                                workspace: Optional[torch.Tensor] = None):
    """The decoding step of flex_attention_decode over a paged cache: k_pages,
    v_pages [num_pages, H, page_size, D] hold the pages of every sequence and
    block_table, a device int32 [B, n_logical] tensor, maps logical page j of
    batch element b to its physical page (key kv sits at row kv % page_size
    of page block_table[b, kv // page_size]).  The logical capacity is
    n_logical * page_size: spec, block_mask and kv_len refer to it.
    page_size is a positive multiple of 64.  Returns (out, lse) as
    flex_attention_decode, which gives the same bits on the gathered cache."""
    num_pages, H, page_size, D = k_pages.shape
    if v_pages.shape != k_pages.shape:
        raise ValueError(f"v_pages {tuple(v_pages.shape)} must have the shape of k_pages {tuple(k_pages.shape)}")
    if (block_table.dim() != 2 or block_table.dtype != torch.int32 or not block_table.is_contiguous()
            or block_table.device != q.device):
        raise ValueError("block_table must be a contiguous int32 [B, n_logical] tensor on q's device")
    B, n_logical = block_table.shape
    capacity = n_logical * page_size
    if q.shape != (B, H, 1, D):
        raise ValueError(f"q must be [B, H, 1, D] = {(B, H, 1, D)}, got {tuple(q.shape)}")
    if spec.T != capacity:
        raise ValueError(f"mask spec length {spec.T} != logical capacity {capacity}")
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
    ts = [_tensor(x, n) for x, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (out, "out"))]
    cs = spec.c_struct()
    cb = block_mask.c_struct() if block_mask is not None else None
    cm = mod.c_struct() if mod is not None else None
    check(lib.bsm_flex_attention_decode_paged(
        B, H, D, page_size, num_pages, _ptr(block_table, "block_table"), n_logical, _ptr(kvl, "kv_len"), stride,
        ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]),
        ctypes.byref(cs), ctypes.byref(cb) if cb is not None else None,
        ctypes.byref(cm) if cm is not None else None, float(scale) if scale is not None else 0.0,
        ctypes.byref(ts[3]), _ptr(lse, "lse"), _ptr(workspace, "workspace"), workspace.numel(), _stream()))
    return out, lse


def gather_kv_pages(k_pages, v_pages, block_table, n_keys: int, k_out=None, v_out=None):
    """The first n_keys keys and values of every sequence of a paged cache
    (pools [num_pages, H, page_size, D], block_table int32 [B, n_logical] on
    the device) copied into contiguous [B, H, n_keys, D] tensors by the
    library's gather kernel.  Returns (k_out, v_out)."""
    num_pages, H, page_size, D = k_pages.shape
    if v_pages.shape != k_pages.shape:
        raise ValueError(f"v_pages {tuple(v_pages.shape)} must have the shape of k_pages {tuple(k_pages.shape)}")
    if block_table.dim() != 2 or block_table.dtype != torch.int32 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, n_logical] tensor")
    B, n_logical = block_table.shape
    if not 1 <= n_keys <= n_logical * page_size:
        raise ValueError(f"n_keys {n_keys} must be in [1, {n_logical * page_size}]")
    shape = (B, H, n_keys, D)
    k_out = torch.empty(shape, dtype=k_pages.dtype, device=k_pages.device) if k_out is None else k_out
    v_out = torch.empty(shape, dtype=v_pages.dtype, device=v_pages.device) if v_out is None else v_out
    if k_out.shape != shape or v_out.shape != shape:
        raise ValueError(f"k_out and v_out must be {shape}")
    ts = [_tensor(x, n) for x, n in ((k_pages, "k_pages"), (v_pages, "v_pages"), (k_out, "k_out"), (v_out, "v_out"))]
    check(lib.bsm_gather_kv_pages(B, H, D, page_size, num_pages, _ptr(block_table, "block_table"), n_logical,
                                  int(n_keys), *[ctypes.byref(t) for t in ts], _stream()))
    return k_out, v_out


def flex_attention_decode_multi_paged(q, k_pages, v_pages, block_table, spec: MaskSpec, kv_len: int,
                                      mod: Optional[ScoreMod] = None, scale: Optional[float] = None,
                                      step_spec: Optional[MaskSpec] = None,
                                      block_mask: Optional[BlockMask] = None, out=None, lse=None):
    """flex_attention_decode_multi over a paged cache (spec.T = the logical
    capacity n_logical * page_size): the live keys are gathered into
    contiguous rows (gather_kv_pages), then the rectangular forward runs over
    them.  Returns (out [B, H, n, D], lse [B, H, n])."""
    B, H, n, D = q.shape
    if k_pages.dim() != 4 or k_pages.shape[1] != H or k_pages.shape[3] != D or block_table.shape[0] != B:
        raise ValueError(f"k_pages [num_pages, H, page_size, D] and block_table [B, n_logical] must match q "
                         f"{tuple(q.shape)}")
    if spec.T != block_table.shape[1] * k_pages.shape[2]:
        raise ValueError(f"mask spec length {spec.T} != logical capacity {block_table.shape[1] * k_pages.shape[2]}")
    if step_spec is None:
        step_spec = decode_multi_spec(spec, kv_len, n)
    elif (step_spec.T, step_spec.Q, step_spec.q_offset) != (kv_len, n, kv_len - n):
        raise ValueError("step_spec was built for another live length or query count")
    if block_mask is None:
        block_mask = build_block_mask(step_spec)
    k, v = gather_kv_pages(k_pages, v_pages, block_table, kv_len)
    return flex_attention_fwd(q, k, v, block_mask, step_spec, mod, scale, out, lse)


def decode_multi_spec(spec: MaskSpec, kv_len: int, n: int) -> MaskSpec:
    """The mask of a block of n queries at positions kv_len - n .. kv_len - 1
    against the first kv_len positions of a cache described by spec (whose T
    is the cache capacity): KV_LEN = kv_len, Q_LEN = n, q_offset = kv_len - n.
    Document ids are restricted to the live positions (a copy when the mask
    batch has several rows)."""
    if not 1 <= n <= kv_len <= spec.T:
        raise ValueError(f"need 1 <= n={n} <= kv_len={kv_len} <= capacity={spec.T}")
    docs = spec.doc_ids[:, :kv_len].contiguous() if spec.doc_ids is not None else None
    return MaskSpec(int(kv_len), spec.causal, docs, spec.window, spec.sinks, spec.prefix, int(n),
                    int(kv_len - n), spec.composed, spec.kv_block)


def flex_attention_decode_multi(q, k, v, spec: MaskSpec, kv_len: int, mod: Optional[ScoreMod] = None,
                                scale: Optional[float] = None, step_spec: Optional[MaskSpec] = None,
                                block_mask: Optional[BlockMask] = None, out=None, lse=None):
    """A block of n = q.shape[2] new queries (speculative or chunked decoding)
    at positions kv_len - n .. kv_len - 1 of the cache k, v [B, H, capacity,
    D], on the matrix cores: the rectangular forward over the live keys
    (views of the cache, no copy).  kv_len is a host int here, since the
    block mask of the step is built for it: pass step_spec =
    decode_multi_spec(spec, kv_len, n) and its block mask to reuse them,
    otherwise both are built on this call.  Returns (out [B, H, n, D], lse
    [B, H, n])."""
    B, H, n, D = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"k, v must be [B, H, capacity, D] matching q {tuple(q.shape)}")
    if spec.T != k.shape[2]:
        raise ValueError(f"mask spec length {spec.T} != cache capacity {k.shape[2]}")
    if step_spec is None:
        step_spec = decode_multi_spec(spec, kv_len, n)
    elif (step_spec.T, step_spec.Q, step_spec.q_offset) != (kv_len, n, kv_len - n):
        raise ValueError("step_spec was built for another live length or query count")
    if block_mask is None:
        block_mask = build_block_mask(step_spec)
    return flex_attention_fwd(q, k[:, :, :kv_len], v[:, :, :kv_len], block_mask, step_spec, mod, scale, out, lse)


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
        B, H, capacity, D, _ptr(kvl, "kv_len"), stride, ctypes.byref(ts[0]), ctypes.byref(ts[1]), ctypes.byref(ts[2]),
        ctypes.byref(cs), ctypes.byref(cb) if cb is not None else None,
        ctypes.byref(cm) if cm is not None else None, float(scale) if scale is not None else 0.0,
        ctypes.byref(ts[3]), _ptr(lse, "lse"), _stream()))
    return out, lse


__all__ = ["MaskSpec", "MaskTerm", "CAUSAL", "SAME_DOC", "IN_WINDOW", "SINK", "PREFIX", "and_masks", "or_masks",
           "ScoreMod", "BlockMask", "mask_spec", "from_spec_data", "score_mod",
           "empty_block_mask", "build_block_mask", "flex_attention_fwd", "flex_attention_bwd",
           "flex_attention_decode", "decode_workspace", "flex_attention_decode_static",
           "flex_attention_decode_paged", "gather_kv_pages", "flex_attention_decode_multi_paged",
           "decode_multi_spec", "flex_attention_decode_multi",
           "bwd_workspace", "block_mask_workspace", "_lib"]
