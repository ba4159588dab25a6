"""C ABI checks that need no GPU: the library loads, exports every function
include/bsm.h declares, and rejects bad arguments on the host before any
launch (the fake device pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from block_sparse_masked_build_amd import _lib
from block_sparse_masked_build_amd._lib import (BsmBlockMask, BsmMaskSpec, BsmScoreMod, BsmTensor,
                                                lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced: every call below fails host checks


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "bsm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsm_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_version():
    assert lib.bsm_version().decode().startswith("bsm ")


def _spec(**kw):
    d = dict(flags=1, seq_len=1024, mask_b=1, doc_ids=None, window=None, num_sinks=0)
    d.update(kw)
    return BsmMaskSpec(**d)


def _bm(null=None):
    v = [FAKE] * 11
    if null is not None:
        v[null] = None
    return BsmBlockMask(*v)


def _build(spec, bm=None, ws=FAKE, nbytes=1 << 30):
    bm = bm or _bm()
    return lib.bsm_build_block_mask(ctypes.byref(spec), ctypes.byref(bm), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(seq_len=0), _lib.BSM_E_INVALID),
    (dict(seq_len=-128), _lib.BSM_E_INVALID),
    (dict(q_len=-1), _lib.BSM_E_INVALID),
    (dict(q_offset=-1), _lib.BSM_E_INVALID),
    (dict(q_len=1 << 21, q_offset=(1 << 21) + 1), _lib.BSM_E_INVALID),  # last position past the maximum
    (dict(seq_len=(1 << 22) + 128), _lib.BSM_E_INVALID),
    (dict(mask_b=0), _lib.BSM_E_INVALID),
    (dict(flags=2), _lib.BSM_E_INVALID),          # DOCUMENT without doc_ids
    (dict(flags=4), _lib.BSM_E_INVALID),          # WINDOW without window
    (dict(flags=64), _lib.BSM_E_INVALID),         # unknown bit
    (dict(flags=32 | 2), _lib.BSM_E_INVALID),     # composed mask with the document term, no doc_ids
    (dict(kv_block=32), _lib.BSM_E_INVALID),      # block width other than 64 / 128
    (dict(flags=12, window=FAKE, num_sinks=-1), _lib.BSM_E_INVALID),
])
def test_build_rejects_bad_spec(kw, code):
    assert _build(_spec(**kw)) == code
    assert lib.bsm_last_error().decode() != ""


def test_build_rejects_null_outputs_and_small_workspace():
    for i in list(range(8)) + [9, 10]:  # tile lists and work orders
        assert _build(_spec(), _bm(null=i)) == _lib.BSM_E_INVALID
    # doc_range is required only with the document term
    assert _build(_spec(flags=3, doc_ids=FAKE), _bm(null=8)) == _lib.BSM_E_INVALID
    assert b"doc_range" in lib.bsm_last_error()
    need = lib.bsm_block_mask_workspace_bytes(ctypes.byref(_spec()))
    assert need >= 64  # 8x8 class bytes + flags
    assert _build(_spec(), ws=FAKE, nbytes=need - 1) == _lib.BSM_E_WORKSPACE
    assert _build(_spec(), ws=None, nbytes=need) == _lib.BSM_E_WORKSPACE
    assert _build(_spec(), ws=FAKE + 16, nbytes=need) == _lib.BSM_E_WORKSPACE
    assert b"workspace" in lib.bsm_last_error()


def _ws(**kw):
    return lib.bsm_block_mask_workspace_bytes(ctypes.byref(_spec(**kw)))


def test_workspace_sizes():
    assert _ws(seq_len=0) == 0
    assert lib.bsm_block_mask_workspace_bytes(None) == 0
    assert _ws(seq_len=100) >= 1                               # one ragged tile
    assert _ws(seq_len=65536) >= 512 * 512
    assert _ws(seq_len=65536, mask_b=2, flags=3, doc_ids=FAKE) >= 2 * 512 * 512
    # rectangular: class bytes for QT x KT tiles
    assert _ws(seq_len=65536, q_len=128) >= 512
    assert _ws(seq_len=65536, q_len=128) < _ws(seq_len=65536)
    assert _ws(seq_len=1000, q_len=300, q_offset=700) >= 3 * 8
    assert lib.bsm_bwd_workspace_bytes(2, 16, 16384, 128) >= 2 * (2 * 16 * 16384 * 4)  # Delta and L per row
    assert lib.bsm_bwd_workspace_bytes(1, 1, 1024, 96) == 0


def _t(ptr=FAKE, sb=8 * 1024 * 64, sh=1024 * 64, st=64, dtype=0):
    return BsmTensor(ptr, sb, sh, st, dtype)


def _fwd(B=1, H=1, T=1024, D=64, spec=None, mod=None, q=None, k=None, v=None, o=None, lse=FAKE,
         bm=None, scale=0.0):
    spec = spec or _spec()
    bm = bm or _bm()
    q, k, v, o = (x or _t() for x in (q, k, v, o))
    return lib.bsm_flex_attention_fwd(B, H, T, D, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                      ctypes.byref(bm), ctypes.byref(spec),
                                      ctypes.byref(mod) if mod is not None else None, scale,
                                      ctypes.byref(o), lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), _lib.BSM_E_UNSUPPORTED),
    (dict(D=192), _lib.BSM_E_UNSUPPORTED),
    (dict(T=0), _lib.BSM_E_INVALID),
    (dict(T=2048), _lib.BSM_E_INVALID),            # != spec seq_len
    (dict(B=0), _lib.BSM_E_INVALID),
    (dict(B=3, spec=_spec(flags=3, mask_b=2, doc_ids=FAKE)), _lib.BSM_E_INVALID),
    (dict(q=_t(ptr=FAKE + 8)), _lib.BSM_E_INVALID),  # misaligned
    (dict(k=_t(st=60)), _lib.BSM_E_INVALID),        # stride not a multiple of 8
    (dict(v=_t(ptr=0)), _lib.BSM_E_INVALID),
    (dict(k=_t(dtype=1)), _lib.BSM_E_INVALID),      # fp16 k with bf16 q, v, out
    (dict(q=_t(dtype=2), k=_t(dtype=2), v=_t(dtype=2), o=_t(dtype=2)), _lib.BSM_E_INVALID),  # unknown dtype
    (dict(lse=None), _lib.BSM_E_INVALID),
    (dict(bm=_bm(null=0)), _lib.BSM_E_INVALID),
    (dict(bm=_bm(null=9)), _lib.BSM_E_INVALID),     # work order
    (dict(mod=BsmScoreMod(1, None, 0.0)), _lib.BSM_E_INVALID),        # ALiBi without slopes
    (dict(mod=BsmScoreMod(2, None, 0.0)), _lib.BSM_E_INVALID),        # cap must be > 0
    (dict(mod=BsmScoreMod(2, None, float("inf"))), _lib.BSM_E_INVALID),
    (dict(mod=BsmScoreMod(8, None, 1.0)), _lib.BSM_E_INVALID),
    (dict(mod=BsmScoreMod(2, None, 1.0, FAKE)), _lib.BSM_E_INVALID),  # slope gradient without ALiBi
    (dict(scale=float("nan")), _lib.BSM_E_INVALID),
    (dict(spec=_spec(flags=1 | 16, prefix_len=-1)), _lib.BSM_E_INVALID),  # negative prefix
    (dict(spec=_spec(flags=64)), _lib.BSM_E_INVALID),                     # unknown mask flag
])
def test_fwd_rejects(kw, code):
    assert _fwd(**kw) == code
    assert lib.bsm_last_error().decode() != ""


def test_bwd_rejects_small_workspace_and_missing_transposed_lists():
    spec = _spec()
    t = _t()
    need = lib.bsm_bwd_workspace_bytes(1, 1, 1024, 64)

    def call(bm, ws, n):
        return lib.bsm_flex_attention_bwd(
            1, 1, 1024, 64, *([ctypes.byref(t)] * 4), FAKE, ctypes.byref(t), ctypes.byref(bm),
            ctypes.byref(spec), None, 0.0, *([ctypes.byref(t)] * 3), ws, n, None)

    assert need == 2 * 4096 + 256  # Delta and lse log2 e per query, one slope partial per query tile
    assert call(_bm(), FAKE, need - 4) == _lib.BSM_E_WORKSPACE
    assert call(_bm(), None, need) == _lib.BSM_E_WORKSPACE
    for i in range(4, 8):
        assert call(_bm(null=i), FAKE, need) == _lib.BSM_E_INVALID


def test_bwd_rejects_slope_gradient_without_alibi():
    spec = _spec()
    t = _t()
    need = lib.bsm_bwd_workspace_bytes(1, 1, 1024, 64)
    mod = BsmScoreMod(2, None, 30.0, FAKE)
    rc = lib.bsm_flex_attention_bwd(
        1, 1, 1024, 64, *([ctypes.byref(t)] * 4), FAKE, ctypes.byref(t), ctypes.byref(_bm()),
        ctypes.byref(spec), ctypes.byref(mod), 0.0, *([ctypes.byref(t)] * 3), FAKE, need, None)
    assert rc == _lib.BSM_E_INVALID
    assert "alibi_slopes_grad" in lib.bsm_last_error().decode()


def test_bias_table_checks_and_workspace():
    """Relative-position bias table: a table is required, its radius is at
    most BSM_BIAS_MAX_RADIUS, ALiBi and a table together are not built, a
    gradient output needs the table, and the backward workspace grows by one
    partial row of 2R + 1 floats per (batch, head, query tile)."""
    R = 100
    ok = BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, FAKE, R, None)
    assert _fwd(mod=BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, None, R, None)) == _lib.BSM_E_INVALID
    assert _fwd(mod=BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, FAKE, -1, None)) == _lib.BSM_E_UNSUPPORTED
    assert _fwd(mod=BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, FAKE, _lib.BSM_BIAS_MAX_RADIUS + 1,
                                None)) == _lib.BSM_E_UNSUPPORTED
    assert _fwd(mod=BsmScoreMod(_lib.BSM_MOD_BIAS | _lib.BSM_MOD_ALIBI, FAKE, 0.0, None, FAKE, R,
                                None)) == _lib.BSM_E_UNSUPPORTED
    assert _fwd(mod=BsmScoreMod(0, None, 0.0, None, None, 0, FAKE)) == _lib.BSM_E_INVALID  # gradient, no table
    assert "bias_grad" in lib.bsm_last_error().decode()
    base = lib.bsm_bwd_workspace_bytes(2, 3, 1000, 64)
    assert lib.bsm_bwd_workspace_bytes_mod(2, 3, 1000, 64, None) == base
    need = lib.bsm_bwd_workspace_bytes_mod(2, 3, 1000, 64, ctypes.byref(ok))
    part = 2 * 3 * 8 * (2 * R + 1) * 4  # 8 query tiles
    assert need == base + (part + 255) // 256 * 256
    bad = BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, None, R, None)
    assert lib.bsm_bwd_workspace_bytes_mod(2, 3, 1000, 64, ctypes.byref(bad)) == 0
    # the backward asks for the larger workspace
    spec = _spec()
    t = _t()
    small = lib.bsm_bwd_workspace_bytes(1, 1, 1024, 64)
    rc = lib.bsm_flex_attention_bwd(
        1, 1, 1024, 64, *([ctypes.byref(t)] * 4), FAKE, ctypes.byref(t), ctypes.byref(_bm()),
        ctypes.byref(spec), ctypes.byref(ok), 0.0, *([ctypes.byref(t)] * 3), FAKE, small, None)
    assert rc == _lib.BSM_E_WORKSPACE
    # a decoding step computes no gradient
    dmod = BsmScoreMod(_lib.BSM_MOD_BIAS, None, 0.0, None, FAKE, R, FAKE)
    rc = lib.bsm_flex_attention_decode(1, 1, 1024, 64, FAKE, 0, *([ctypes.byref(t)] * 3), ctypes.byref(spec), None,
                                       ctypes.byref(dmod), 0.0, ctypes.byref(t), FAKE, FAKE, 1 << 20, None)
    assert rc == _lib.BSM_E_INVALID and "bias_grad" in lib.bsm_last_error().decode()


def test_decode_rejects_bad_arguments():
    spec = _spec()
    t = _t()
    need = lib.bsm_decode_workspace_bytes(1, 1, 1024, 64)
    assert need == 512  # one slot of 8 tiles: (64 + 2) floats = 264 bytes, rounded up to a multiple of 256
    assert lib.bsm_decode_workspace_bytes(1, 1, 1000, 64) == 512  # any capacity
    assert lib.bsm_decode_workspace_bytes(2, 3, 1025, 128) == 6400  # 2 x 3 x 2 slots x 130 floats x 4 B, to 256

    def call(D=64, ws=FAKE, n=need, s=spec, lse=FAKE, kvl=FAKE, stride=0, cap=1024, bm=None):
        return lib.bsm_flex_attention_decode(1, 1, cap, D, kvl, stride, *([ctypes.byref(t)] * 3),
                                             ctypes.byref(s), ctypes.byref(bm) if bm is not None else None, None,
                                             0.0, ctypes.byref(t), lse, ws, n, None)

    assert call(D=96) == _lib.BSM_E_UNSUPPORTED
    assert call(n=need - 4) == _lib.BSM_E_WORKSPACE
    assert call(ws=None) == _lib.BSM_E_WORKSPACE
    assert call(lse=None) == _lib.BSM_E_INVALID
    assert call(kvl=None) == _lib.BSM_E_INVALID
    assert call(stride=2) == _lib.BSM_E_INVALID
    assert call(cap=0) == _lib.BSM_E_INVALID
    assert call(s=_spec(seq_len=2048)) == _lib.BSM_E_INVALID   # seq_len must equal the capacity
    assert call(bm=_bm(null=0)) == _lib.BSM_E_INVALID           # block mask row arrays
    # a capacity that is not a multiple of 128 is fine without a block mask
    # (fails only at the workspace check here), not with one
    assert call(cap=1000, s=_spec(seq_len=1000), ws=None) == _lib.BSM_E_WORKSPACE
    assert call(cap=1000, s=_spec(seq_len=1000), bm=_bm()) == _lib.BSM_E_INVALID
    # the decoding step reads block masks of 128-key blocks only
    assert call(s=_spec(kv_block=64), bm=_bm()) == _lib.BSM_E_UNSUPPORTED
    assert call(s=_spec(kv_block=64), ws=None) == _lib.BSM_E_WORKSPACE  # fine without a block mask
    # a workspace for 64-key blocks holds twice the class bytes
    assert lib.bsm_block_mask_workspace_bytes(ctypes.byref(_spec(seq_len=65536, kv_block=64))) >= 512 * 1024


def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_python_decode_checks_shapes_before_launch():
    """The binding rejects shapes the C ABI cannot see (CPU tensors: nothing
    reaches the library)."""
    import torch
    from block_sparse_masked_build_amd import api
    B, H, T, D = 2, 3, 256, 64
    k, v = _cpu((B, H, T, D)), _cpu((B, H, T, D))
    spec = api.MaskSpec(T)
    with pytest.raises(ValueError, match="q must be"):
        api.flex_attention_decode(_cpu((B, H, T, D)), k, v, spec)       # a full-length q
    with pytest.raises(ValueError, match="q must be"):
        api.flex_attention_decode(_cpu((B, H, 1, 32)), k, v, spec)      # smaller D
    with pytest.raises(ValueError, match="v "):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, _cpu((B, H, T - 128, D)), spec)
    with pytest.raises(ValueError, match="lse"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, v, spec, lse=_cpu((B, H + 1), torch.float32))
    with pytest.raises(ValueError, match="lse"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, v, spec, lse=_cpu((H, B), torch.float32).t())
    with pytest.raises(ValueError, match="alibi_slopes"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, v, spec,
                                  api.ScoreMod(alibi_slopes=_cpu((H - 1,), torch.float32)))
    with pytest.raises(ValueError, match="kv_len"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, v, spec, kv_len=T + 1)
    with pytest.raises(ValueError, match="kv_len"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), k, v, spec, kv_len=torch.ones(B + 1, dtype=torch.int32))


def test_python_fwd_bwd_check_slopes_and_lse():
    import torch
    from block_sparse_masked_build_amd import api
    B, H, T, D = 1, 4, 256, 64
    q = _cpu((B, H, T, D))
    spec = api.MaskSpec(T)
    bm = None
    short = api.ScoreMod(alibi_slopes=_cpu((H - 1,), torch.float32))
    with pytest.raises(ValueError, match="alibi_slopes"):
        api.flex_attention_fwd(q, q, q, bm, spec, short)
    lse = _cpu((B, H, T), torch.float32)
    with pytest.raises(ValueError, match="alibi_slopes"):
        api.flex_attention_bwd(q, q, q, q, lse, q, bm, spec, short)
    with pytest.raises(ValueError, match="lse"):
        api.flex_attention_bwd(q, q, q, q, _cpu((B, H, T), torch.bfloat16), q, bm, spec, None)
    with pytest.raises(ValueError, match="dout"):
        api.flex_attention_bwd(q, q, q, q, lse, _cpu((B, H, T, 32)), bm, spec, None)


def test_static_decode_rejects_oversize_on_the_host():
    """The allocation-free decoding entry point checks the size of its
    partials against the static scratch before touching the device."""
    assert lib.bsm_decode_static_max_bytes() == 16 << 20
    t = _t()
    spec = _spec(seq_len=32768)
    rc = lib.bsm_flex_attention_decode_static(64, 32, 32768, 128, FAKE, 0, *([ctypes.byref(t)] * 3),
                                              ctypes.byref(spec), None, None, 0.0, ctypes.byref(t), FAKE, None)
    assert rc == _lib.BSM_E_WORKSPACE
    assert b"static scratch" in lib.bsm_last_error()


def test_paged_decode_rejects_bad_arguments():
    """Host checks of the paged decoding step: page size, pool, table and
    capacity, then the decoding step's own checks on the logical capacity."""
    t = _t()
    spec = _spec(seq_len=1024)
    need = lib.bsm_decode_workspace_bytes(1, 1, 1024, 64)

    def call(page=256, pages=8, table=FAKE, tstride=4, s=spec, ws=FAKE, n=need, D=64):
        return lib.bsm_flex_attention_decode_paged(1, 1, D, page, pages, table, tstride, FAKE, 0,
                                                   *([ctypes.byref(t)] * 3), ctypes.byref(s), None, None, 0.0,
                                                   ctypes.byref(t), FAKE, ws, n, None)

    assert call(page=0) == _lib.BSM_E_INVALID
    assert call(page=96) == _lib.BSM_E_INVALID        # not a multiple of 64
    assert call(pages=0) == _lib.BSM_E_INVALID
    assert call(table=None) == _lib.BSM_E_INVALID
    assert call(tstride=0) == _lib.BSM_E_INVALID
    assert call(page=1 << 16, tstride=1 << 7) == _lib.BSM_E_INVALID  # capacity past 2^22
    assert call(s=_spec(seq_len=2048)) == _lib.BSM_E_INVALID          # spec must be the logical capacity
    assert call(D=96) == _lib.BSM_E_UNSUPPORTED
    assert call(n=need - 4) == _lib.BSM_E_WORKSPACE
    assert call(ws=None) == _lib.BSM_E_WORKSPACE
    assert call(page=64, tstride=16, ws=None) == _lib.BSM_E_WORKSPACE


def test_python_paged_decode_checks_shapes_before_launch():
    import torch
    from block_sparse_masked_build_amd import api
    B, H, P, D, npg = 2, 3, 128, 64, 5
    kp, vp = _cpu((npg, H, P, D)), _cpu((npg, H, P, D))
    table = torch.zeros((B, 4), dtype=torch.int32)
    spec = api.MaskSpec(4 * P)
    with pytest.raises(ValueError, match="v_pages"):
        api.flex_attention_decode_paged(_cpu((B, H, 1, D)), kp, _cpu((npg, H, 2 * P, D)), table, spec)
    with pytest.raises(ValueError, match="block_table"):
        api.flex_attention_decode_paged(_cpu((B, H, 1, D)), kp, vp, table.long(), spec)
    with pytest.raises(ValueError, match="q must be"):
        api.flex_attention_decode_paged(_cpu((B + 1, H, 1, D)), kp, vp, table, spec)
    with pytest.raises(ValueError, match="logical capacity"):
        api.flex_attention_decode_paged(_cpu((B, H, 1, D)), kp, vp, table, api.MaskSpec(3 * P))


def test_python_binding_rejects_host_tensors():
    """Every address handed to the library must be device memory: host
    tensors of the right shapes are refused before any call."""
    import torch
    from block_sparse_masked_build_amd import api
    B, H, T, D = 1, 2, 256, 64
    q = _cpu((B, H, T, D))
    spec = api.MaskSpec(T)
    with pytest.raises(ValueError, match="on the GPU"):
        api.flex_attention_fwd(q, q, q, None, spec, out=_cpu((B, H, T, D)),
                               lse=_cpu((B, H, T), torch.float32))
    with pytest.raises(ValueError, match="on the GPU"):
        api.flex_attention_decode(_cpu((B, H, 1, D)), q, q, spec)
    with pytest.raises(ValueError, match="on the GPU"):
        api.flex_attention_decode_paged(_cpu((B, H, 1, D)), q, q, torch.zeros((B, 1), dtype=torch.int32),
                                        api.MaskSpec(T))
    with pytest.raises(ValueError, match="on the GPU"):
        api.ScoreMod(alibi_slopes=_cpu((H,), torch.float32)).c_struct()
    with pytest.raises(ValueError, match="on the GPU"):
        api.MaskSpec(T, doc_ids=torch.zeros((1, T), dtype=torch.int32)).c_struct()
