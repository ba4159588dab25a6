"""The allocation-free decoding entry point (bsm_flex_attention_decode_static)
against the workspace one (bsm_flex_attention_decode): the same kernels, so
the outputs must be bitwise equal.  Two calls in a row on the shared static
scratch, the second with a smaller input, then a request beyond the scratch
is rejected on the host."""
import numpy as np
import pytest
import torch

from parity_utils import log, needs_gpu
from workloads import random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _inputs(B, H, cap, D, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return [random_bf16(sh, g).cuda() for sh in ((B, H, 1, D), (B, H, cap, D), (B, H, cap, D))]


def _both(api, q, k, v, spec, mod, kvl, bm):
    B, H, cap, D = k.shape
    ref_o, ref_l = api.flex_attention_decode(q, k, v, spec, mod, kv_len=kvl, block_mask=bm)
    out = torch.full((B, H, 1, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    api.flex_attention_decode_static(q, k, v, spec, mod, None, kvl, bm, out, lse)
    torch.cuda.synchronize()
    return (out, lse), (ref_o, ref_l)


def test_static_decode_matches_workspace_decode_twice():
    from block_sparse_masked_build_amd import api
    # call 1: B4 H8 cap 16384 D128 (partials 4*8*16*130*4 = 266 KB), documents
    # through the block mask, ALiBi + soft-cap, per-batch live lengths
    B, H, cap, D = 4, 8, 16384, 128
    rng = np.random.default_rng(71)
    docs = np.cumsum(rng.random(cap) < 1 / 600).astype(np.int32)[None]
    spec = api.mask_spec(cap, causal=True, doc_ids=docs)
    bm = api.build_block_mask(spec)
    mod = api.score_mod(np.power(2.0, -np.arange(1, H + 1)).astype(np.float32), 30.0)
    kvl = torch.tensor([16384, 9000, 129, 1], dtype=torch.int32, device="cuda")
    q, k, v = _inputs(B, H, cap, D, 72)
    log("[no-alloc] call 1: B4 H8 cap 16384 D128, documents via block mask, ALiBi + soft-cap")
    got, ref = _both(api, q, k, v, spec, mod, kvl, bm)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    # call 2, smaller: B1 H2 cap 1000 D64, window + sinks, no block mask,
    # one live length; the scratch still holds call 1's partials
    B, H, cap, D = 1, 2, 1000, 64
    spec = api.mask_spec(cap, causal=True, window=200, sinks=4)
    kvl = torch.tensor([777], dtype=torch.int32, device="cuda")
    q, k, v = _inputs(B, H, cap, D, 73)
    log("[no-alloc] call 2: B1 H2 cap 1000 D64, window 200 + 4 sinks")
    got, ref = _both(api, q, k, v, spec, None, kvl, None)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert torch.isfinite(got[0].float()).all()


def test_static_decode_rejects_requests_beyond_the_scratch():
    from block_sparse_masked_build_amd import api
    from block_sparse_masked_build_amd._lib import BSM_E_WORKSPACE, BsmError, lib
    limit = lib.bsm_decode_static_max_bytes()
    assert limit == 16 << 20
    # B 64, H 32, cap 8192 (8 slots), D 128: 64*32*8*130*4 = 8.5 MB fits; cap 32768 does not
    B, H, D = 64, 32, 128
    q = torch.zeros((B, H, 1, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, H, 32768, D), dtype=torch.bfloat16, device="cuda")
    spec = api.mask_spec(32768, causal=True)
    kvl = torch.tensor([32768], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    log("[no-alloc] a request beyond the scratch is rejected")
    with pytest.raises(BsmError) as ei:
        api.flex_attention_decode_static(q, kv, kv, spec, None, None, kvl, None, out, lse)
    assert ei.value.status == BSM_E_WORKSPACE
