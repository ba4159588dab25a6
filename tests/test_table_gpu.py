"""GPU parity for composed masks: any and / or / not combination of the five
terms (causal, same document, window, sink, prefix) given as its truth table
(tutorial "FlexAttention in PyTorch", Pattern 3: and_masks / or_masks).

  * block masks: the eight tile lists bit for bit against the oracle;
  * forward and backward: every element against the fp64 oracle within the
    operand bound (parity_utils), lse within 1e-3;
  * the decoding step with a composed mask against the oracle's row;
  * named compositions built with api.and_masks / or_masks / ~ agree with the
    standard combination where they spell the same predicate.
Tables are drawn at random (any 32-bit value) or spelled from the terms;
shapes include Q_LEN != KV_LEN, query offsets and lengths off tile edges."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_block_masks_equal, assert_close, assert_lse_close, assert_within_bound, f64,
                          gpu_block_mask, log, needs_gpu, oracle_block_mask, per_head_f64)
from test_rect_gpu import LENGTHS, _check_sentinel, _desc, _offset, _run, _spec
from workloads import MaskSpecData, ScoreModData, alibi_slopes, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]

# truth tables of the terms alone (bit C + 2 Dc + 4 W + 8 S + 16 P)
T_C, T_D, T_W, T_S, T_P = 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00, 0xFFFF0000
ALL = 0xFFFFFFFF


def _table(rng):
    kind = int(rng.integers(0, 3))
    if kind == 0:
        return int(rng.integers(0, 2 ** 32))
    terms = [T_C, T_D, T_W, T_S, T_P]
    a, b, c = (terms[int(rng.integers(0, 5))] for _ in range(3))
    if rng.integers(0, 2):
        a ^= ALL
    # (a AND b) OR c, or (a OR b) AND c
    return ((a & b) | c) if kind == 1 else ((a | b) & c)


def _case(it, square=False):
    rng = np.random.default_rng(12000 + it)
    T = int(rng.choice(LENGTHS + [256, 512]))
    Q = T if square else int(rng.choice(LENGTHS + [T]))
    off = 0 if square else _offset(rng, T, Q)
    B, spec = _spec(rng, T, Q, off, table=_table(rng))
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(12000 + it)
    tensors = {"q": random_bf16((B, H, Q, D), g), "k": random_bf16((B, H, T, D), g),
               "v": random_bf16((B, H, T, D), g), "dout": random_bf16((B, H, Q, D), g)}
    return B, H, Q, T, D, spec, mod, tensors


@pytest.mark.parametrize("it", range(40))
def test_table_block_mask_bit_exact(it):
    rng = np.random.default_rng(11000 + it)
    T = int(rng.choice(LENGTHS + [1000, 2048]))
    Q = int(rng.choice(LENGTHS + [T]))
    off = _offset(rng, T, Q)
    _, spec = _spec(rng, T, Q, off, table=_table(rng))
    ctx = f"[table bm {it}] Q{Q} KV{T} off{off} table=0x{spec.table:08X} docs={spec.document} " \
          f"window={spec.window} sinks={spec.sinks} prefix={spec.prefix}"
    log(ctx)
    _, _, gpu = gpu_block_mask(spec)
    assert_block_masks_equal(gpu, oracle_block_mask(spec), ctx, spec)


@pytest.mark.parametrize("it", range(24))
def test_table_forward(it):
    B, H, Q, T, D, spec, mod, tensors = _case(it)
    ctx = f"[table fwd {it}] table=0x{spec.table:08X} " + _desc(B, H, Q, T, D, spec, mod)
    log(ctx)
    res = _run(B, H, Q, T, D, spec, mod, tensors, backward=False)
    _check_sentinel(res, Q, T, ctx)
    for b in range(B):
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, b, h, with_mass=True)
            assert_within_bound(f64(res["out"][b, h, :Q]), ro, rm, f"{ctx} b{b} h{h} out")
            assert_lse_close(res["lse"][b, h].double().numpy(), rl, f"{ctx} b{b} h{h}")


@pytest.mark.parametrize("it", range(24))
def test_table_backward(it):
    B, H, Q, T, D, spec, mod, tensors = _case(100 + it)
    ctx = f"[table bwd {it}] table=0x{spec.table:08X} " + _desc(B, H, Q, T, D, spec, mod)
    log(ctx)
    res = _run(B, H, Q, T, D, spec, mod, tensors, backward=True)
    _check_sentinel(res, Q, T, ctx)
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, L, ref, mass in (("dq", Q, rq, mq), ("dk", T, rk, mk), ("dv", T, rv, mv)):
                assert_within_bound(f64(res[name][b, h, :L]), ref, mass, f"{ctx} b{b} h{h} {name}")


def test_table_2k_document_or_window():
    """A composed mask over several tiles: (same document AND causal) OR
    (window 200 AND NOT same document) at 2,048 positions, B2 H2 D128,
    contiguous documents, forward and backward."""
    from block_sparse_masked_build_amd import api
    T = 2048
    rng = np.random.default_rng(12500)
    docs = np.cumsum(rng.random(T) < 1 / 300).astype(np.int32)[None]
    table = (api.and_masks(api.SAME_DOC, api.CAUSAL) | api.and_masks(api.IN_WINDOW, ~api.SAME_DOC)).table
    spec = MaskSpecData(T, causal=False, document=True, doc_ids=docs, window=200, table=table)
    B, H, D = 2, 2, 128
    g = torch.Generator("cpu").manual_seed(12500)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    log(f"[table 2k] table=0x{table:08X}")
    _, _, gpu = gpu_block_mask(spec)
    assert_block_masks_equal(gpu, oracle_block_mask(spec), "table 2k", spec)
    res = _run(B, H, T, T, D, spec, ScoreModData(), tensors, backward=True)
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            ro, rl = oracle.forward_dense(Qm, K, V, spec, None, b, h)
            assert_close(f64(res["out"][b, h, :T]), ro, f"table 2k b{b} h{h} out")
            assert_lse_close(res["lse"][b, h].double().numpy(), rl, f"table 2k b{b} h{h}")
            rq, rk, rv = oracle.backward_dense(Qm, K, V, dO, spec, None, b, h)
            for name, ref in (("dq", rq), ("dk", rk), ("dv", rv)):
                assert_close(f64(res[name][b, h, :T]), ref, f"table 2k b{b} h{h} {name}")


def test_standard_combination_as_table_matches():
    """Pattern 2 (causal AND (window OR sink)) with documents and a prefix,
    spelled with and_masks / or_masks, gives the same block mask, output and
    gradients as the standard combination on the GPU."""
    from block_sparse_masked_build_amd import api
    T, B, H, D = 1000, 1, 2, 64
    rng = np.random.default_rng(12600)
    docs = np.cumsum(rng.random(T) < 1 / 250).astype(np.int32)[None]
    std = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=100, sinks=4, prefix=30)
    expr = api.and_masks(api.or_masks(api.CAUSAL, api.PREFIX), api.SAME_DOC, api.or_masks(api.IN_WINDOW, api.SINK))
    tab = dataclasses.replace(std, table=expr.table)
    log(f"[table = standard] table=0x{expr.table:08X}")
    _, _, g_std = gpu_block_mask(std)
    _, _, g_tab = gpu_block_mask(tab)
    for n in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"):
        assert np.array_equal(g_std[n], g_tab[n]), n
    g = torch.Generator("cpu").manual_seed(12600)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    r_std = _run(B, H, T, T, D, std, ScoreModData(), tensors, backward=True)
    r_tab = _run(B, H, T, T, D, tab, ScoreModData(), tensors, backward=True)
    for n in ("out", "dq", "dk", "dv"):
        assert torch.equal(r_std[n], r_tab[n]), n
    assert torch.equal(r_std["lse"], r_tab["lse"])


@pytest.mark.parametrize("listed", [False, True])
def test_table_decode(listed):
    """Decoding steps at several live lengths with a composed mask: sinks OR
    (window AND same document), against the oracle's row over the live
    keys."""
    from block_sparse_masked_build_amd import api
    cap, B, H, D = 4096, 2, 2, 64
    rng = np.random.default_rng(12700)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 500).astype(np.int32) for _ in range(B)])
    table = (api.SINK | api.and_masks(api.IN_WINDOW, api.SAME_DOC, api.CAUSAL)).table
    spec = MaskSpecData(cap, causal=False, document=True, doc_ids=docs, window=700, sinks=8, table=table)
    log(f"[table decode] cap {cap} table=0x{table:08X} listed={listed}")
    g = torch.Generator("cpu").manual_seed(12700)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s) if listed else None
    for lens in ([4096, 2049], [1, 3000]):
        kvl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), s, None, kv_len=kvl, block_mask=bm)
        torch.cuda.synchronize()
        out, lse = out.cpu(), lse.cpu()
        for b in range(B):
            L = lens[b]
            live = dataclasses.replace(spec, T=L, doc_ids=spec.doc_ids[:, :L])
            Qf = np.zeros((L, D))
            for h in range(H):
                Qf[L - 1] = q[b, h, 0].double().numpy()
                ro, rl = oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                                             live, None, b, h, np.array([L - 1]))
                assert_close(f64(out[b, h]), ro, f"decode b{b} h{h} L{L}")
                assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"decode b{b} h{h} L{L}")
