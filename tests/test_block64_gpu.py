"""GPU parity with 128 x 64 blocks (kv_block = 64; tutorial "FlexAttention
in PyTorch", "What to expect, and the sharp edges", item 4: the block size
is a tunable, smaller blocks capture more sparsity).

  * block masks: row lists at 64-key blocks and column lists at 128 x 128
    tiles, bit for bit against the oracle; work orders by their properties;
  * forward and backward (which then visits only the listed 64-key blocks)
    against the fp64 oracle within the operand bound (parity_utils);
  * the 64-key block lists skip work: on a document + window mask they list
    fewer keys than the 128-key tiles do."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_block_masks_equal, assert_lse_close, assert_within_bound, f64, gpu_block_mask,
                          log, needs_gpu, oracle_block_mask, per_head_f64)
from test_rect_gpu import LENGTHS, _check_sentinel, _desc, _offset, _run, _spec
from workloads import MaskSpecData, ScoreModData, alibi_slopes, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _spec64(rng, T, Q, off, table=None):
    B, spec = _spec(rng, T, Q, off, table)
    return B, dataclasses.replace(spec, kv_block=64)


@pytest.mark.parametrize("it", range(40))
def test_block64_masks_bit_exact(it):
    rng = np.random.default_rng(16000 + it)
    T = int(rng.choice(LENGTHS + [64, 1000, 2048]))
    Q = int(rng.choice(LENGTHS + [T]))
    off = _offset(rng, T, Q)
    table = int(rng.integers(0, 2 ** 32)) if it % 5 == 4 else None
    _, spec = _spec64(rng, T, Q, off, table)
    ctx = f"[bm64 {it}] Q{Q} KV{T} off{off} causal={spec.causal} docs={spec.document} window={spec.window} " \
          f"sinks={spec.sinks} prefix={spec.prefix} table={spec.table}"
    log(ctx)
    _, _, gpu = gpu_block_mask(spec)
    ref = oracle_block_mask(spec)
    assert gpu["kv_indices"].shape[-1] == -(-T // 64)
    assert_block_masks_equal(gpu, ref, ctx, spec)


def _case(it):
    rng = np.random.default_rng(17000 + it)
    T = int(rng.choice(LENGTHS + [64, 256, 512]))
    Q = int(rng.choice(LENGTHS + [T])) if it % 2 else T
    off = _offset(rng, T, Q) if it % 2 else 0
    table = int(rng.integers(0, 2 ** 32)) if it % 6 == 5 else None
    B, spec = _spec64(rng, T, Q, off, table)
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(17000 + it)
    tensors = {"q": random_bf16((B, H, Q, D), g), "k": random_bf16((B, H, T, D), g),
               "v": random_bf16((B, H, T, D), g), "dout": random_bf16((B, H, Q, D), g)}
    return B, H, Q, T, D, spec, mod, tensors


@pytest.mark.parametrize("it", range(24))
def test_block64_forward_backward(it):
    B, H, Q, T, D, spec, mod, tensors = _case(it)
    ctx = f"[block64 {it}] table={spec.table} " + _desc(B, H, Q, T, D, spec, mod)
    log(ctx)
    res = _run(B, H, Q, T, D, spec, mod, tensors, backward=True)
    _check_sentinel(res, Q, T, ctx)
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, b, h, with_mass=True)
            assert_within_bound(f64(res["out"][b, h, :Q]), ro, rm, f"{ctx} b{b} h{h} out")
            assert_lse_close(res["lse"][b, h].double().numpy(), rl, f"{ctx} b{b} h{h}")
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, L, ref, mass in (("dq", Q, rq, mq), ("dk", T, rk, mk), ("dv", T, rv, mv)):
                assert_within_bound(f64(res[name][b, h, :L]), ref, mass, f"{ctx} b{b} h{h} {name}")


def test_block64_lists_fewer_keys_on_documents_and_window():
    """Packed documents (mean length 300) with a window of 200 at 8,192
    positions: the 64-key lists cover fewer keys than the 128-key tiles,
    and every 128 x 128 tile is listed iff one of its 64-key halves is."""
    T = 8192
    rng = np.random.default_rng(17500)
    docs = np.cumsum(rng.random(T) < 1 / 300).astype(np.int32)[None]
    s128 = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=200)
    s64 = dataclasses.replace(s128, kv_block=64)
    _, _, g128 = gpu_block_mask(s128)
    _, _, g64 = gpu_block_mask(s64)
    keys128 = 128 * int(g128["kv_num_blocks"].sum() + g128["full_kv_num_blocks"].sum())
    keys64 = 64 * int(g64["kv_num_blocks"].sum() + g64["full_kv_num_blocks"].sum())
    log(f"  listed keys per query-tile row, summed: 128-key tiles {keys128}, 64-key blocks {keys64}")
    assert keys64 < keys128
    for n in ("q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices"):
        assert np.array_equal(g64[n], g128[n]), n
