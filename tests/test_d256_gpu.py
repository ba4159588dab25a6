"""GPU parity at head dimension 256 (tutorial "FlexAttention in PyTorch",
"What to expect, and the sharp edges": head dims that are multiples of 64)
against the fp64 oracle, which takes any D.

  * forward on random shapes: Q_LEN != KV_LEN, lengths off the 128 grid,
    documents, windows, sinks, prefixes, composed masks, 64-key blocks,
    ALiBi, soft-cap, a bias table and fp16, every element within the
    operand bound of parity_utils, lse within 1e-3;
  * the decoding step at several live lengths, with and without a block
    mask;
  * the backward (dkdv256_kernel for dK/dV) on the same random shapes and
    a 2K document + window mask, bit-identical over two calls; a bias
    table's backward returns BSM_E_UNSUPPORTED at D = 256.
Inputs: N(0, 1) draws rounded to the tensor type, seeded per case."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_close, assert_lse_close, assert_within_bound, f64, log, needs_gpu, per_head_f64
from workloads import MaskSpecData, ScoreModData, alibi_slopes, bias_table, random_bf16, random_f16

pytestmark = [pytest.mark.gpu, needs_gpu]

D = 256
LENGTHS = [1, 77, 128, 129, 200, 383, 640]
T_C, T_D, T_W, T_S, T_P = 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00, 0xFFFF0000


def _case(it):
    rng = np.random.default_rng(17000 + it)
    T = int(rng.choice(LENGTHS + [256, 1000]))
    Q = int(rng.choice(LENGTHS + [T]))
    kind = int(rng.integers(0, 3))
    off = 0 if kind == 0 else (max(T - Q, 0) if kind == 1 else int(rng.integers(0, T + 1)))
    npos = max(T, off + Q)
    B = int(rng.integers(1, 3))
    docs = None
    if rng.integers(0, 2):
        mb = B if rng.integers(0, 2) else 1
        docs = np.stack([np.cumsum(rng.random(npos) < 1.0 / rng.integers(8, 200)).astype(np.int32)
                         for _ in range(mb)])
    window = int(rng.choice([17, 129, 300])) if rng.integers(0, 2) else None
    sinks = int(rng.choice([1, 4])) if window is not None and rng.integers(0, 2) else 0
    causal = bool(rng.integers(0, 4) > 0)
    prefix = int(rng.choice([0, 50])) if causal else 0
    table = None
    if rng.integers(0, 4) == 0:
        terms = [T_C, T_D, T_W, T_S, T_P]
        a, b, c = (terms[int(rng.integers(0, 5))] for _ in range(3))
        table = (a & b) | c
    spec = MaskSpecData(T, causal=causal, document=docs is not None, doc_ids=docs, window=window, sinks=sinks,
                        prefix=prefix, q_len=Q, q_offset=off, table=table,
                        kv_block=64 if rng.integers(0, 4) == 0 else 128)
    H = int(rng.integers(1, 3))
    add = int(rng.integers(0, 3))
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if add == 1 else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None,
                       bias_table=bias_table(H, int(rng.choice([0, 64, 1024])), seed=17000 + it) if add == 2 else None)
    fmt = "f16" if rng.integers(0, 4) == 0 else "bf16"
    rand = random_f16 if fmt == "f16" else random_bf16
    g = torch.Generator("cpu").manual_seed(17000 + it)
    tensors = {"q": rand((B, H, Q, D), g), "k": rand((B, H, T, D), g), "v": rand((B, H, T, D), g)}
    return B, H, Q, T, spec, mod, tensors, fmt


def _mod(api, mod):
    if mod.alibi_slopes is None and mod.softcap is None and mod.bias_table is None:
        return None
    return api.score_mod(mod.alibi_slopes, mod.softcap, bias=mod.bias_table)


@pytest.mark.parametrize("it", range(24))
def test_d256_forward(it):
    from block_sparse_masked_build_amd import api
    B, H, Q, T, spec, mod, tensors, fmt = _case(it)
    ctx = (f"[d256 fwd {it}] B{B} H{H} Q{Q} KV{T} off{spec.q_offset} {fmt} causal={spec.causal} "
           f"docs={spec.document} window={spec.window} sinks={spec.sinks} prefix={spec.prefix} "
           f"table={spec.table} kv_block={spec.kv_block} alibi={mod.alibi_slopes is not None} cap={mod.softcap} "
           f"bias={mod.bias_table is not None}")
    log(ctx)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    q, k, v = (tensors[n].cuda() for n in ("q", "k", "v"))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s, _mod(api, mod))
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, b, h, with_mass=True)
            assert_within_bound(f64(out[b, h]), ro, rm, f"{ctx} b{b} h{h} out", fmt=fmt)
            assert_lse_close(lse[b, h].double().numpy(), rl, f"{ctx} b{b} h{h}")


def test_d256_forward_doc_window_4k():
    """The 64K workload's mask kind at T = 4096, D = 256, whole tiles."""
    from block_sparse_masked_build_amd import api
    T, H = 4096, 2
    rng = np.random.default_rng(17500)
    docs = np.cumsum(rng.random(T) < 1 / 500).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=1024)
    g = torch.Generator("cpu").manual_seed(17500)
    tensors = {n: random_bf16((1, H, T, D), g) for n in ("q", "k", "v")}
    log("[d256 4k] causal+docs+window 1024")
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    out, lse = api.flex_attention_fwd(*(tensors[n].cuda() for n in ("q", "k", "v")), bm, s)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for h in range(H):
        Qm, K, V = (per_head_f64(tensors[n], 0, h) for n in ("q", "k", "v"))
        ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, None, 0, h, with_mass=True)
        assert_within_bound(f64(out[0, h]), ro, rm, f"4k h{h} out")
        assert_lse_close(lse[0, h].double().numpy(), rl, f"4k h{h}")


@pytest.mark.parametrize("listed", [False, True])
def test_d256_decode(listed):
    from block_sparse_masked_build_amd import api
    cap, B, H = 4096, 2, 2
    rng = np.random.default_rng(17600)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 900).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=1500)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=20.0)
    log(f"[d256 decode] cap {cap} listed={listed}")
    g = torch.Generator("cpu").manual_seed(17600)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s) if listed else None
    m = api.score_mod(mod.alibi_slopes, mod.softcap)
    for lens in ([4096, 1], [2049, 3000]):
        kvl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), s, m, kv_len=kvl, block_mask=bm)
        torch.cuda.synchronize()
        out, lse = out.cpu(), lse.cpu()
        for b in range(B):
            L = lens[b]
            live = dataclasses.replace(spec, T=L, doc_ids=spec.doc_ids[:, :L])
            Qf = np.zeros((L, D))
            for h in range(H):
                Qf[L - 1] = q[b, h, 0].double().numpy()
                ro, rl = oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                                             live, mod, b, h, np.array([L - 1]))
                assert_close(f64(out[b, h]), ro, f"decode b{b} h{h} L{L}")
                assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"decode b{b} h{h} L{L}")


@pytest.mark.parametrize("it", range(16))
def test_d256_backward(it):
    """dQ, dK and dV at D = 256 (dkdv256_kernel: 16 keys per wave in
    16x16x32 blocks, 64-query steps) on the forward cases' shapes and masks
    (no bias table: its backward is built for D = 64 and 128)."""
    from block_sparse_masked_build_amd import api
    B, H, Q, T, spec, mod, tensors, fmt = _case(100 + it)
    mod = dataclasses.replace(mod, bias_table=None)
    ctx = (f"[d256 bwd {it}] B{B} H{H} Q{Q} KV{T} off{spec.q_offset} {fmt} causal={spec.causal} "
           f"docs={spec.document} window={spec.window} sinks={spec.sinks} table={spec.table} "
           f"kv_block={spec.kv_block} alibi={mod.alibi_slopes is not None} cap={mod.softcap}")
    log(ctx)
    g = torch.Generator("cpu").manual_seed(17900 + it)
    rand = random_f16 if fmt == "f16" else random_bf16
    tensors["dout"] = rand((B, H, Q, D), g)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    m = _mod(api, mod)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s, m)
    dq, dk, dv = api.flex_attention_bwd(q, k, v, out, lse, do, bm, s, m)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, x, ref, mass in (("dq", dq, rq, mq), ("dk", dk, rk, mk), ("dv", dv, rv, mv)):
                assert_within_bound(f64(x[b, h]), ref, mass, f"{ctx} b{b} h{h} {name}", fmt=fmt)


def test_d256_backward_doc_window_2k_deterministic():
    """Causal + documents + window at T = 2048: parity of every element and
    two calls bit-identical."""
    from block_sparse_masked_build_amd import api
    T, H = 2048, 2
    rng = np.random.default_rng(17800)
    docs = np.cumsum(rng.random(T) < 1 / 400).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=700)
    g = torch.Generator("cpu").manual_seed(17800)
    tensors = {n: random_bf16((1, H, T, D), g) for n in ("q", "k", "v", "dout")}
    log("[d256 bwd 2k] causal+docs+window 700")
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s)
    r1 = [x.cpu() for x in api.flex_attention_bwd(q, k, v, out, lse, do, bm, s)]
    r2 = [x.cpu() for x in api.flex_attention_bwd(q, k, v, out, lse, do, bm, s)]
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    for h in range(H):
        Qm, K, V, dO = (per_head_f64(tensors[n], 0, h) for n in ("q", "k", "v", "dout"))
        rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, None, 0, h, with_mass=True)
        for name, x, ref, mass in (("dq", r1[0], rq, mq), ("dk", r1[1], rk, mk), ("dv", r1[2], rv, mv)):
            assert_within_bound(f64(x[0, h]), ref, mass, f"2k h{h} {name}")


def test_d256_bias_backward_is_unsupported():
    from block_sparse_masked_build_amd import _lib, api
    T, H = 256, 1
    spec = MaskSpecData(T, causal=True)
    g = torch.Generator("cpu").manual_seed(17700)
    q, k, v, do = (random_bf16((1, H, T, D), g).cuda() for _ in range(4))
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    m = api.score_mod(bias=bias_table(H, 16, seed=1))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s, m)
    with pytest.raises(RuntimeError) as e:
        api.flex_attention_bwd(q, k, v, out, lse, do, bm, s, m,
                               workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
    assert e.value.status == _lib.BSM_E_UNSUPPORTED and "bias" in str(e.value)
