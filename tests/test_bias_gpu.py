"""GPU parity of the relative-position bias table (a learned bias trains
through the fused backward: tutorial "FlexAttention in PyTorch", Pattern 3)
against the fp64 oracle: the score gets bias[h, R + clip(q - kv, -R, R)]
before the soft-cap.

  * forward and backward on random shapes (Q_LEN != KV_LEN, lengths off the
    128 grid, composed masks, 64-key blocks, fp16), every element within the
    operand bound of parity_utils, lse within 1e-3;
  * dL/dbias: both sides take the oracle's own forward (out rounded to the
    tensor type, lse to fp32) as the backward's inputs, as for the slope
    gradient.  What is left is fp32 against fp64: p from an fp32 exp2
    (about 3e-6 relative per term), the dot products dP and Delta that g
    subtracts, each summed in fp32 over D products, and the sums over at
    most 32 terms per wave array, 8 arrays and B * QT partial rows in fp32.
    The bound per entry j is 5e-5 of sum |g| over the entry's pairs (the
    oracle's mass, above 3e-6 + 2^-24 * (32 + 8 + B*QT) for every case
    here) plus 2 D 2^-24 times the oracle's pmass, the sum over the pairs of
    p c' (sum |dO v| + sum |dO out|): what rounding dP and Delta can move g
    by, which matters where they cancel (one visible key: g is 0 in exact
    arithmetic).  Entries that no visible pair reads must come out exactly
    zero;
  * determinism: two backward calls give identical bits;
  * decoding steps with the table against the oracle's row at L - 1.
Bias radii 0 .. 1024 (the largest the kernels take), so that tiles both
inside the table and past its ends (clipped distances) are covered."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_close, assert_lse_close, assert_within_bound, f64, log, needs_gpu,
                          per_head_f64)
from workloads import MaskSpecData, ScoreModData, bias_table, random_bf16, random_f16

pytestmark = [pytest.mark.gpu, needs_gpu]

LENGTHS = [1, 77, 128, 129, 200, 383, 640]
RADII = [0, 1, 5, 64, 300, 1024]
T_C, T_D, T_W, T_S, T_P = 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0, 0xFF00FF00, 0xFFFF0000
REL_TOL = 5e-5


def _case(it):
    rng = np.random.default_rng(15000 + it)
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
    table = None
    if rng.integers(0, 4) == 0:
        terms = [T_C, T_D, T_W, T_S, T_P]
        a, b, c = (terms[int(rng.integers(0, 5))] for _ in range(3))
        table = (a & b) | c
    spec = MaskSpecData(T, causal=causal, document=docs is not None, doc_ids=docs, window=window, sinks=sinks,
                        q_len=Q, q_offset=off, table=table, kv_block=64 if rng.integers(0, 4) == 0 else 128)
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    R = int(rng.choice(RADII))
    mod = ScoreModData(softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None,
                       bias_table=bias_table(H, R, seed=15000 + it))
    fmt = "f16" if rng.integers(0, 4) == 0 else "bf16"
    rand = random_f16 if fmt == "f16" else random_bf16
    g = torch.Generator("cpu").manual_seed(15000 + it)
    tensors = {"q": rand((B, H, Q, D), g), "k": rand((B, H, T, D), g), "v": rand((B, H, T, D), g),
               "dout": rand((B, H, Q, D), g)}
    return B, H, Q, T, D, spec, mod, tensors, fmt


def _desc(B, H, Q, T, D, spec, mod, fmt):
    tab = f"0x{spec.table:08X}" if spec.table is not None else None
    return (f"B{B} H{H} Q{Q} KV{T} off{spec.q_offset} D{D} {fmt} causal={spec.causal} docs={spec.document} "
            f"window={spec.window} sinks={spec.sinks} table={tab} kv_block={spec.kv_block} "
            f"R={(mod.bias_table.shape[1] - 1) // 2} cap={mod.softcap}")


def _mod(mod):
    from block_sparse_masked_build_amd import api
    return api.score_mod(None, mod.softcap, bias=mod.bias_table)


def _forward(tensors, spec, mod):
    from block_sparse_masked_build_amd import api
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    q, k, v = (tensors[n].cuda() for n in ("q", "k", "v"))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s, _mod(mod))
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _backward(tensors, spec, mod, out, lse):
    """dq, dk, dv and dbias from the given forward outputs."""
    from block_sparse_masked_build_amd import api
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    m = _mod(mod)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    db = torch.full(m.bias.shape, float("nan"), dtype=torch.float32, device="cuda")
    dq, dk, dv = api.flex_attention_bwd(q, k, v, out.cuda(), lse.cuda(), do, bm, s, m, dbias=db)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), db.cpu()


def _oracle_forward(tensors, spec, mod, B, H, dtype):
    Q, D = tensors["q"].shape[2], tensors["q"].shape[3]
    out = torch.zeros((B, H, Q, D), dtype=dtype)
    lse = torch.zeros((B, H, Q), dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            o, l = oracle.forward_dense(Qm, K, V, spec, mod, b, h)
            out[b, h] = torch.from_numpy(o).to(dtype)
            lse[b, h] = torch.from_numpy(l).to(torch.float32)
    return out, lse


def _pairs_per_entry(spec, mod, b, Q, T):
    """Visible (query, key) pairs that read each table entry."""
    rows = np.arange(Q)
    vis = oracle.visible(spec, b, rows[:, None], np.arange(T)[None, :])
    idx = oracle.bias_index(mod, rows + spec.q_offset, np.arange(T))
    return np.bincount(idx[vis], minlength=mod.bias_table.shape[1])


def _check_dbias(got, tensors, spec, mod, B, H, out, lse, ctx):
    worst = 0.0
    Q, D, T = tensors["q"].shape[2], tensors["q"].shape[3], tensors["k"].shape[2]
    npairs = sum(_pairs_per_entry(spec, mod, b, Q, T) for b in range(B))
    for h in range(H):
        ref = mass = pmass = 0.0
        for b in range(B):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            g, m, pm = oracle.bias_grad_dense(Qm, K, V, dO, spec, mod, b, h, out=out[b, h].double().numpy(),
                                              lse=lse[b, h].double().numpy(), with_pmass=True)
            ref = ref + g
            mass = mass + m
            pmass = pmass + pm
        gh = got[h].double().numpy()
        err = np.abs(gh - ref)
        bound = REL_TOL * mass + 2 * D * 2.0 ** -24 * pmass
        assert np.all(np.isfinite(gh)), (ctx, h)
        assert np.all(gh[npairs == 0] == 0), (ctx, h, "an entry no pair reads is not zero")
        bad = np.nonzero(err > bound)[0]
        assert len(bad) == 0, (ctx, h, bad[:5], gh[bad[:5]], ref[bad[:5]], mass[bad[:5]])
        live = mass > 0
        if live.any():
            worst = max(worst, float((err[live] / mass[live]).max()))
    log(f"  {ctx}: dbias max |err|/mass {worst:.2e}")


@pytest.mark.parametrize("it", range(24))
def test_bias_forward(it):
    B, H, Q, T, D, spec, mod, tensors, fmt = _case(it)
    ctx = f"[bias fwd {it}] " + _desc(B, H, Q, T, D, spec, mod, fmt)
    log(ctx)
    out, lse = _forward(tensors, spec, mod)
    for b in range(B):
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, b, h, with_mass=True)
            assert_within_bound(f64(out[b, h]), ro, rm, f"{ctx} b{b} h{h} out", fmt=fmt)
            assert_lse_close(lse[b, h].double().numpy(), rl, f"{ctx} b{b} h{h}")


@pytest.mark.parametrize("it", range(24))
def test_bias_backward_and_gradient(it):
    B, H, Q, T, D, spec, mod, tensors, fmt = _case(100 + it)
    ctx = f"[bias bwd {it}] " + _desc(B, H, Q, T, D, spec, mod, fmt)
    log(ctx)
    dtype = tensors["q"].dtype
    out, lse = _oracle_forward(tensors, spec, mod, B, H, dtype)
    dq, dk, dv, db = _backward(tensors, spec, mod, out, lse)
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, x, ref, mass in (("dq", dq, rq, mq), ("dk", dk, rk, mk), ("dv", dv, rv, mv)):
                assert_within_bound(f64(x[b, h]), ref, mass, f"{ctx} b{b} h{h} {name}", fmt=fmt)
    _check_dbias(db, tensors, spec, mod, B, H, out, lse, ctx)


def _doc_window_case(T, H, R, cap, seed):
    rng = np.random.default_rng(seed)
    docs = np.cumsum(rng.random(T) < 1 / 700).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=1024)
    mod = ScoreModData(softcap=cap, bias_table=bias_table(H, R, seed=seed, sd=0.5))
    g = torch.Generator("cpu").manual_seed(seed)
    tensors = {n: random_bf16((1, H, T, 128), g) for n in ("q", "k", "v", "dout")}
    return spec, mod, tensors


def test_bias_doc_window_4k_radius_1024():
    """The 64K workload's mask kind (causal, documents, window 1024) at
    T = 4096, D = 128, R = 1024: the tiles at the window's edge read
    distances past R (the clipped path), the others take the direct one."""
    H = 2
    spec, mod, tensors = _doc_window_case(4096, H, 1024, 30.0, 15500)
    log("[bias 4k] causal+docs+window 1024, R 1024, cap 30")
    out_g, lse_g = _forward(tensors, spec, mod)
    out, lse = _oracle_forward(tensors, spec, mod, 1, H, torch.bfloat16)
    for h in range(H):
        Qm, K, V = (per_head_f64(tensors[n], 0, h) for n in ("q", "k", "v"))
        ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, 0, h, with_mass=True)
        assert_within_bound(f64(out_g[0, h]), ro, rm, f"4k h{h} out")
        assert_lse_close(lse_g[0, h].double().numpy(), rl, f"4k h{h}")
    dq, dk, dv, db = _backward(tensors, spec, mod, out, lse)
    for h in range(H):
        Qm, K, V, dO = (per_head_f64(tensors[n], 0, h) for n in ("q", "k", "v", "dout"))
        rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, 0, h, with_mass=True)
        for name, x, ref, mass in (("dq", dq, rq, mq), ("dk", dk, rk, mk), ("dv", dv, rv, mv)):
            assert_within_bound(f64(x[0, h]), ref, mass, f"4k h{h} {name}")
    _check_dbias(db, tensors, spec, mod, 1, H, out, lse, "4k")


def test_bias_backward_is_deterministic():
    """Two backward calls on the same inputs give identical bits for dq, dk,
    dv and dbias (no atomics across waves; fixed-order sums)."""
    H = 2
    spec, mod, tensors = _doc_window_case(2048, H, 512, None, 15600)
    out, lse = _forward(tensors, spec, mod)
    r1 = _backward(tensors, spec, mod, out, lse)
    r2 = _backward(tensors, spec, mod, out, lse)
    for n, a, b in zip(("dq", "dk", "dv", "dbias"), r1, r2):
        assert torch.equal(a, b), n


def test_bias_zero_table_equals_no_bias():
    """A table of zeros changes nothing: the forward and the backward match
    the kernels without a bias bit for bit where the same arithmetic runs
    (the bias kernels take the general path, so the comparison is against
    the oracle bound instead where it does not)."""
    from block_sparse_masked_build_amd import api
    B, H, T, D = 1, 2, 640, 64
    spec = MaskSpecData(T, causal=True, window=200)
    g = torch.Generator("cpu").manual_seed(15700)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    zero = ScoreModData(bias_table=np.zeros((H, 2 * 64 + 1), np.float32))
    out_z, lse_z = _forward(tensors, spec, zero)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s)
    q, k, v = (tensors[n].cuda() for n in ("q", "k", "v"))
    out_n, lse_n = api.flex_attention_fwd(q, k, v, bm, s, None)
    torch.cuda.synchronize()
    assert torch.allclose(out_z.float(), out_n.cpu().float(), atol=1e-2, rtol=0)
    assert torch.allclose(lse_z, lse_n.cpu(), atol=1e-5, rtol=0)
    dq, dk, dv, db = _backward(tensors, spec, zero, out_z, lse_z)
    # without a cap the entries of dL/dbias sum to zero (each row of g does)
    tot = db.double().sum(dim=1).abs()
    assert torch.all(tot <= 1e-3 * db.double().abs().sum(dim=1) + 1e-6), tot


@pytest.mark.parametrize("listed", [False, True])
def test_bias_decode(listed):
    """Decoding steps with the table at several live lengths (one per batch
    element), with and without a block mask, against the oracle's row at
    L - 1 over the live keys."""
    from block_sparse_masked_build_amd import api
    cap, B, H, D, R = 4096, 2, 2, 128, 700
    rng = np.random.default_rng(15800)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 900).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=1500)
    mod = ScoreModData(softcap=20.0, bias_table=bias_table(H, R, seed=15800))
    log(f"[bias decode] cap {cap} R {R} listed={listed}")
    g = torch.Generator("cpu").manual_seed(15800)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    bm = api.build_block_mask(s) if listed else None
    m = _mod(mod)
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
