"""GPU parity for masks whose query and key lengths differ (Q_LEN != KV_LEN,
query i at absolute position q_offset + i) and for lengths that are not
multiples of 128 (tutorial "FlexAttention in PyTorch", quick start: a block
mask is built for given Q_LEN and KV_LEN; a cut-short tile is never full).

  * block masks: the eight tile lists bit for bit against the oracle, the
    exported schedule by its properties;
  * forward and backward: every element against the fp64 oracle on the same
    bf16-rounded inputs, within the operand bound of parity_utils (out, dQ,
    dK, dV) and 1e-3 on lse; rows and keys past the lengths are never
    written.
Shapes: KV_LEN and Q_LEN from 1 to 640 around tile edges, q_offset 0, at the
end of the keys (queries are the last positions of a cache) or anywhere,
with documents, windows, sinks, prefixes, ALiBi and soft-cap drawn at
random."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_block_masks_equal, assert_lse_close, assert_within_bound, f64, gpu_block_mask,
                          log, needs_gpu, oracle_block_mask, per_head_f64)
from workloads import MaskSpecData, ScoreModData, alibi_slopes, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]

LENGTHS = [1, 77, 128, 129, 200, 383, 640]


def _spec(rng, T, Q, off, table=None):
    npos = max(T, off + Q)
    B = int(rng.integers(1, 3))
    docs = None
    if rng.integers(0, 3) > 0:
        mb = B if rng.integers(0, 2) else 1
        if rng.integers(0, 4) == 0:
            docs = rng.integers(0, 3, size=(mb, npos)).astype(np.int32)
        else:
            docs = np.stack([np.cumsum(rng.random(npos) < 1.0 / rng.integers(8, 200)).astype(np.int32)
                             for _ in range(mb)])
    window, sinks, prefix = None, 0, 0
    if rng.integers(0, 2):
        window = int(rng.choice([1, 17, 64, 129, 300]))
        if rng.integers(0, 2):
            sinks = int(rng.choice([1, 4, 130]))
    causal = bool(rng.integers(0, 4) > 0)
    if causal and rng.integers(0, 3) == 0:
        prefix = int(rng.choice([1, 50, 200]))
    spec = MaskSpecData(T, causal=causal, document=docs is not None, doc_ids=docs, window=window, sinks=sinks,
                        prefix=prefix, q_len=Q, q_offset=off, table=table)
    return B, spec


def _offset(rng, T, Q):
    kind = int(rng.integers(0, 3))
    if kind == 0:
        return 0
    if kind == 1:
        return max(T - Q, 0)  # queries are the last positions
    return int(rng.integers(0, T + 1))


def _rect_case(it, table=None):
    rng = np.random.default_rng(9000 + it)
    T = int(rng.choice(LENGTHS))
    Q = int(rng.choice(LENGTHS + [T]))
    off = _offset(rng, T, Q)
    B, spec = _spec(rng, T, Q, off, table)
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(9000 + it)
    tensors = {"q": random_bf16((B, H, Q, D), g), "k": random_bf16((B, H, T, D), g),
               "v": random_bf16((B, H, T, D), g), "dout": random_bf16((B, H, Q, D), g)}
    return B, H, Q, T, D, spec, mod, tensors


def _desc(B, H, Q, T, D, spec, mod):
    return (f"B{B} H{H} Q{Q} KV{T} off{spec.q_offset} D{D} causal={spec.causal} docs={spec.document} "
            f"mb={spec.mask_b} window={spec.window} sinks={spec.sinks} prefix={spec.prefix} "
            f"alibi={mod.alibi_slopes is not None} cap={mod.softcap}")


@pytest.mark.parametrize("it", range(40))
def test_rect_block_mask_bit_exact(it):
    rng = np.random.default_rng(7000 + it)
    T = int(rng.choice(LENGTHS + [1000, 1500]))
    Q = int(rng.choice(LENGTHS + [T, 1]))
    off = _offset(rng, T, Q)
    _, spec = _spec(rng, T, Q, off)
    ctx = f"[rect bm {it}] Q{Q} KV{T} off{off} causal={spec.causal} docs={spec.document} " \
          f"window={spec.window} sinks={spec.sinks} prefix={spec.prefix}"
    log(ctx)
    _, _, gpu = gpu_block_mask(spec)
    assert_block_masks_equal(gpu, oracle_block_mask(spec), ctx, spec)


def _mods(mod):
    from block_sparse_masked_build_amd import api
    if mod.alibi_slopes is None and mod.softcap is None:
        return None
    return api.score_mod(mod.alibi_slopes, mod.softcap)


def _run(B, H, Q, T, D, spec, mod, tensors, backward):
    """Runs the HIP path with outputs pre-filled with a sentinel, so that a
    write past the lengths would show."""
    from block_sparse_masked_build_amd import api
    s = api.from_spec_data(spec)
    m = _mods(mod)
    bm = api.build_block_mask(s)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    # one extra row past each length: the kernels must leave it alone
    big = lambda n, L: torch.full((B, H, L + 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    out_buf = big("out", Q)
    out = out_buf[:, :, :Q]
    lse = torch.empty((B, H, Q), dtype=torch.float32, device="cuda")
    api.flex_attention_fwd(q, k, v, bm, s, m, None, out, lse)
    res = {"out": out_buf, "lse": lse}
    if backward:
        dq_buf, dk_buf, dv_buf = big("dq", Q), big("dk", T), big("dv", T)
        api.flex_attention_bwd(q, k, v, out, lse, do, bm, s, m, None, dq_buf[:, :, :Q], dk_buf[:, :, :T],
                               dv_buf[:, :, :T])
        res.update(dq=dq_buf, dk=dk_buf, dv=dv_buf)
    torch.cuda.synchronize()
    return {n: x.cpu() for n, x in res.items()}


def _check_sentinel(res, Q, T, ctx):
    for n, L in (("out", Q), ("dq", Q), ("dk", T), ("dv", T)):
        if n in res:
            tail = res[n][:, :, L].float()
            assert torch.all(tail == 7.0), f"{ctx} {n}: row {L} (past the length) was written"


@pytest.mark.parametrize("it", range(24))
def test_rect_forward(it):
    B, H, Q, T, D, spec, mod, tensors = _rect_case(it)
    ctx = f"[rect fwd {it}] " + _desc(B, H, Q, T, D, spec, mod)
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
def test_rect_backward(it):
    B, H, Q, T, D, spec, mod, tensors = _rect_case(100 + it)
    ctx = f"[rect bwd {it}] " + _desc(B, H, Q, T, D, spec, mod)
    log(ctx)
    res = _run(B, H, Q, T, D, spec, mod, tensors, backward=True)
    _check_sentinel(res, Q, T, ctx)
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, L, ref, mass in (("dq", Q, rq, mq), ("dk", T, rk, mk), ("dv", T, rv, mv)):
                assert_within_bound(f64(res[name][b, h, :L]), ref, mass, f"{ctx} b{b} h{h} {name}")


def test_rect_slope_gradient():
    """dL/dslope with queries at the end of a longer key range (ALiBi uses
    absolute positions).  As for the square case, both sides take the
    oracle's forward (out rounded to bf16, lse to fp32) as the backward's
    inputs, and the difference must stay under 1e-6 of the oracle's
    sum |g_qj (j - q)|."""
    from block_sparse_masked_build_amd import api
    B, H, Q, T, D = 2, 3, 200, 700, 64
    spec = MaskSpecData(T, causal=True, window=300, q_len=Q, q_offset=T - Q)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H))
    g = torch.Generator("cpu").manual_seed(9500)
    tensors = {"q": random_bf16((B, H, Q, D), g), "k": random_bf16((B, H, T, D), g),
               "v": random_bf16((B, H, T, D), g), "dout": random_bf16((B, H, Q, D), g)}
    log("[rect slopes] B2 H3 Q200 KV700 off500 D64 causal window 300 ALiBi")
    out = torch.zeros((B, H, Q, D), dtype=torch.bfloat16)
    lse = torch.zeros((B, H, Q), dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            o, l = oracle.forward_dense(Qm, K, V, spec, mod, b, h)
            out[b, h] = torch.from_numpy(o).to(torch.bfloat16)
            lse[b, h] = torch.from_numpy(l).to(torch.float32)
    s = api.from_spec_data(spec)
    m = api.score_mod(mod.alibi_slopes)
    bm = api.build_block_mask(s)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    ds = torch.full((H,), float("nan"), dtype=torch.float32, device="cuda")
    api.flex_attention_bwd(q, k, v, out.cuda(), lse.cuda(), do, bm, s, m, dslopes=ds)
    torch.cuda.synchronize()
    ds = ds.cpu().double().numpy()
    for h in range(H):
        tot, mass = 0.0, 0.0
        for b in range(B):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            t, ms = oracle.slope_grad_dense(Qm, K, V, dO, spec, mod, b, h, out=out[b, h].double().numpy(),
                                            lse=lse[b, h].double().numpy())
            tot += t
            mass += ms
        err = abs(ds[h] - tot)
        log(f"  h{h}: gpu {ds[h]:.6e} oracle {tot:.6e} |err|/mass {err / mass:.2e}")
        assert np.isfinite(ds[h]) and err <= 1e-6 * mass, (h, ds[h], tot, mass)


def test_rect_block_mask_sizes_and_all_empty():
    """A query range wholly before the keys under causality sees nothing:
    every tile empty, the forward gives zeros and lse -inf, the backward
    zeros."""
    from block_sparse_masked_build_amd import api
    B, H, Q, T, D = 1, 2, 130, 300, 64
    # queries at positions 0..129 with a window of 0 keys: nothing visible
    spec = MaskSpecData(T, causal=True, window=0, q_len=Q, q_offset=0)
    log("[rect empty] Q130 KV300 window 0")
    _, _, gpu = gpu_block_mask(spec)
    ref = oracle_block_mask(spec)
    assert_block_masks_equal(gpu, ref, "all empty", spec)
    assert int(gpu["kv_num_blocks"].sum() + gpu["full_kv_num_blocks"].sum()) == 0
    g = torch.Generator("cpu").manual_seed(9600)
    tensors = {"q": random_bf16((B, H, Q, D), g), "k": random_bf16((B, H, T, D), g),
               "v": random_bf16((B, H, T, D), g), "dout": random_bf16((B, H, Q, D), g)}
    res = _run(B, H, Q, T, D, spec, ScoreModData(), tensors, backward=True)
    assert torch.all(res["out"][:, :, :Q] == 0)
    assert torch.all(torch.isneginf(res["lse"]))
    for n in ("dq", "dk", "dv"):
        L = Q if n == "dq" else T
        assert torch.all(res[n][:, :, :L] == 0), n
