"""GPU parity with fp16 tensors (tutorial "FlexAttention in PyTorch", "What
to expect, and the sharp edges": bf16 and fp16 inputs).  The matrix-core
products take fp16 operands -- the inputs, the probabilities P and the score
gradients dS -- and accumulate in fp32; outputs are fp16.  Bound per element
(parity_utils, fmt="f16"): 2e-3 + half_ulp_fp16(|ref|) + 2^-11 * mass, a
tenth of the bf16 fixed term, which a path that rounded to bf16 anywhere
would miss; lse within 1e-3.  Inputs are N(0, 1) draws rounded to fp16, the
oracle runs in fp64 on the same values."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_lse_close, assert_within_bound, f64, log, needs_gpu, per_head_f64
from test_rect_gpu import LENGTHS, _offset, _spec
from workloads import ScoreModData, alibi_slopes, random_f16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _case(it, rect, table=None):
    rng = np.random.default_rng(15000 + it)
    T = int(rng.choice(LENGTHS + [256, 512]))
    Q = int(rng.choice(LENGTHS + [T])) if rect else T
    off = _offset(rng, T, Q) if rect else 0
    B, spec = _spec(rng, T, Q, off, table)
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(15000 + it)
    tensors = {"q": random_f16((B, H, Q, D), g), "k": random_f16((B, H, T, D), g),
               "v": random_f16((B, H, T, D), g), "dout": random_f16((B, H, Q, D), g)}
    return B, H, Q, T, D, spec, mod, tensors


def _run(spec, mod, tensors, backward):
    from block_sparse_masked_build_amd import api
    s = api.from_spec_data(spec)
    m = None if mod.alibi_slopes is None and mod.softcap is None else api.score_mod(mod.alibi_slopes, mod.softcap)
    bm = api.build_block_mask(s)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    out, lse = api.flex_attention_fwd(q, k, v, bm, s, m)
    res = {"out": out, "lse": lse}
    if backward:
        dq, dk, dv = api.flex_attention_bwd(q, k, v, out, lse, do, bm, s, m)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for n in ("out", "dq", "dk", "dv"):
        if n in res:
            assert res[n].dtype == torch.float16, n
    return {n: x.cpu() for n, x in res.items()}


@pytest.mark.parametrize("it", range(16))
def test_fp16_forward_backward(it):
    rect = it % 2 == 1
    table = None
    if it % 4 == 3:
        table = int(np.random.default_rng(it).integers(0, 2 ** 32))
    B, H, Q, T, D, spec, mod, tensors = _case(it, rect, table)
    ctx = (f"[fp16 {it}] B{B} H{H} Q{Q} KV{T} off{spec.q_offset} D{D} causal={spec.causal} docs={spec.document} "
           f"window={spec.window} sinks={spec.sinks} prefix={spec.prefix} table={spec.table} "
           f"alibi={mod.alibi_slopes is not None} cap={mod.softcap}")
    log(ctx)
    res = _run(spec, mod, tensors, backward=True)
    worst = {}
    for b in range(B):
        for h in range(H):
            Qm, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            ro, rl, rm = oracle.forward_dense(Qm, K, V, spec, mod, b, h, with_mass=True)
            worst["out"] = assert_within_bound(f64(res["out"][b, h]), ro, rm, f"{ctx} b{b} h{h} out", fmt="f16")
            assert_lse_close(res["lse"][b, h].double().numpy(), rl, f"{ctx} b{b} h{h}")
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Qm, K, V, dO, spec, mod, b, h, with_mass=True)
            for name, ref, mass in (("dq", rq, mq), ("dk", rk, mk), ("dv", rv, mv)):
                worst[name] = assert_within_bound(f64(res[name][b, h]), ref, mass, f"{ctx} b{b} h{h} {name}",
                                                  fmt="f16")
    log("  max-abs " + " ".join(f"{n} {mx:.2e}" for n, (mx, _) in worst.items()))


def test_fp16_is_more_accurate_than_bf16():
    """The same N(0, 1) draws through the fp16 and the bf16 paths (each on
    its own rounding of the inputs, each against the oracle on those inputs):
    the fp16 forward's worst error is several times below the bf16 one's."""
    from workloads import MaskSpecData, random_bf16
    T, B, H, D = 512, 1, 2, 128
    rng = np.random.default_rng(15900)
    docs = np.cumsum(rng.random(T) < 1 / 100).astype(np.int32)[None]
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=200)
    errs = {}
    for name, gen in (("f16", random_f16), ("bf16", random_bf16)):
        g = torch.Generator("cpu").manual_seed(15900)
        tensors = {n: gen((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
        res = _run(spec, ScoreModData(), tensors, backward=False) if name == "f16" else None
        if res is None:
            from block_sparse_masked_build_amd import api
            s = api.from_spec_data(spec)
            out, _ = api.flex_attention_fwd(*(tensors[n].cuda() for n in ("q", "k", "v")), api.build_block_mask(s), s)
            res = {"out": out.cpu()}
        e = 0.0
        for h in range(H):
            Qm, K, V = (per_head_f64(tensors[n], 0, h) for n in ("q", "k", "v"))
            ro, _ = oracle.forward_dense(Qm, K, V, spec, None, 0, h)
            e = max(e, float(np.abs(f64(res["out"][0, h]) - ro).max()))
        errs[name] = e
    log(f"  forward max-abs: fp16 {errs['f16']:.2e}, bf16 {errs['bf16']:.2e}")
    assert errs["f16"] * 4 < errs["bf16"], errs


def test_fp16_decode():
    """Decoding steps with fp16 caches at several live lengths."""
    from block_sparse_masked_build_amd import api
    from workloads import MaskSpecData
    import dataclasses
    cap, B, H, D = 2048, 2, 2, 128
    rng = np.random.default_rng(15950)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 400).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=500)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0)
    g = torch.Generator("cpu").manual_seed(15950)
    q = random_f16((B, H, 1, D), g)
    k = random_f16((B, H, cap, D), g)
    v = random_f16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    m = api.score_mod(mod.alibi_slopes, mod.softcap)
    lens = [2048, 777]
    out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), s, m,
                                         kv_len=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        L = lens[b]
        live = dataclasses.replace(spec, T=L, doc_ids=spec.doc_ids[:, :L])
        for h in range(H):
            Qf = np.zeros((L, D))
            Qf[L - 1] = q[b, h, 0].double().numpy()
            ro, rl, rm = oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                                             live, mod, b, h, np.array([L - 1]), with_mass=True)
            assert_within_bound(f64(out[b, h]), ro, rm, f"decode fp16 b{b} h{h} L{L}", fmt="f16")
            assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"decode fp16 b{b} h{h}")
