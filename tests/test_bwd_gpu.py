"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle on
the same bf16-rounded inputs: max-abs <= 2e-2 and mean-abs <= 2e-3.  Small
cases compare every element; full-size workloads compare whole sampled query
tiles (dQ) and key tiles (dK, dV)."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_close, assert_within_bound, f64, log, needs_gpu, per_head_f64
from workloads import MaskSpecData, ScoreModData, alibi_slopes, make_config, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run(tensors, spec_data, mod_data, scale=None, layout="bhtd"):
    from block_sparse_masked_build_amd import api
    spec = api.from_spec_data(spec_data)
    mod = None
    if mod_data is not None and (mod_data.alibi_slopes is not None or mod_data.softcap is not None):
        mod = api.score_mod(mod_data.alibi_slopes, mod_data.softcap)
    bm = api.build_block_mask(spec)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    if layout == "bthd":  # same values, [B, T, H, D] memory viewed as [B, H, T, D]
        q, k, v, do = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v, do))
    out, lse = api.flex_attention_fwd(q, k, v, bm, spec, mod, scale)
    dq, dk, dv = api.flex_attention_bwd(q, k, v, out, lse, do, bm, spec, mod, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _full(tensors, spec, mod, B, H, T, ctx, scale=None, derived=False, layout="bhtd"):
    """Every element of dQ, dK, dV: the fixed bar, or with derived=True the
    operand bound (parity_utils)."""
    dq, dk, dv = _run(tensors, spec, mod, scale, layout)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            rq, rk, rv, mq, mk, mv = oracle.backward_dense(Q, K, V, dO, spec, mod, b, h, scale, with_mass=True)
            for name, got, ref, mass in (("dq", dq, rq, mq), ("dk", dk, rk, mk), ("dv", dv, rv, mv)):
                if derived:
                    assert_within_bound(f64(got[b, h]), ref, mass, f"{ctx} b{b} h{h} {name}")
                else:
                    assert_close(f64(got[b, h]), ref, f"{ctx} b{b} h{h} {name}")


def _random_case(rng, it):
    T = int(rng.choice([128, 256, 384, 512]))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    docs = None
    if rng.integers(0, 3) > 0:
        mb = B if rng.integers(0, 2) else 1
        if rng.integers(0, 4) == 0:
            docs = rng.integers(0, 3, size=(mb, T)).astype(np.int32)
        else:
            docs = np.stack([np.cumsum(rng.random(T) < 1.0 / rng.integers(8, 200)).astype(np.int32)
                             for _ in range(mb)])
    window, sinks = None, 0
    if rng.integers(0, 2):
        window = int(rng.choice([1, 17, 64, 128, 129, 300]))
        if rng.integers(0, 2):
            sinks = int(rng.choice([1, 4, 130]))
    spec = MaskSpecData(T, causal=bool(rng.integers(0, 4) > 0), document=docs is not None,
                        doc_ids=docs, window=window, sinks=sinks)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(2000 + it)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    return B, H, T, D, spec, mod, tensors


def test_random_small_cases_every_element():
    rng = np.random.default_rng(99)
    for it in range(16):
        B, H, T, D, spec, mod, tensors = _random_case(rng, it)
        ctx = (f"random#{it} B{B} H{H} T{T} D{D} causal={spec.causal} doc={spec.document} "
               f"w={spec.window} s={spec.sinks} alibi={mod.alibi_slopes is not None} cap={mod.softcap}")
        log(f"[bwd] {ctx}")
        _full(tensors, spec, mod, B, H, T, ctx, derived=True)


def test_strided_layout_every_element():
    """[B, T, H, D] memory for every input, so that out, dQ, dK and dV (made
    like the inputs) have row strides H * D: both the row loads and the row
    stores of the kernels follow the strides.  D = 128 and D = 64."""
    rng = np.random.default_rng(7)
    for D in (128, 64):
        B, H, T = 2, 3, 384
        docs = np.cumsum(rng.random((1, T)) < 0.01, axis=1).astype(np.int32)
        spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs, window=200)
        mod = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=20.0)
        g = torch.Generator("cpu").manual_seed(77 + D)
        tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
        ctx = f"strided B{B} H{H} T{T} D{D}"
        log(f"[bwd] {ctx}")
        _full(tensors, spec, mod, B, H, T, ctx, derived=True, layout="bthd")


def test_config1_every_element():
    w = make_config(1)
    log("[bwd] config 1")
    _full(w.tensors(with_dout=True), w.spec, w.mod, w.B, w.H, w.T, "config 1")


def test_config5_shape_every_element_small_T():
    """Config 5 structure (ALiBi + soft-cap 30, per-batch documents) at
    T = 1024 so every element is compared."""
    w = make_config(5, T=1024, H=4)
    log("[bwd] config 5 structure at T=1024")
    _full(w.tensors(), w.spec, w.mod, w.B, w.H, w.T, "config 5 small")


def test_empty_rows_give_zero_gradients():
    T, D = 256, 64
    spec = MaskSpecData(T, causal=True, window=0)
    g = torch.Generator("cpu").manual_seed(6)
    tensors = {n: random_bf16((1, 1, T, D), g) for n in ("q", "k", "v", "dout")}
    log("[bwd] empty rows")
    dq, dk, dv = _run(tensors, spec, None)
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def _sampled(key, q_tiles, k_tiles, bh_pairs, T=None):
    w = make_config(key, T=T)
    log(f"[bwd] config {key}: B{w.B} H{w.H} T{w.T} D{w.D}")
    tensors = w.tensors(with_dout=True)
    dq, dk, dv = _run(tensors, w.spec, w.mod)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in bh_pairs:
        Q, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
        rows = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in q_tiles])
        rq = oracle.backward_dq_rows(Q, K, V, dO, w.spec, w.mod, b, h, rows)
        mx, mn = assert_close(f64(dq[b, h])[rows], rq, f"config {key} b{b} h{h} dq")
        log(f"  b{b} h{h} dq: max-abs {mx:.2e} mean-abs {mn:.2e}")
        cols = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in k_tiles])
        rk, rv = oracle.backward_dkdv_cols(Q, K, V, dO, w.spec, w.mod, b, h, cols)
        mx, mn = assert_close(f64(dk[b, h])[cols], rk, f"config {key} b{b} h{h} dk")
        log(f"  b{b} h{h} dk: max-abs {mx:.2e} mean-abs {mn:.2e}")
        mx, mn = assert_close(f64(dv[b, h])[cols], rv, f"config {key} b{b} h{h} dv")
        log(f"  b{b} h{h} dv: max-abs {mx:.2e} mean-abs {mn:.2e}")


def test_config5_sampled():
    _sampled(5, q_tiles=[0, 77, 127], k_tiles=[0, 50, 127], bh_pairs=[(0, 0), (1, 15)])


def test_config2_sampled():
    _sampled(2, q_tiles=[0, 300, 511], k_tiles=[0, 299, 511], bh_pairs=[(0, 3)])


def test_config4b_sinks_sampled():
    _sampled("4b", q_tiles=[0, 9, 255], k_tiles=[0, 1, 200], bh_pairs=[(0, 11)])


def test_backward_is_deterministic():
    w = make_config(5, T=2048, H=2)
    tensors = w.tensors()
    log("[bwd] determinism")
    a = _run(tensors, w.spec, w.mod)
    b = _run(tensors, w.spec, w.mod)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
