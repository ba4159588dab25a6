"""GPU parity of the ALiBi slope gradient dL/dslope[h] (a learned bias
trains through the fused backward: tutorial "FlexAttention in PyTorch",
Pattern 3) against the fp64 oracle.

The backward takes the forward's out and lse as inputs, so both sides are
given the same ones: the oracle's own forward, out rounded to bf16 and lse to
fp32 (Delta = <dO, out> and p = exp(s - lse) are formed from them on both
sides).  What is left is fp32 against fp64 arithmetic.  S and dP sum exact
bf16 products in fp32.  p comes from an fp32 exp2 whose argument (at most
about 44 in the log2 domain where p matters) carries up to 44 * 2^-24, i.e.
3e-6 relative per term, with rounding signs that vary from term to term.
The terms are summed in fp32 over at most T/64 steps per lane and then in
fixed-order trees.  So the difference stays well under 1e-6 of
sum |g_qj (j - q)| (the oracle's second value), which is the bound below.
Measured: at most 2.3e-8 on every case here.
The terms cancel heavily: the result is 1e-5 .. 2e-2 of that sum on these
inputs.  On the config 5 structure at T = 1024, a wrong sign moves the
result by at least 9e-4 of the sum, and a key offset off by one lane group
(4 keys in half of the scores) by 2e-6 .. 5e-3, on every head.  A uniform
key offset moves it by only 1e-7 .. 2e-5, because each row of g sums to
nearly zero: the gradient itself is nearly blind to such an offset."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import log, needs_gpu, per_head_f64
from workloads import MaskSpecData, ScoreModData, alibi_slopes, make_config, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]

REL_TOL = 1e-6


def _gpu_slopes(tensors, spec_data, mod_data, out, lse):
    from block_sparse_masked_build_amd import api
    spec = api.from_spec_data(spec_data)
    mod = api.score_mod(mod_data.alibi_slopes, mod_data.softcap)
    bm = api.build_block_mask(spec)
    q, k, v, do = (tensors[n].cuda() for n in ("q", "k", "v", "dout"))
    H = q.shape[1]
    ds = torch.full((H,), float("nan"), dtype=torch.float32, device="cuda")
    api.flex_attention_bwd(q, k, v, out.cuda(), lse.cuda(), do, bm, spec, mod, dslopes=ds)
    torch.cuda.synchronize()
    return ds.cpu().double().numpy()


def _check(tensors, spec_data, mod_data, B, H, heads, ctx, fill_gpu_forward=False):
    """Oracle out/lse for the checked heads (the other heads, whose slopes are
    not compared, get the GPU forward's) and the comparison per checked head."""
    T, D = tensors["q"].shape[2], tensors["q"].shape[3]
    if fill_gpu_forward:
        from block_sparse_masked_build_amd import api
        spec = api.from_spec_data(spec_data)
        mod = api.score_mod(mod_data.alibi_slopes, mod_data.softcap)
        bm = api.build_block_mask(spec)
        o, l = api.flex_attention_fwd(*(tensors[n].cuda() for n in ("q", "k", "v")), bm, spec, mod)
        out, lse = o.cpu(), l.cpu()
    else:
        out = torch.zeros((B, H, T, D), dtype=torch.bfloat16)
        lse = torch.zeros((B, H, T), dtype=torch.float32)
    for b in range(B):
        for h in heads:
            Q, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
            o, l = oracle.forward_dense(Q, K, V, spec_data, mod_data, b, h)
            out[b, h] = torch.from_numpy(o).to(torch.bfloat16)
            lse[b, h] = torch.from_numpy(l).to(torch.float32)
    got = _gpu_slopes(tensors, spec_data, mod_data, out, lse)
    for h in heads:
        ref = mass = 0.0
        for b in range(B):
            Q, K, V, dO = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v", "dout"))
            g, m = oracle.slope_grad_dense(Q, K, V, dO, spec_data, mod_data, b, h,
                                           out=out[b, h].double().numpy(), lse=lse[b, h].double().numpy())
            ref += g
            mass += m
        err = abs(got[h] - ref)
        log(f"  {ctx} h{h}: gpu {got[h]:.6e} oracle {ref:.6e} |err|/mass {err / mass:.2e}")
        assert np.isfinite(got[h]) and err <= REL_TOL * mass, (ctx, h, got[h], ref, mass)


def test_config5_structure_small_T():
    """ALiBi + soft-cap 30, per-batch documents (contiguous-run path)."""
    w = make_config(5, T=1024, H=4)
    log("[slopes] config 5 structure at T=1024")
    _check(w.tensors(), w.spec, w.mod, w.B, w.H, range(w.H), "config 5 T1024")


def test_window_with_sinks_alibi_only():
    T, B, H, D = 512, 2, 2, 64
    spec = MaskSpecData(T, causal=True, window=300, sinks=130)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H))
    g = torch.Generator("cpu").manual_seed(31)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    log("[slopes] causal + window 300 + 130 sinks, ALiBi")
    _check(tensors, spec, mod, B, H, range(H), "window+sinks")


def test_scattered_documents_softcap():
    """Document ids that are not contiguous runs (per-key compare path), no
    causal term, soft-cap 5."""
    T, B, H, D = 384, 1, 2, 128
    rng = np.random.default_rng(7)
    docs = rng.integers(0, 3, size=(1, T)).astype(np.int32)
    spec = MaskSpecData(T, causal=False, document=True, doc_ids=docs)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=5.0)
    g = torch.Generator("cpu").manual_seed(32)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v", "dout")}
    log("[slopes] scattered documents, ALiBi + soft-cap 5")
    _check(tensors, spec, mod, B, H, range(H), "scattered docs")


def test_config5_shape_T4096_two_heads():
    """Config 5's shape (B2 H16 D128, ALiBi + soft-cap 30, per-batch
    documents) at T = 4096; heads 0 and 15 (steepest and flattest slope)."""
    w = make_config(5, T=4096)
    log("[slopes] config 5 shape at T=4096, heads 0 and 15")
    _check(w.tensors(), w.spec, w.mod, w.B, w.H, [0, 15], "config 5 T4096", fill_gpu_forward=True)


def test_slope_gradient_deterministic_and_leaves_dq_unchanged():
    """Bitwise-equal slopes over two calls at config 5's full shape, and dQ,
    dK, dV identical to a backward without the slope gradient."""
    from block_sparse_masked_build_amd import api
    w = make_config(5)
    log("[slopes] determinism at config 5 (B2 H16 T16384 D128)")
    t = {n: x.cuda() for n, x in w.tensors().items()}
    spec = api.from_spec_data(w.spec)
    mod = api.score_mod(w.mod.alibi_slopes, w.mod.softcap)
    bm = api.build_block_mask(spec)
    out, lse = api.flex_attention_fwd(t["q"], t["k"], t["v"], bm, spec, mod)
    base = api.flex_attention_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], bm, spec, mod)
    runs = []
    for _ in range(2):
        ds = torch.full((w.H,), float("nan"), dtype=torch.float32, device="cuda")
        grads = api.flex_attention_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], bm, spec, mod, dslopes=ds)
        torch.cuda.synchronize()
        runs.append(ds.cpu())
        for x, y in zip(grads, base):
            assert torch.equal(x, y)
    assert torch.isfinite(runs[0]).all()
    assert torch.equal(runs[0], runs[1])
