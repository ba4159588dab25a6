"""GPU parity of the forward pass against the fp64 oracle on the same
bf16-rounded inputs: max-abs <= 2e-2 and mean-abs <= 2e-3 on out, max-abs
<= 1e-3 on lse.  Small cases compare every element; the full-size workloads
compare whole sampled query tiles (every row of them) plus scattered rows."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_close, assert_lse_close, assert_within_bound, f64, log, needs_gpu,
                          per_head_f64)
from workloads import MaskSpecData, ScoreModData, alibi_slopes, make_config, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run_gpu(tensors, spec_data, mod_data, scale=None, layout="bhtd"):
    from block_sparse_masked_build_amd import api
    spec = api.from_spec_data(spec_data)
    mod = None
    if mod_data is not None and (mod_data.alibi_slopes is not None or mod_data.softcap is not None):
        mod = api.score_mod(mod_data.alibi_slopes, mod_data.softcap)
    bm = api.build_block_mask(spec)
    q, k, v = (tensors[n].cuda() for n in ("q", "k", "v"))
    if layout == "bthd":  # same values, [B, T, H, D] memory viewed as [B, H, T, D]
        q, k, v = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    out, lse = api.flex_attention_fwd(q, k, v, bm, spec, mod, scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _compare_rows(tensors, out, lse, spec_data, mod_data, b, h, rows, ctx, scale=None, derived=False):
    """Rows of one (b, h) against the oracle: the fixed bar, or with
    derived=True the operand bound (parity_utils)."""
    Q, K, V = (per_head_f64(tensors[n], b, h) for n in ("q", "k", "v"))
    ro, rl, rm = oracle.forward_rows(Q, K, V, spec_data, mod_data, b, h, rows, scale, with_mass=True)
    go = f64(out[b, h])[rows]
    gl = lse[b, h].double().numpy()[rows]
    if derived:
        mx, mn = assert_within_bound(go, ro, rm, ctx)
    else:
        mx, mn = assert_close(go, ro, ctx)
    assert_lse_close(gl, rl, ctx)
    return mx, mn


def _full_compare(tensors, spec_data, mod_data, B, H, T, ctx, scale=None, layout="bhtd", derived=False):
    out, lse = _run_gpu(tensors, spec_data, mod_data, scale, layout)
    for b in range(B):
        for h in range(H):
            _compare_rows(tensors, out, lse, spec_data, mod_data, b, h, np.arange(T), f"{ctx} b{b} h{h}",
                          scale, derived)


def _random_case(rng, it):
    T = int(rng.choice([128, 256, 384, 640]))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
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
        window = int(rng.choice([1, 17, 64, 128, 129, 300, 5000]))
        if rng.integers(0, 2):
            sinks = int(rng.choice([1, 4, 130]))
    spec = MaskSpecData(T, causal=bool(rng.integers(0, 4) > 0), document=docs is not None,
                        doc_ids=docs, window=window, sinks=sinks)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H) if rng.integers(0, 2) else None,
                       softcap=float(rng.choice([30.0, 5.0])) if rng.integers(0, 2) else None)
    g = torch.Generator("cpu").manual_seed(1000 + it)
    tensors = {n: random_bf16((B, H, T, D), g) for n in ("q", "k", "v")}
    return B, H, T, D, spec, mod, tensors


def test_random_small_cases_every_element():
    rng = np.random.default_rng(77)
    for it in range(24):
        B, H, T, D, spec, mod, tensors = _random_case(rng, it)
        ctx = (f"random#{it} B{B} H{H} T{T} D{D} causal={spec.causal} doc={spec.document} "
               f"w={spec.window} s={spec.sinks} alibi={mod.alibi_slopes is not None} cap={mod.softcap}")
        log(f"[fwd] {ctx}")
        _full_compare(tensors, spec, mod, B, H, T, ctx, derived=True)


def test_config1_every_element():
    w = make_config(1)
    log("[fwd] config 1")
    _full_compare(w.tensors(), w.spec, w.mod, w.B, w.H, w.T, "config 1")


def test_explicit_scale_and_strided_layout():
    w = make_config(1)
    log("[fwd] config 1, scale 0.05, [B,T,H,D] memory")
    _full_compare(w.tensors(), w.spec, w.mod, w.B, w.H, w.T, "scale/strided", scale=0.05,
                  layout="bthd")


def test_empty_rows_give_zero_and_neg_inf():
    """window = 0 with causality leaves no visible key: every tile list is
    empty, out = 0 and lse = -inf."""
    T, D = 256, 64
    spec = MaskSpecData(T, causal=True, window=0)
    g = torch.Generator("cpu").manual_seed(5)
    tensors = {n: random_bf16((1, 2, T, D), g) for n in ("q", "k", "v")}
    log("[fwd] empty rows")
    out, lse = _run_gpu(tensors, spec, None)
    assert torch.all(out == 0)
    assert torch.all(torch.isneginf(lse))


def _sampled(key, tiles, heads, extra_rows=16, seed=0):
    w = make_config(key)
    log(f"[fwd] config {key}: B{w.B} H{w.H} T{w.T} D{w.D}")
    tensors = w.tensors(with_dout=False)
    out, lse = _run_gpu(tensors, w.spec, w.mod)
    rng = np.random.default_rng(seed)
    assert torch.isfinite(out.float()).all()
    for b in range(w.B):
        for h in heads:
            rows = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in tiles if t * 128 < w.T] +
                                  [rng.integers(0, w.T, size=extra_rows)])
            mx, mn = _compare_rows(tensors, out, lse, w.spec, w.mod, b, h, rows, f"config {key} b{b} h{h}")
            log(f"  b{b} h{h}: max-abs {mx:.2e} mean-abs {mn:.2e}")
    return w, out, lse


def test_config2_sampled():
    _sampled(2, tiles=[0, 1, 7, 255, 511], heads=[0, 5])


def test_config2_variants_sampled():
    for key in ("2-causal", "2-window", "2-chunks"):
        _sampled(key, tiles=[0, 9, 511], heads=[3], extra_rows=8)


def test_config3_windows_sampled():
    """The window schedule 64..1792 (step 64): at every one of the 28 steps
    only the device window scalar changes, the block mask is rebuilt and the
    same forward kernel runs.  Each step compares whole query tiles at the
    start, the middle and the end of the sequence (0, 256, 511) on heads 1
    and 4."""
    from block_sparse_masked_build_amd import api
    w = make_config(3)
    assert len(w.windows) == 28
    tensors = w.tensors(with_dout=False)
    spec = api.from_spec_data(w.spec)
    q, k, v = (tensors[n].cuda() for n in ("q", "k", "v"))
    bm = api.empty_block_mask(w.T, 1)
    ws = api.block_mask_workspace(spec)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
    rows = np.concatenate([np.arange(128 * t, 128 * t + 128) for t in (0, 256, 511)])
    for win in w.windows:
        spec.set_window(win)
        api.build_block_mask(spec, out=bm, workspace=ws)
        api.flex_attention_fwd(q, k, v, bm, spec, out=out, lse=lse)
        torch.cuda.synchronize()
        s = MaskSpecData(w.T, causal=True, document=True, doc_ids=w.spec.doc_ids, window=win)
        o_c, l_c = out.cpu(), lse.cpu()
        for h in (1, 4):
            mx, mn = _compare_rows(tensors, o_c, l_c, s, None, 0, h, rows, f"config 3 w={win} h{h}")
        log(f"[fwd] config 3 window {win}: max-abs {mx:.2e} mean-abs {mn:.2e}")


def test_config4_sampled():
    _sampled("4a", tiles=[0, 31, 63], heads=[0, 15])
    _sampled("4b", tiles=[0, 8, 9, 255], heads=[7])


def test_config5_forward_sampled():
    _sampled(5, tiles=[0, 64, 127], heads=[0, 15])


def test_forward_is_deterministic():
    """Repeated forwards on identical inputs are bitwise equal (documents +
    windows 640 and 1792, plain and ALiBi + soft-cap variants)."""
    from block_sparse_masked_build_amd import api
    B, H, T, D = 1, 2, 4096, 128
    rng = np.random.default_rng(11)
    docs = np.cumsum(rng.random(T) < 1 / 300).astype(np.int32)[None]
    g = torch.Generator("cpu").manual_seed(5)
    q, k, v = (random_bf16((B, H, T, D), g).cuda() for _ in range(3))
    for w in (640, 1792):
        for mod in (None, api.score_mod(alibi_slopes(H), 30.0)):
            log(f"[fwd] determinism window {w} mods {mod is not None}")
            spec = api.mask_spec(T, causal=True, doc_ids=docs, window=w)
            bm = api.build_block_mask(spec)
            runs = [api.flex_attention_fwd(q, k, v, bm, spec, mod) for _ in range(4)]
            torch.cuda.synchronize()
            for o, l in runs[1:]:
                assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])
