"""Pins for the oracle's fp64 attention forward and backward (CPU only).

Pins used: torch's scaled_dot_product_attention in fp64 (library routine) for
the unmasked, causal and per-document cases; special cases with closed forms
(window of 1, a two-key row through the soft-cap); invariants from the pages
(masking equals a -inf score, tutorial "The two hooks"); the softmax's row
shift invariance for ALiBi; central finite differences and torch.autograd for
the backward; sum rules of the gradients.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import MaskSpecData, ScoreModData, doc_ids_geometric, alibi_slopes


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def _sdpa(Q, K, V, **kw):
    t = lambda x: torch.from_numpy(x)[None, None]
    return F.scaled_dot_product_attention(t(Q), t(K), t(V), **kw)[0, 0].numpy()


T, D = 384, 32


def test_forward_no_mask_matches_sdpa():
    Q, K, V = (_rand((T, D), s) for s in (1, 2, 3))
    spec = MaskSpecData(T, causal=False)
    out, lse = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    np.testing.assert_allclose(out, _sdpa(Q, K, V), rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_forward_causal_matches_sdpa():
    Q, K, V = (_rand((T, D), s) for s in (4, 5, 6))
    out, _ = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True), None, 0, 0)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, is_causal=True), rtol=0, atol=1e-12)


def test_forward_document_equals_independent_documents():
    """Packed documents (tutorial Pattern 1) = causal attention run on each
    document alone, concatenated."""
    Q, K, V = (_rand((T, D), s) for s in (7, 8, 9))
    docs = doc_ids_geometric(T, 60, np.random.default_rng(3))
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs[None])
    out, _ = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    ref = np.zeros_like(out)
    for d in np.unique(docs):
        idx = np.nonzero(docs == d)[0]
        ref[idx] = _sdpa(Q[idx], K[idx], V[idx], is_causal=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_forward_window_one_and_wide():
    Q, K, V = (_rand((T, D), s) for s in (10, 11, 12))
    out1, lse1 = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True, window=1), None, 0, 0)
    np.testing.assert_allclose(out1, V, rtol=0, atol=1e-14)
    s_self = np.einsum("td,td->t", Q, K) / math.sqrt(D)
    np.testing.assert_allclose(lse1, s_self, rtol=0, atol=1e-12)
    outw, lsew = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True, window=T + 5), None, 0, 0)
    np.testing.assert_allclose(outw, _sdpa(Q, K, V, is_causal=True), rtol=0, atol=1e-12)


def test_forward_sinks_match_explicit_mask():
    """Tutorial Pattern 2 expressed as an explicit boolean mask in SDPA."""
    Q, K, V = (_rand((T, D), s) for s in (13, 14, 15))
    spec = MaskSpecData(T, causal=True, window=50, sinks=4)
    out, _ = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    qi = torch.arange(T)[:, None]
    ki = torch.arange(T)[None, :]
    m = (qi >= ki) & (((qi - ki) < 50) | (ki < 4))
    np.testing.assert_allclose(out, _sdpa(Q, K, V, attn_mask=m), rtol=0, atol=1e-12)


def test_alibi_is_a_column_bias():
    """-slope*(q - kv) = -slope*q + slope*kv: the first term is constant along
    a row, so the output equals SDPA with a per-column bias +slope*kv, and the
    lse shifts by -slope*q."""
    Q, K, V = (_rand((T, D), s) for s in (16, 17, 18))
    H = 8
    slopes = alibi_slopes(H)
    h = 2
    spec = MaskSpecData(T, causal=True)
    out, lse = oracle.forward_dense(Q, K, V, spec, ScoreModData(alibi_slopes=slopes), 0, h)
    sl = float(slopes[h])
    bias = torch.full((T, T), -math.inf, dtype=torch.float64)
    qi = torch.arange(T)[:, None]
    ki = torch.arange(T)[None, :]
    colb = (sl * ki.double()).expand(T, T)
    bias = torch.where(qi >= ki, colb, bias)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, attn_mask=bias), rtol=0, atol=1e-12)
    logits = torch.from_numpy(Q @ K.T / math.sqrt(D)) + bias
    lse_ref = torch.logsumexp(logits, dim=1).numpy() - sl * np.arange(T)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-10)
    out0, _ = oracle.forward_dense(Q, K, V, spec, ScoreModData(alibi_slopes=np.zeros(H, np.float32)), 0, h)
    np.testing.assert_allclose(out0, _sdpa(Q, K, V, is_causal=True), rtol=0, atol=1e-12)


def test_softcap_two_key_closed_form():
    """A row with two visible keys whose raw scores are 0 and c*atanh(1/2):
    the capped scores are 0 and c/2 (tanh(atanh x) = x), so the softmax
    weights are 1/(1+e^{c/2}) and e^{c/2}/(1+e^{c/2})."""
    c = 30.0
    Dd = 4
    Tt = 128
    Q = np.zeros((Tt, Dd))
    K = np.zeros((Tt, Dd))
    V = np.arange(Tt * Dd, dtype=np.float64).reshape(Tt, Dd) / 7.0
    target = c * math.atanh(0.5)
    # row 1 sees keys 0 and 1 (window 2); score(1, 0) = 0, score(1, 1) = target
    Q[1, 0] = 1.0
    K[1, 0] = target * math.sqrt(Dd)
    spec = MaskSpecData(Tt, causal=True, window=2)
    out, lse = oracle.forward_rows(Q, K, V, spec, ScoreModData(softcap=c), 0, 0, np.array([1]))
    w1 = math.exp(c / 2) / (1 + math.exp(c / 2))
    np.testing.assert_allclose(out[0], (1 - w1) * V[0] + w1 * V[1], rtol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(1 + math.exp(c / 2)), rtol=1e-12)


def test_softcap_bounds_and_limit():
    Q, K, V = (_rand((T, D), s) for s in (19, 20, 21))
    Q = Q * 40.0  # large logits so the cap bites
    spec = MaskSpecData(T, causal=True)
    out_big, _ = oracle.forward_dense(Q, K, V, spec, ScoreModData(softcap=1e9), 0, 0)
    np.testing.assert_allclose(out_big, _sdpa(Q, K, V, is_causal=True), rtol=0, atol=1e-9)
    _, lse_c = oracle.forward_dense(Q, K, V, spec, ScoreModData(softcap=30.0), 0, 0)
    # every capped score lies in (-30, 30), so lse < 30 + log(#keys)
    assert np.all(lse_c < 30.0 + np.log(np.arange(1, T + 1)) + 1e-12)


def test_restricted_columns_equal_dense_minus_inf():
    """Skipping keys no query of the block sees = scoring them -inf (tutorial,
    "The two hooks": a -inf score gives the same numerics as a mask)."""
    Q, K, V = (_rand((T, D), s) for s in (22, 23, 24))
    docs = doc_ids_geometric(T, 50, np.random.default_rng(5))
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs[None], window=70)
    mod = ScoreModData(alibi_slopes=alibi_slopes(4), softcap=30.0)
    o1, l1 = oracle.forward_dense(Q, K, V, spec, mod, 0, 1, restrict=True)
    o2, l2 = oracle.forward_dense(Q, K, V, spec, mod, 0, 1, restrict=False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_empty_rows():
    Q, K, V = (_rand((128, 8), s) for s in (25, 26, 27))
    spec = MaskSpecData(128, causal=True, window=0)  # q - kv < 0 with q >= kv: nothing
    out, lse = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    dq, dk, dv = oracle.backward_dense(Q, K, V, _rand((128, 8), 28), spec, None, 0, 0)
    assert not dq.any() and not dk.any() and not dv.any()


# ---------------------------------------------------------------- backward

def _specs_for_bwd(Tt):
    docs = doc_ids_geometric(Tt, 40, np.random.default_rng(9))
    return [
        (MaskSpecData(Tt, causal=True), None),
        (MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None]),
         ScoreModData(alibi_slopes=alibi_slopes(2), softcap=30.0)),
        (MaskSpecData(Tt, causal=True, window=37, sinks=3), ScoreModData(softcap=5.0)),
        (MaskSpecData(Tt, causal=False, document=True, doc_ids=docs[None]),
         ScoreModData(alibi_slopes=alibi_slopes(2))),
    ]


@pytest.mark.parametrize("case", range(4))
def test_backward_finite_differences(case):
    Tt, Dd = 256, 16
    spec, mod = _specs_for_bwd(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 30 + s) * 1.5 for s in range(4))
    h = 1
    dQ, dK, dV = oracle.backward_dense(Q, K, V, dO, spec, mod, 0, h)

    def loss(Qx, Kx, Vx):
        o, _ = oracle.forward_dense(Qx, Kx, Vx, spec, mod, 0, h)
        return float(np.sum(o * dO))

    rng = np.random.default_rng(case)
    eps = 1e-6
    for which, G in (("q", dQ), ("k", dK), ("v", dV)):
        for _ in range(4):
            t, d = int(rng.integers(0, Tt)), int(rng.integers(0, Dd))
            X = {"q": Q, "k": K, "v": V}
            Xp = {n: a.copy() for n, a in X.items()}
            Xm = {n: a.copy() for n, a in X.items()}
            Xp[which][t, d] += eps
            Xm[which][t, d] -= eps
            fd = (loss(Xp["q"], Xp["k"], Xp["v"]) - loss(Xm["q"], Xm["k"], Xm["v"])) / (2 * eps)
            assert abs(fd - G[t, d]) <= 1e-6 * max(1.0, abs(fd)), (which, t, d, fd, G[t, d])


@pytest.mark.parametrize("case", range(4))
def test_backward_matches_autograd(case):
    """Autograd through a dense explicit-mask fp64 reference (tutorial, sharp
    edge 5: check against a dense reference with an explicit mask)."""
    Tt, Dd = 256, 16
    spec, mod = _specs_for_bwd(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 40 + s) for s in range(4))
    h = 1
    dQ, dK, dV = oracle.backward_dense(Q, K, V, dO, spec, mod, 0, h)
    m = torch.from_numpy(oracle.visible(spec, 0, np.arange(Tt)[:, None], np.arange(Tt)[None, :]))
    q, k, v = (torch.from_numpy(x).clone().requires_grad_(True) for x in (Q, K, V))
    s = (q @ k.T) / math.sqrt(Dd)
    if mod is not None and mod.alibi_slopes is not None:
        pos = torch.arange(Tt, dtype=torch.float64)
        s = s - float(mod.alibi_slopes[h]) * (pos[:, None] - pos[None, :])
    if mod is not None and mod.softcap is not None:
        s = mod.softcap * torch.tanh(s / mod.softcap)
    s = s.masked_fill(~m, -math.inf)
    p = torch.softmax(s, dim=1)
    p = torch.nan_to_num(p, nan=0.0)
    o = p @ v
    o.backward(torch.from_numpy(dO))
    for a, b_ in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        np.testing.assert_allclose(a, b_.numpy(), rtol=0, atol=1e-11)


def test_backward_sum_rules():
    """sum_j dV_j = sum of dO over queries that see something; without a cap,
    every row of g sums to zero so sum_j dK_j = 0."""
    Tt, Dd = 256, 16
    spec, _ = _specs_for_bwd(Tt)[1]
    mod = ScoreModData(alibi_slopes=alibi_slopes(2))
    Q, K, V, dO = (_rand((Tt, Dd), 50 + s) for s in range(4))
    _, dK, dV = oracle.backward_dense(Q, K, V, dO, spec, mod, 0, 0)
    np.testing.assert_allclose(dV.sum(0), dO.sum(0), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dK.sum(0), np.zeros(Dd), rtol=0, atol=1e-11)


def test_sampled_backward_paths_match_dense():
    Tt, Dd = 512, 16
    docs = doc_ids_geometric(Tt, 90, np.random.default_rng(2))
    spec = MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None], window=200)
    mod = ScoreModData(alibi_slopes=alibi_slopes(4), softcap=30.0)
    Q, K, V, dO = (_rand((Tt, Dd), 60 + s) for s in range(4))
    dQ, dK, dV = oracle.backward_dense(Q, K, V, dO, spec, mod, 0, 3)
    rows = np.array([0, 5, 127, 128, 300, 511])
    np.testing.assert_allclose(oracle.backward_dq_rows(Q, K, V, dO, spec, mod, 0, 3, rows), dQ[rows],
                               rtol=0, atol=1e-12)
    cols = np.array([0, 1, 130, 255, 256, 400, 511])
    dk, dv = oracle.backward_dkdv_cols(Q, K, V, dO, spec, mod, 0, 3, cols)
    np.testing.assert_allclose(dk, dK[cols], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dV[cols], rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", [1, 3])
def test_slope_gradient_finite_differences(case):
    """dL/dslope[h] against central differences of the fp64 forward in the
    slope (cases with ALiBi; case 1 also has the soft-cap)."""
    Tt, Dd = 256, 16
    spec, mod = _specs_for_bwd(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 70 + s) for s in range(4))
    h = 1
    gs, mass = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, h)
    assert mass > 0

    def loss(slope):
        sl = np.array(mod.alibi_slopes, dtype=np.float64).copy()
        sl[h] = slope
        m2 = ScoreModData(alibi_slopes=sl, softcap=mod.softcap)
        o, _ = oracle.forward_dense(Q, K, V, spec, m2, 0, h)
        return float(np.sum(o * dO))

    s0 = float(mod.alibi_slopes[h])
    eps = 1e-7
    fd = (loss(s0 + eps) - loss(s0 - eps)) / (2 * eps)
    assert abs(fd - gs) <= 1e-6 * max(1.0, abs(fd)), (fd, gs)


@pytest.mark.parametrize("case", [1, 3])
def test_slope_gradient_matches_autograd(case):
    """The same gradient through torch.autograd on a dense explicit-mask fp64
    reference with the slope as a leaf tensor."""
    Tt, Dd = 256, 16
    spec, mod = _specs_for_bwd(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 80 + s) for s in range(4))
    h = 0
    gs, _ = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, h)
    m = torch.from_numpy(oracle.visible(spec, 0, np.arange(Tt)[:, None], np.arange(Tt)[None, :]))
    slope = torch.tensor(float(mod.alibi_slopes[h]), dtype=torch.float64, requires_grad=True)
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    pos = torch.arange(Tt, dtype=torch.float64)
    s = (q @ k.T) / math.sqrt(Dd) - slope * (pos[:, None] - pos[None, :])
    if mod.softcap is not None:
        s = mod.softcap * torch.tanh(s / mod.softcap)
    s = s.masked_fill(~m, -math.inf)
    p = torch.nan_to_num(torch.softmax(s, dim=1), nan=0.0)
    (p @ v).backward(torch.from_numpy(dO))
    assert abs(slope.grad.item() - gs) <= 1e-9 * max(1.0, abs(gs)), (slope.grad.item(), gs)


def test_slope_gradient_takes_the_backward_inputs():
    """Passing the forward's own fp64 out and lse reproduces the default
    exactly, and rounding out to bf16 moves the result by no more than the
    Delta change it causes: |dDelta_q| * sum_j p_qj |j - q| <= |dDelta_q| * T."""
    Tt, Dd = 256, 16
    spec, mod = _specs_for_bwd(Tt)[1]
    Q, K, V, dO = (_rand((Tt, Dd), 90 + s) for s in range(4))
    gs, mass = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, 1)
    out, lse = oracle.forward_dense(Q, K, V, spec, mod, 0, 1)
    gs2, mass2 = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, 1, out=out, lse=lse)
    assert gs2 == gs and mass2 == mass
    out_b = torch.from_numpy(out).to(torch.bfloat16).double().numpy()
    gs3, _ = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, 1, out=out_b, lse=lse)
    bound = float(np.sum(np.abs(np.sum(dO * (out_b - out), axis=1)))) * Tt
    assert gs3 != gs and abs(gs3 - gs) <= bound


@pytest.mark.parametrize("P", [1, 100, 256, T])
def test_forward_prefix_lm_matches_sdpa(P):
    """Prefix-LM (tutorial introduction): a query inside the prefix sees
    exactly the prefix keys, so its row is unmasked attention over K[:P];
    a query after it sees keys 0..q, so its row is the causal row."""
    Q, K, V = (_rand((T, D), s) for s in (31, 32, 33))
    spec = MaskSpecData(T, causal=True, prefix=P)
    out, _ = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    np.testing.assert_allclose(out[:P], _sdpa(Q[:P], K[:P], V[:P]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[P:], _sdpa(Q, K, V, is_causal=True)[P:], rtol=0, atol=1e-12)


# ---------------------------------------------------------- Q_LEN != KV_LEN,
# ragged lengths, composed masks

def _rect_case(Tk, Lq, seed):
    docs = doc_ids_geometric(Tk, 70, np.random.default_rng(seed))
    sq = MaskSpecData(Tk, causal=True, document=True, doc_ids=docs[None], window=150, sinks=3, prefix=20)
    rect = MaskSpecData(Tk, causal=True, document=True, doc_ids=docs[None], window=150, sinks=3, prefix=20,
                        q_len=Lq, q_offset=Tk - Lq)
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), softcap=20.0)
    return sq, rect, mod


@pytest.mark.parametrize("Tk,Lq", [(300, 1), (300, 77), (384, 384), (257, 130)])
def test_rectangular_is_a_slice_of_the_square_problem(Tk, Lq):
    """Queries at the end of the keys (q_offset = KV_LEN - Q_LEN): the forward
    equals rows q_offset.. of the square problem, and the backward equals the
    square backward with dO zero on the first q_offset rows (dQ on the last
    rows, dK and dV everywhere) -- with documents, window, sinks, prefix,
    ALiBi and soft-cap on, so every term sees absolute positions."""
    sq, rect, mod = _rect_case(Tk, Lq, 5)
    off = Tk - Lq
    Q, K, V, dO = (_rand((Tk, 16), 70 + s) for s in range(4))
    o_sq, l_sq = oracle.forward_dense(Q, K, V, sq, mod, 0, 1)
    o_r, l_r = oracle.forward_dense(Q[off:], K, V, rect, mod, 0, 1)
    np.testing.assert_allclose(o_r, o_sq[off:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_r, l_sq[off:], rtol=0, atol=1e-12)
    dO_sq = dO.copy()
    dO_sq[:off] = 0.0
    dq_sq, dk_sq, dv_sq = oracle.backward_dense(Q, K, V, dO_sq, sq, mod, 0, 1)
    dq, dk, dv = oracle.backward_dense(Q[off:], K, V, dO[off:], rect, mod, 0, 1)
    np.testing.assert_allclose(dq, dq_sq[off:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk_sq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_sq, rtol=0, atol=1e-12)
    # the sampled paths agree with the dense one
    rows = np.array([0, Lq - 1])
    np.testing.assert_allclose(oracle.backward_dq_rows(Q[off:], K, V, dO[off:], rect, mod, 0, 1, rows), dq[rows],
                               rtol=0, atol=1e-12)
    cols = np.array([0, Tk // 2, Tk - 1])
    dkc, dvc = oracle.backward_dkdv_cols(Q[off:], K, V, dO[off:], rect, mod, 0, 1, cols)
    np.testing.assert_allclose(dkc, dk[cols], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dvc, dv[cols], rtol=0, atol=1e-12)


def test_ragged_length_matches_sdpa():
    """T = 1000 (not a multiple of 128), causal: torch's SDPA in fp64."""
    Q, K, V = (_rand((1000, D), s) for s in (81, 82, 83))
    out, _ = oracle.forward_dense(Q, K, V, MaskSpecData(1000, causal=True), None, 0, 0)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, is_causal=True), rtol=0, atol=1e-12)


def test_cross_lengths_without_causal_match_sdpa():
    """Q_LEN = 100 queries over KV_LEN = 300 keys, no mask: SDPA fp64."""
    Q, K, V = _rand((100, D), 84), _rand((300, D), 85), _rand((300, D), 86)
    out, _ = oracle.forward_dense(Q, K, V, MaskSpecData(300, causal=False, q_len=100), None, 0, 0)
    np.testing.assert_allclose(out, _sdpa(Q, K, V), rtol=0, atol=1e-12)


def test_table_of_the_standard_combination_gives_the_same_attention():
    """The standard combination written as a truth table gives the same
    outputs and gradients (documents, window, sinks, prefix, mods)."""
    Tt = 256
    docs = doc_ids_geometric(Tt, 50, np.random.default_rng(8))
    spec = MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None], window=60, sinks=5, prefix=9)
    t = 0
    for idx in range(32):
        c, d, w, s, p = (bool(idx & k) for k in (1, 2, 4, 8, 16))
        t |= int((c or p) and d and (w or s)) << idx
    tab = MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None], window=60, sinks=5, prefix=9, table=t)
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), softcap=30.0)
    Q, K, V, dO = (_rand((Tt, 16), 90 + s) for s in range(4))
    for a, b_ in zip(oracle.forward_dense(Q, K, V, spec, mod, 0, 0), oracle.forward_dense(Q, K, V, tab, mod, 0, 0)):
        np.testing.assert_array_equal(a, b_)
    for a, b_ in zip(oracle.backward_dense(Q, K, V, dO, spec, mod, 0, 0),
                     oracle.backward_dense(Q, K, V, dO, tab, mod, 0, 0)):
        np.testing.assert_array_equal(a, b_)


def test_or_of_masks_matches_explicit_mask_sdpa():
    """A composed mask (causal AND window) OR (NOT causal AND same document)
    as a truth table equals SDPA with the same mask written out densely."""
    Tt = 256
    docs = doc_ids_geometric(Tt, 40, np.random.default_rng(9))
    T_C, T_D, T_W = 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0
    table = (T_C & T_W) | ((0xFFFFFFFF ^ T_C) & T_D)
    spec = MaskSpecData(Tt, document=True, doc_ids=docs[None], window=30, table=table)
    Q, K, V = (_rand((Tt, D), 95 + s) for s in range(3))
    q, k = np.arange(Tt)[:, None], np.arange(Tt)[None, :]
    m = ((q >= k) & ((q - k) < 30)) | ((q < k) & (docs[q] == docs[k]))
    out, _ = oracle.forward_dense(Q, K, V, spec, None, 0, 0)
    ref = _sdpa(Q, K, V, attn_mask=torch.from_numpy(m)[None, None])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_rectangular_backward_finite_differences():
    """Central differences of the rectangular forward (8 queries at the end
    of 200 keys, documents, ALiBi + soft-cap)."""
    sq, rect, mod = _rect_case(200, 8, 6)
    Q, K, V, dO = (_rand(sh, 100 + s) * 1.5 for s, sh in enumerate([(8, 16), (200, 16), (200, 16), (8, 16)]))
    dQ, dK, dV = oracle.backward_dense(Q, K, V, dO, rect, mod, 0, 1)

    def loss(Qx, Kx, Vx):
        o, _ = oracle.forward_dense(Qx, Kx, Vx, rect, mod, 0, 1)
        return float(np.sum(o * dO))

    rng = np.random.default_rng(3)
    eps = 1e-6
    for which, G in (("q", dQ), ("k", dK), ("v", dV)):
        X = {"q": Q, "k": K, "v": V}
        for _ in range(4):
            t, d = int(rng.integers(0, X[which].shape[0])), int(rng.integers(0, 16))
            Xp = {n: a.copy() for n, a in X.items()}
            Xm = {n: a.copy() for n, a in X.items()}
            Xp[which][t, d] += eps
            Xm[which][t, d] -= eps
            fd = (loss(Xp["q"], Xp["k"], Xp["v"]) - loss(Xm["q"], Xm["k"], Xm["v"])) / (2 * eps)
            assert abs(fd - G[t, d]) <= 1e-6 * max(1.0, abs(fd)), (which, t, d, fd, G[t, d])


def test_rectangular_slope_gradient_finite_differences():
    """dL/dslope with absolute query positions (q_offset > 0)."""
    sq, rect, mod = _rect_case(200, 40, 7)
    Q, K, V, dO = (_rand(sh, 110 + s) for s, sh in enumerate([(40, 16), (200, 16), (200, 16), (40, 16)]))
    g, _ = oracle.slope_grad_dense(Q, K, V, dO, rect, mod, 0, 1)
    eps = 1e-6

    def loss(delta):
        sl = mod.alibi_slopes.astype(np.float64).copy()
        sl[1] += delta
        o, _ = oracle.forward_dense(Q, K, V, rect, ScoreModData(alibi_slopes=sl, softcap=mod.softcap), 0, 1)
        return float(np.sum(o * dO))

    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd)), (fd, g)
