"""Pins for the oracle's relative-position bias table (CPU only).

The reading (tutorial "FlexAttention in PyTorch", Pattern 3: a learned
relative-position bias trains through the fused backward): one scalar per
head and query-key distance q - kv, clipped to [-R, R] and added to the
score before the soft-cap.  What pins it, apart from its own formula:
- a constant table is a softmax shift: out unchanged, lse moved by the
  constant (tutorial, Pattern 3 says a score_mod only edits logits);
- a 0 / -1e4 table over distances [0, w) reproduces the window mask of the
  predicate, which is pinned against SDPA and brute force elsewhere; the
  sign of the distance is fixed by it (a table read at kv - q keeps only the
  diagonal);
- a table of -slope d reproduces the ALiBi term, pinned separately;
- the clip: a table widened by copies of its end entries changes nothing;
- the gradient: central finite differences of the fp64 forward in single
  entries and torch.autograd with the table as a leaf of a dense
  explicit-mask reference; without a cap its entries sum to zero (the rows
  of g do), and with ALiBi the slope gradient is minus its first moment.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import MaskSpecData, ScoreModData, alibi_slopes, bias_table, doc_ids_geometric


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).double().numpy()


T, D = 320, 16


def test_bias_index_clips_the_distance():
    mod = ScoreModData(bias_table=np.zeros((1, 7), np.float32))  # R = 3
    assert oracle.bias_radius(mod) == 3
    idx = oracle.bias_index(mod, np.array([0, 5, 100]), np.array([0, 2, 5, 9]))
    # entry R + clip(q - kv, -3, 3)
    np.testing.assert_array_equal(idx, [[3, 1, 0, 0], [6, 6, 3, 0], [6, 6, 6, 6]])


@pytest.mark.parametrize("causal", [True, False])
def test_constant_table_is_a_shift(causal):
    Q, K, V = (_rand((T, D), s) for s in (1, 2, 3))
    docs = doc_ids_geometric(T, 50, np.random.default_rng(4))
    spec = MaskSpecData(T, causal=causal, document=True, doc_ids=docs[None])
    tab = np.full((2, 41), 2.75, np.float32)
    out0, lse0 = oracle.forward_dense(Q, K, V, spec, None, 0, 1)
    out1, lse1 = oracle.forward_dense(Q, K, V, spec, ScoreModData(bias_table=tab), 0, 1)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + 2.75, rtol=0, atol=1e-12)


@pytest.mark.parametrize("w", [1, 37, 200])
def test_window_table_equals_window_mask(w):
    """bias = 0 for 0 <= q - kv < w and -1e4 elsewhere (exp underflows to an
    exact 0 in fp64) on a causal mask = the causal + window predicate."""
    Q, K, V = (_rand((T, D), s) for s in (5, 6, 7))
    R = T
    tab = np.full((1, 2 * R + 1), -1e4, np.float64)
    tab[0, R:R + w] = 0.0
    out_b, lse_b = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True), ScoreModData(bias_table=tab), 0, 0)
    out_w, lse_w = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True, window=w), None, 0, 0)
    np.testing.assert_allclose(out_b, out_w, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_b, lse_w, rtol=0, atol=1e-12)


def test_reversed_distance_would_fail_the_window_pin():
    """The same table read at kv - q keeps only the diagonal: the window pin
    above tells the two readings apart."""
    Q, K, V = (_rand((T, D), s) for s in (5, 6, 7))
    R = T
    tab = np.full((1, 2 * R + 1), -1e4, np.float64)
    tab[0, R:R + 37] = 0.0
    flipped = tab[:, ::-1].copy()
    out_f, _ = oracle.forward_dense(Q, K, V, MaskSpecData(T, causal=True), ScoreModData(bias_table=flipped), 0, 0)
    np.testing.assert_allclose(out_f, V, rtol=0, atol=1e-12)  # each query sees only its own key


def test_linear_table_equals_alibi():
    """bias[R + d] = -slope d with R >= T: the ALiBi term exactly (both in
    fp64; ALiBi with the soft-cap after it, as for the table)."""
    Q, K, V = (_rand((T, D), s) for s in (8, 9, 10))
    docs = doc_ids_geometric(T, 70, np.random.default_rng(5))
    spec = MaskSpecData(T, causal=False, document=True, doc_ids=docs[None])
    slopes = alibi_slopes(4)
    R = T
    d = np.arange(-R, R + 1, dtype=np.float64)
    tab = -slopes.astype(np.float64)[:, None] * d[None, :]
    for cap in (None, 7.0):
        a, la = oracle.forward_dense(Q, K, V, spec, ScoreModData(alibi_slopes=slopes, softcap=cap), 0, 2)
        b, lb = oracle.forward_dense(Q, K, V, spec, ScoreModData(bias_table=tab, softcap=cap), 0, 2)
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lb, la, rtol=0, atol=1e-12)


def test_widened_table_changes_nothing():
    """The clip: entries beyond R repeat the end entries, so a table widened
    to R + 50 with copies of them gives the same scores."""
    Q, K, V = (_rand((T, D), s) for s in (11, 12, 13))
    spec = MaskSpecData(T, causal=False)
    R = 20
    tab = bias_table(2, R, seed=3)
    wide = np.concatenate([np.repeat(tab[:, :1], 50, axis=1), tab, np.repeat(tab[:, -1:], 50, axis=1)], axis=1)
    a, la = oracle.forward_dense(Q, K, V, spec, ScoreModData(bias_table=tab), 0, 1)
    b, lb = oracle.forward_dense(Q, K, V, spec, ScoreModData(bias_table=wide), 0, 1)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def _bwd_cases(Tt):
    docs = doc_ids_geometric(Tt, 40, np.random.default_rng(9))
    return [
        (MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None]), None, 24),
        (MaskSpecData(Tt, causal=True, window=37, sinks=3), 5.0, 50),
        (MaskSpecData(Tt, causal=False, document=True, doc_ids=docs[None]), 30.0, 300),
    ]


@pytest.mark.parametrize("case", range(3))
def test_bias_gradient_finite_differences(case):
    Tt, Dd = 192, 16
    spec, cap, R = _bwd_cases(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 40 + s) for s in range(4))
    tab = bias_table(2, R, seed=case)
    h = 1
    grad, mass = oracle.bias_grad_dense(Q, K, V, dO, spec, ScoreModData(bias_table=tab, softcap=cap), 0, h)

    def loss(t):
        o, _ = oracle.forward_dense(Q, K, V, spec, ScoreModData(bias_table=t, softcap=cap), 0, h)
        return float(np.sum(o * dO))

    # ends (clipped distances), the diagonal, and entries in between
    for e in sorted({0, 1, R - 1, R, R + 1, R + 7, 2 * R - 1, 2 * R}):
        tp = tab.astype(np.float64).copy()
        tm = tp.copy()
        eps = 1e-6
        tp[h, e] += eps
        tm[h, e] -= eps
        fd = (loss(tp) - loss(tm)) / (2 * eps)
        assert abs(fd - grad[e]) <= 1e-7 * max(1.0, mass[e]), (e, fd, grad[e])
    if not spec.causal:
        return
    # no causal pair has a negative distance: those entries get nothing
    assert np.all(grad[:R] == 0.0) and np.all(mass[:R] == 0.0)


@pytest.mark.parametrize("case", range(3))
def test_bias_gradient_matches_autograd(case):
    """The gradient through torch.autograd on a dense explicit-mask fp64
    reference with the table as a leaf (gathered by the clipped distance)."""
    Tt, Dd = 192, 16
    spec, cap, R = _bwd_cases(Tt)[case]
    Q, K, V, dO = (_rand((Tt, Dd), 50 + s) for s in range(4))
    tab = bias_table(2, R, seed=10 + case)
    h = 0
    grad, _ = oracle.bias_grad_dense(Q, K, V, dO, spec, ScoreModData(bias_table=tab, softcap=cap), 0, h)
    m = torch.from_numpy(oracle.visible(spec, 0, np.arange(Tt)[:, None], np.arange(Tt)[None, :]))
    leaf = torch.tensor(tab[h].astype(np.float64), requires_grad=True)
    pos = torch.arange(Tt)
    idx = torch.clamp(pos[:, None] - pos[None, :], -R, R) + R
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    s = (q @ k.T) / math.sqrt(Dd) + leaf[idx]
    if cap is not None:
        s = cap * torch.tanh(s / cap)
    s = s.masked_fill(~m, -math.inf)
    p = torch.nan_to_num(torch.softmax(s, dim=1), nan=0.0)
    (p @ v).backward(torch.from_numpy(dO))
    np.testing.assert_allclose(grad, leaf.grad.numpy(), rtol=0, atol=1e-10)


def test_bias_gradient_sum_rules():
    """Without a cap the entries sum to zero (every row of g does: sum_j
    p (dP - Delta) = <dO, out> - Delta = 0).  With ALiBi also on and R >= T
    (nothing clipped), dL/dslope = sum of g (j - q) = -sum_d d dbias[R + d]."""
    Tt, Dd = 256, 16
    docs = doc_ids_geometric(Tt, 40, np.random.default_rng(2))
    spec = MaskSpecData(Tt, causal=True, document=True, doc_ids=docs[None], window=90)
    Q, K, V, dO = (_rand((Tt, Dd), 60 + s) for s in range(4))
    R = Tt
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), bias_table=bias_table(2, R, seed=7))
    grad, mass = oracle.bias_grad_dense(Q, K, V, dO, spec, mod, 0, 1)
    assert abs(grad.sum()) <= 1e-12 * mass.sum()
    gs, gmass = oracle.slope_grad_dense(Q, K, V, dO, spec, mod, 0, 1)
    d = np.arange(-R, R + 1, dtype=np.float64)
    assert abs(gs - (-(d * grad).sum())) <= 1e-12 * gmass


def test_bias_on_rectangular_queries_uses_absolute_positions():
    """Queries at q_offset + i: the table is read at the absolute distance, so
    the last rows of a square run equal a rectangular run of those rows."""
    Q, K, V = (_rand((T, D), s) for s in (14, 15, 16))
    spec = MaskSpecData(T, causal=True)
    tab = bias_table(1, 64, seed=1)
    mod = ScoreModData(bias_table=tab, softcap=11.0)
    out, lse = oracle.forward_dense(Q, K, V, spec, mod, 0, 0)
    n = 70
    rect = MaskSpecData(T, causal=True, q_len=n, q_offset=T - n)
    o2, l2 = oracle.forward_dense(Q[T - n:], K, V, rect, mod, 0, 0)
    np.testing.assert_allclose(o2, out[T - n:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse[T - n:], rtol=0, atol=1e-12)
