"""Softmax attention with a mask predicate and score modifications, in fp64.
Oracle; test infrastructure only.

What is computed, per batch element b, head h and query position q
(notation: s = score, V_q = set of visible keys of q):

  s_j    = scale * <q, k_j>                      scale = 1/sqrt(D) by default
  ALiBi:   s_j <- s_j - slope[h] * (q - j)        (tutorial "FlexAttention in
                                                   PyTorch", Pattern 3; q the
                                                   query's absolute position,
                                                   q_offset + its index)
  bias:    s_j <- s_j + bias[h, R + clip(q - j, -R, R)]
                                                 (a learned relative-position
                                                   bias, same section; reading
                                                   below)
  cap:     s_j <- c * tanh(s_j / c)              (same section, c = 30 there)
  out_q  = sum_{j in V_q} softmax(s)_j v_j        over visible keys only
  lse_q  = log sum_{j in V_q} exp(s_j)            natural log

The pages fix the mask and score hooks (tutorial, section "The two hooks":
a score_mod edits the logit after the query-key dot product; a mask_mod
removes pairs) and the exact, fused softmax attention they feed (speedrun
notes "FlexAttention", Context paragraph).  Readings taken where they are
silent: the scale is applied before any score modification; ALiBi comes
before the soft-cap when both are on; ALiBi uses absolute positions; a query
with no visible key gives out = 0 and lse = -inf.  The pages name a learned
relative-position bias without fixing its form; the reading here is the
clipped relative position of Shaw, Uszkoreit and Vaswani (2018) with one
scalar per head: a table of 2R + 1 entries per head indexed by the
query-key distance clipped to [-R, R], added like ALiBi before the cap.

Backward, with upstream gradient dO (the pages state that the score
modifications are differentiable and get a fused backward pass -- tutorial,
Pattern 3):
  Delta_q = <dO_q, out_q>
  p_qj    = exp(s_qj - lse_q) on visible pairs, 0 elsewhere
  dP_qj   = <dO_q, v_j>
  g_qj    = p_qj (dP_qj - Delta_q) * (1 - tanh^2(u_qj / c) if capped,
            u = score before the cap; ALiBi is additive and contributes 1)
  dQ_q = scale sum_j g_qj k_j,  dK_j = scale sum_q g_qj q_q,
  dV_j = sum_q p_qj dO_q

Gradient of the same loss with respect to the ALiBi slope of head h (the
pages: a learned relative-position bias trains through the fused backward --
tutorial, Pattern 3).  The slope enters every visible score through
u_qj = ... - slope[h] (q - j), so
  dL/dslope[h] = sum over b and visible (q, j) of g_qj (j - q)
with g as above (the gradient with respect to u).

The same for the bias table: every visible pair adds g_qj to the entry it
reads, so
  dL/dbias[h, R + r] = sum over b and visible (q, j) with clip(q - j, -R, R) = r
                       of g_qj.

Operand masses (for the parity bound of a bf16 implementation).  Each
output element is a sum of products; its "mass" is the same sum with every
factor replaced by its absolute value -- the size of the sum that rounding
its operands to bf16 (unit roundoff u = 2^-8) can disturb, to first order:
  out_qd:  sum_j w_qj |v_jd|                     w = p / l, the softmax weights
  A_q:     sum_d |dO_qd| (|out_qd| + Mout_qd)    Delta_q's error from out in bf16
  Mg_qj:   |g_qj| + p_qj c'_qj A_q               c' = cap derivative (1 uncapped)
  dQ_qd:   scale sum_j Mg_qj |k_jd|
  dK_jd:   scale sum_q Mg_qj |q_qd|
  dV_jd:   sum_q p_qj |dO_qd|
so |computed - exact| <= u * mass + the output's own rounding.  The masses
are sums of absolute values (triangle inequality): mass >= |value|, with
equality when every term has one sign.

Arithmetic columns: by default only keys visible to at least one query of the
row block take part in the arithmetic; the others would enter the softmax as
exp(-inf) = 0 exactly (the tutorial notes that a -inf score is numerically the
same as masking).  restrict=False keeps every column (fully dense), and the
tests check that both give the same values.

All inputs are per (b, h) float64 arrays [T, D] holding the bf16-rounded
values the GPU reads.
"""
from __future__ import annotations

import math

import numpy as np

from .predicate import visible

ROW_CHUNK = 128


def _qoff(spec):
    return int(getattr(spec, "q_offset", 0))


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)


def _scores(Qr, Kc, rows, cols, h, scale, mod, q_offset=0):
    """Returns (u, s): score before the cap and final score, [R, C]; rows are
    query indices (absolute position q_offset + row), cols key positions."""
    s = scale * (Qr @ Kc.T)
    if mod is not None and mod.alibi_slopes is not None:
        slope = float(mod.alibi_slopes[h])
        s = s - slope * ((rows[:, None] + q_offset) - cols[None, :]).astype(np.float64)
    if mod is not None and getattr(mod, "bias_table", None) is not None:
        s = s + np.asarray(mod.bias_table, dtype=np.float64)[h][bias_index(mod, rows + q_offset, cols)]
    u = s
    if mod is not None and mod.softcap is not None:
        c = float(mod.softcap)
        s = c * np.tanh(u / c)
    return u, s


def bias_radius(mod):
    """R of a bias table with 2R + 1 entries per head."""
    n = np.asarray(mod.bias_table).shape[1]
    assert n % 2 == 1, "a bias table has 2R + 1 entries per head"
    return (n - 1) // 2


def bias_index(mod, qpos, cols):
    """Table entry of every (query position, key) pair, [len(qpos), len(cols)]:
    R + the distance q - kv clipped to [-R, R] (one learned scalar per head
    and clipped relative distance)."""
    R = bias_radius(mod)
    d = np.asarray(qpos, dtype=np.int64)[:, None] - np.asarray(cols, dtype=np.int64)[None, :]
    return np.clip(d, -R, R) + R


def _row_block(Q, K, V, spec, mod, b, h, rows, scale, restrict):
    T = K.shape[0]
    allcols = np.arange(T)
    m = visible(spec, b, rows[:, None], allcols[None, :])
    cols = np.nonzero(m.any(axis=0))[0] if restrict else allcols
    m = m[:, cols]
    u, s = _scores(Q[rows], K[cols], rows, cols, h, scale, mod, _qoff(spec))
    s = np.where(m, s, -np.inf)
    return cols, m, u, s


def forward_rows(Q, K, V, spec, mod, b, h, rows, scale=None, restrict=True, with_mass=False):
    """out [R, D] and lse [R] for the query positions `rows` (and the
    operand mass of out, [R, D], with with_mass)."""
    rows = np.asarray(rows, dtype=np.int64)
    D = Q.shape[1]
    sc = _scale(D, scale)
    out = np.zeros((len(rows), V.shape[1]), dtype=np.float64)
    mass = np.zeros_like(out)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    for a in range(0, len(rows), ROW_CHUNK):
        r = rows[a:a + ROW_CHUNK]
        cols, m, _, s = _row_block(Q, K, V, spec, mod, b, h, r, sc, restrict)
        if len(cols) == 0:
            continue
        mx = s.max(axis=1)
        live = np.isfinite(mx)
        mx_safe = np.where(live, mx, 0.0)
        with np.errstate(invalid="ignore"):
            p = np.exp(s - mx_safe[:, None])
        p = np.where(m, p, 0.0)
        ell = p.sum(axis=1)
        o = p @ V[cols]
        ell_safe = np.where(live, ell, 1.0)[:, None]
        with np.errstate(invalid="ignore", divide="ignore"):
            out[a:a + len(r)] = np.where(live[:, None], o / ell_safe, 0.0)
            lse[a:a + len(r)] = np.where(live, mx_safe + np.log(np.where(live, ell, 1.0)), -np.inf)
        if with_mass:
            mass[a:a + len(r)] = np.where(live[:, None], (p @ np.abs(V[cols])) / ell_safe, 0.0)
    if with_mass:
        return out, lse, mass
    return out, lse


def forward_dense(Q, K, V, spec, mod, b, h, scale=None, restrict=True, with_mass=False):
    """out [T, D], lse [T] for every query position (and out's operand mass)."""
    return forward_rows(Q, K, V, spec, mod, b, h, np.arange(Q.shape[0]), scale, restrict, with_mass)


def _grad_block(Q, K, V, dO, spec, mod, b, h, rows, cols_sel, out_r, lse_r, sc, with_cap=False):
    """g [R, C], p [R, C] on rows x cols_sel (visible pairs only), and with
    with_cap the cap derivative c' [R, C] (ones without a cap)."""
    m = visible(spec, b, rows[:, None], cols_sel[None, :])
    u, s = _scores(Q[rows], K[cols_sel], rows, cols_sel, h, sc, mod, _qoff(spec))
    live = np.isfinite(lse_r)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp(s - np.where(live, lse_r, 0.0)[:, None])
    p = np.where(m & live[:, None], p, 0.0)
    delta = np.sum(dO[rows] * out_r, axis=1)
    dP = dO[rows] @ V[cols_sel].T
    g = p * (dP - delta[:, None])
    cprime = np.ones_like(g)
    if mod is not None and mod.softcap is not None:
        c = float(mod.softcap)
        cprime = 1.0 - np.tanh(u / c) ** 2
        g = g * cprime
    if with_cap:
        return g, p, cprime
    return g, p


def _delta_mass(dO_r, out_r, mout_r):
    """A_q = sum_d |dO_qd| (|out_qd| + Mout_qd): what rounding out to bf16
    (and its own operand error) can move Delta_q, over u."""
    return np.sum(np.abs(dO_r) * (np.abs(out_r) + mout_r), axis=1)


def _mg(g, p, cprime, A_r):
    """Mg_qj = |g_qj| + p_qj c'_qj A_q."""
    return np.abs(g) + p * cprime * A_r[:, None]


def backward_dense(Q, K, V, dO, spec, mod, b, h, scale=None, with_mass=False):
    """dQ, dK, dV [T, D] (small T); with with_mass also their operand masses
    (mass_dQ, mass_dK, mass_dV)."""
    T, D = Q.shape
    sc = _scale(D, scale)
    out, lse, mout = forward_dense(Q, K, V, spec, mod, b, h, scale, with_mass=True)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    mQ, mK, mV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    allcols = np.arange(K.shape[0])
    for a in range(0, T, ROW_CHUNK):
        r = np.arange(a, min(T, a + ROW_CHUNK))
        g, p, cp = _grad_block(Q, K, V, dO, spec, mod, b, h, r, allcols, out[r], lse[r], sc, with_cap=True)
        dQ[r] = sc * (g @ K)
        dK += sc * (g.T @ Q[r])
        dV += p.T @ dO[r]
        if with_mass:
            mg = _mg(g, p, cp, _delta_mass(dO[r], out[r], mout[r]))
            mQ[r] = sc * (mg @ np.abs(K))
            mK += sc * (mg.T @ np.abs(Q[r]))
            mV += p.T @ np.abs(dO[r])
    if with_mass:
        return dQ, dK, dV, mQ, mK, mV
    return dQ, dK, dV


def backward_dq_rows(Q, K, V, dO, spec, mod, b, h, rows, scale=None, with_mass=False):
    """dQ for the query positions `rows` [R, D] (and its operand mass)."""
    rows = np.asarray(rows, dtype=np.int64)
    T, D = Q.shape
    sc = _scale(D, scale)
    out, lse, mout = forward_rows(Q, K, V, spec, mod, b, h, rows, scale, with_mass=True)
    dQ = np.zeros((len(rows), D), dtype=np.float64)
    mQ = np.zeros_like(dQ)
    for a in range(0, len(rows), ROW_CHUNK):
        r = rows[a:a + ROW_CHUNK]
        m = visible(spec, b, r[:, None], np.arange(K.shape[0])[None, :])
        cols = np.nonzero(m.any(axis=0))[0]
        if len(cols) == 0:
            continue
        sl = slice(a, a + len(r))
        g, p, cp = _grad_block(Q, K, V, dO, spec, mod, b, h, r, cols, out[sl], lse[sl], sc, with_cap=True)
        dQ[sl] = sc * (g @ K[cols])
        if with_mass:
            mQ[sl] = sc * (_mg(g, p, cp, _delta_mass(dO[r], out[sl], mout[sl])) @ np.abs(K[cols]))
    if with_mass:
        return dQ, mQ
    return dQ


def backward_dkdv_cols(Q, K, V, dO, spec, mod, b, h, cols, scale=None, with_mass=False):
    """dK, dV for the key positions `cols` [C, D]: sums over every query that
    sees at least one of them, with that query's own forward recomputed (and
    their operand masses with with_mass)."""
    cols = np.asarray(cols, dtype=np.int64)
    T, D = Q.shape
    sc = _scale(D, scale)
    seen = visible(spec, b, np.arange(Q.shape[0])[:, None], cols[None, :]).any(axis=1)
    rows = np.nonzero(seen)[0]
    dK = np.zeros((len(cols), D), dtype=np.float64)
    dV = np.zeros((len(cols), V.shape[1]), dtype=np.float64)
    mK, mV = np.zeros_like(dK), np.zeros_like(dV)
    if len(rows) == 0:
        return (dK, dV, mK, mV) if with_mass else (dK, dV)
    out, lse, mout = forward_rows(Q, K, V, spec, mod, b, h, rows, scale, with_mass=True)
    for a in range(0, len(rows), ROW_CHUNK):
        r = rows[a:a + ROW_CHUNK]
        sl = slice(a, a + len(r))
        g, p, cp = _grad_block(Q, K, V, dO, spec, mod, b, h, r, cols, out[sl], lse[sl], sc, with_cap=True)
        dK += sc * (g.T @ Q[r])
        dV += p.T @ dO[r]
        if with_mass:
            mK += sc * (_mg(g, p, cp, _delta_mass(dO[r], out[sl], mout[sl])).T @ np.abs(Q[r]))
            mV += p.T @ np.abs(dO[r])
    if with_mass:
        return dK, dV, mK, mV
    return dK, dV


def slope_grad_dense(Q, K, V, dO, spec, mod, b, h, scale=None, out=None, lse=None):
    """(dL/dslope[h] for batch element b, sum of |g_qj (j - q)|) over every
    visible pair (small T).  The second value bounds the sum's conditioning:
    the rows of g sum to zero without a cap, so the terms cancel heavily.
    out, lse: the forward's outputs as a backward receives them (its inputs
    Delta = <dO, out> and p = exp(s - lse) are formed from them); by default
    they are computed here in fp64."""
    T, D = Q.shape
    sc = _scale(D, scale)
    if out is None or lse is None:
        out, lse = forward_dense(Q, K, V, spec, mod, b, h, scale)
    allcols = np.arange(K.shape[0])
    total = 0.0
    mass = 0.0
    for a in range(0, T, ROW_CHUNK):
        r = np.arange(a, min(T, a + ROW_CHUNK))
        g, _ = _grad_block(Q, K, V, dO, spec, mod, b, h, r, allcols, out[r], lse[r], sc)
        term = g * (allcols[None, :] - (r[:, None] + _qoff(spec))).astype(np.float64)
        total += float(term.sum())
        mass += float(np.abs(term).sum())
    return total, mass


def bias_grad_dense(Q, K, V, dO, spec, mod, b, h, scale=None, out=None, lse=None, with_pmass=False):
    """(dL/dbias[h, :] for batch element b, the same sums of |g|), float64
    [2R + 1] each, over every visible pair (small T).  out, lse: as for
    slope_grad_dense.  with_pmass also returns, per entry, the sum over its
    pairs of p c' (sum_d |dO_qd v_jd| + sum_d |dO_qd out_qd|): the size of
    the dot products dP and Delta that g subtracts, which bounds what
    rounding them moves g by."""
    T, D = Q.shape
    sc = _scale(D, scale)
    R = bias_radius(mod)
    if out is None or lse is None:
        out, lse = forward_dense(Q, K, V, spec, mod, b, h, scale)
    allcols = np.arange(K.shape[0])
    grad = np.zeros(2 * R + 1, dtype=np.float64)
    mass = np.zeros(2 * R + 1, dtype=np.float64)
    pmass = np.zeros(2 * R + 1, dtype=np.float64)
    for a in range(0, T, ROW_CHUNK):
        r = np.arange(a, min(T, a + ROW_CHUNK))
        g, p, cp = _grad_block(Q, K, V, dO, spec, mod, b, h, r, allcols, out[r], lse[r], sc, with_cap=True)
        idx = bias_index(mod, r + _qoff(spec), allcols).ravel()
        grad += np.bincount(idx, weights=g.ravel(), minlength=2 * R + 1)
        mass += np.bincount(idx, weights=np.abs(g).ravel(), minlength=2 * R + 1)
        if with_pmass:
            dots = np.abs(dO[r]) @ np.abs(V).T + np.sum(np.abs(dO[r] * out[r]), axis=1)[:, None]
            pmass += np.bincount(idx, weights=(p * cp * dots).ravel(), minlength=2 * R + 1)
    if with_pmass:
        return grad, mass, pmass
    return grad, mass
