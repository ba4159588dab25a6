"""The parity bound for bf16 outputs (CPU only).

The GPU tests bound each element by
    2e-2 + half_ulp_bf16(|ref|) + 2^-8 * mass
(tests/parity_utils.py), where mass is the oracle's operand mass.  Here:
  * the masses are pinned by the triangle inequality (mass >= |value|), by
    equality when every term of the sum has one sign, and by a closed form
    (a window of one key);
  * a numpy emulation of the interface's bf16 rounding points (P and dS as
    bf16 operands, Delta from the bf16 forward output, bf16 outputs) stays
    within the first-order term u * mass + the output rounding, without the
    2e-2 floor, on random small cases;
  * on the 8K prefix-LM case with ALiBi (B1 H4 T8192 D128, prefix 3000) the
    same emulation misses the fixed 2e-2 bar on dK of the key tile that holds
    the prefix end -- what bf16 operands give, whatever the kernel does --
    and stays inside the derived bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from error_model import bf16, emulate_dkdv_cols
from parity_utils import BF16_U, F16_U, half_ulp_bf16, half_ulp_f16, operand_bound
from workloads import MaskSpecData, ScoreModData, alibi_slopes, doc_ids_geometric


def _rand(shape, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(torch.bfloat16).double().numpy()


def test_half_ulp_bf16():
    assert half_ulp_bf16(1.0) == 2.0 ** -8
    assert half_ulp_bf16(1.99) == 2.0 ** -8
    assert half_ulp_bf16(30.0) == 2.0 ** -4
    assert half_ulp_bf16(-0.3) == 2.0 ** -10
    assert half_ulp_bf16(0.0) == 0.0
    # rounding to bf16 moves a value by at most half_ulp_bf16
    x = np.random.default_rng(1).normal(size=1000) * 10
    assert np.all(np.abs(bf16(x) - x) <= half_ulp_bf16(x))


def _case():
    T, D = 256, 16
    docs = doc_ids_geometric(T, 50, np.random.default_rng(4))
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs[None], window=90)
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), softcap=20.0)
    return T, D, spec, mod


def test_masses_bound_the_values():
    T, D, spec, mod = _case()
    Q, K, V, dO = (_rand((T, D), 10 + s) for s in range(4))
    out, _, mo = oracle.forward_dense(Q, K, V, spec, mod, 0, 1, with_mass=True)
    assert np.all(mo >= np.abs(out) - 1e-12) and np.any(mo > np.abs(out) + 1e-3)
    dq, dk, dv, mq, mk, mv = oracle.backward_dense(Q, K, V, dO, spec, mod, 0, 1, with_mass=True)
    for val, mass in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(mass >= np.abs(val) - 1e-12)
        assert np.any(mass > np.abs(val) + 1e-3)


def test_masses_equal_values_for_one_signed_terms():
    """With V >= 0 every term of out is >= 0, so its mass equals out; with
    dO >= 0 the same holds for dV."""
    T, D, spec, mod = _case()
    Q, K, dO = (_rand((T, D), 20 + s) for s in range(3))
    V = np.abs(_rand((T, D), 23))
    out, _, mo = oracle.forward_dense(Q, K, V, spec, mod, 0, 0, with_mass=True)
    np.testing.assert_allclose(mo, out, rtol=1e-12, atol=1e-14)
    _, _, dv, _, _, mv = oracle.backward_dense(Q, K, V, np.abs(dO), spec, mod, 0, 0, with_mass=True)
    np.testing.assert_allclose(mv, dv, rtol=1e-12, atol=1e-14)


def test_mass_closed_form_window_of_one():
    """A window of one key: each query sees only itself, so out_q = v_q,
    Mout_q = |v_q|, p = 1 and g = dO.v - dO.out = 0.  Then dK = 0 and its
    mass is the Delta term alone: scale |q_j| sum_d |dO_jd| (|v_jd| + |v_jd|)."""
    T, D = 128, 8
    spec = MaskSpecData(T, causal=True, window=1)
    Q, K, V, dO = (_rand((T, D), 30 + s) for s in range(4))
    dq, dk, dv, mq, mk, mv = oracle.backward_dense(Q, K, V, dO, spec, None, 0, 0, with_mass=True)
    sc = 1.0 / math.sqrt(D)
    A = np.sum(np.abs(dO) * 2 * np.abs(V), axis=1)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(mk, sc * A[:, None] * np.abs(Q), rtol=1e-12)
    np.testing.assert_allclose(mq, sc * A[:, None] * np.abs(K), rtol=1e-12)
    np.testing.assert_allclose(mv, np.abs(dO), rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_emulated_bf16_errors_within_first_order_term(seed):
    """Random small cases (documents, window, ALiBi + soft-cap, larger-than-
    unit inputs so that errors are visible): the emulated bf16 dK and dV
    differ from the exact ones by at most u * mass + the output's own
    rounding (2 half-ulps: the computed value may sit in the next binade),
    with 5% for second-order terms."""
    T, D = 256, 32
    rng = np.random.default_rng(seed)
    docs = np.cumsum(rng.random(T) < 1 / 80).astype(np.int32)
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs[None], window=int(rng.integers(40, 200)))
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), softcap=float(rng.choice([5.0, 30.0])))
    Q, K, V, dO = (_rand((T, D), 100 * seed + s, 2.0) for s in range(4))
    cols = np.arange(T)
    rk, rv, mk, mv = oracle.backward_dkdv_cols(Q, K, V, dO, spec, mod, 0, 1, cols, with_mass=True)
    ek, ev = emulate_dkdv_cols(Q, K, V, dO, spec, mod, 0, 1, cols)
    for e, r, m in ((ek, rk, mk), (ev, rv, mv)):
        err = np.abs(e - r)
        assert np.all(err <= 1.05 * BF16_U * m + 2 * half_ulp_bf16(r) + 1e-12)
        assert err.max() > 0  # the emulation does round


def test_alibi_prefix_8k_dk_error_is_bf16_rounding():
    """B1 H4 T8192 D128, causal + prefix 3000, ALiBi slopes 2^(-8(h+1)/4),
    head 0, key tile 23 (it holds the prefix end): the emulated bf16 dK
    misses the fixed 2e-2 bar (dK reaches |x| ~ 30 there, whose bf16 spacing
    alone is 0.125) and stays within the derived bound."""
    T, H, D, P = 8192, 4, 128, 3000
    spec = MaskSpecData(T, causal=True, prefix=P)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H))
    g = torch.Generator("cpu").manual_seed(44)
    t = {n: torch.randn((1, H, T, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
         for n in ("q", "k", "v", "dout")}
    Q, K, V, dO = (t[n][0, 0].double().numpy() for n in ("q", "k", "v", "dout"))
    cols = np.arange(23 * 128, 24 * 128)
    rk, rv, mk, mv = oracle.backward_dkdv_cols(Q, K, V, dO, spec, mod, 0, 0, cols, with_mass=True)
    ek, ev = emulate_dkdv_cols(Q, K, V, dO, spec, mod, 0, 0, cols)
    err = np.abs(ek - rk)
    print(f"emulated dK max-abs {err.max():.3e} at |ref| {np.abs(rk).flat[np.argmax(err)]:.2f}; "
          f"max |dK| {np.abs(rk).max():.2f}")
    assert err.max() > 2e-2
    assert np.all(err <= operand_bound(rk, mk))
    assert np.all(np.abs(ev - rv) <= operand_bound(rv, mv))


@pytest.mark.parametrize("seed", [1, 2])
def test_fp16_emulation_within_the_f16_bound(seed):
    """The same emulation with fp16 rounding points (fp16 inputs, P and dS
    operands, out and outputs) stays within the fp16 operand bound, far
    below what bf16 rounding gives on the same inputs.  The first-order
    term alone does not hold everywhere in fp16: probabilities below 2^-14
    are subnormal and round by up to 2^-25 absolute, not 2^-11 relative;
    over at most T terms of |dO| < 8 that adds under 7e-5, which the fixed
    fp16 term (2e-3) covers."""
    from error_model import f16
    T, D = 256, 32
    rng = np.random.default_rng(300 + seed)
    docs = np.cumsum(rng.random(T) < 1 / 80).astype(np.int32)
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs[None], window=int(rng.integers(40, 200)))
    mod = ScoreModData(alibi_slopes=alibi_slopes(2), softcap=30.0)
    Q, K, V, dO = (f16(_rand((T, D), 300 * seed + s, 2.0)) for s in range(4))
    cols = np.arange(T)
    rk, rv, mk, mv = oracle.backward_dkdv_cols(Q, K, V, dO, spec, mod, 0, 1, cols, with_mass=True)
    ek, ev = emulate_dkdv_cols(Q, K, V, dO, spec, mod, 0, 1, cols, rnd=f16)
    bk, bv = emulate_dkdv_cols(Q, K, V, dO, spec, mod, 0, 1, cols)
    for e, bf, r, m in ((ek, bk, rk, mk), (ev, bv, rv, mv)):
        err = np.abs(e - r)
        assert np.all(err <= 1.05 * F16_U * m + 2 * half_ulp_f16(r) + T * 8 * 2.0 ** -25)
        assert np.all(err <= operand_bound(r, m, fmt="f16"))
        assert np.abs(bf - r).max() > 4 * err.max()  # bf16 rounding is visibly coarser
