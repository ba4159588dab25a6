"""A numpy emulation of where a bf16 (or fp16) implementation of the
attention path must round, used to check the parity bound (test
infrastructure; CPU).

The interface fixes three roundings: the forward's output is bf16, so the
backward forms Delta = <dO, out> from the bf16 out; and a bf16 matrix-core
implementation feeds the probabilities P to the PV product and the score
gradients dS to the dQ / dK products as bf16 operands.  Every other step is
done here in fp64.  Outputs are rounded to bf16 at the end, as the GPU
returns them.  The exact values come from the oracle.
"""
import numpy as np
import torch

from oracle import attention as oa
from oracle import visible


def bf16(x):
    """Round to nearest-even bf16, returned as float64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def f16(x):
    """Round to nearest-even fp16, returned as float64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float16).double().numpy()


def _emulated_rows(Q, K, V, spec, mod, b, h, rows, sc, rnd=bf16):
    """bf16 out of the forward for `rows` with bf16 probabilities in the PV
    product and the fp64 row sum, and the exact lse."""
    out = np.zeros((len(rows), V.shape[1]))
    lse = np.full(len(rows), -np.inf)
    for a in range(0, len(rows), oa.ROW_CHUNK):
        r = rows[a:a + oa.ROW_CHUNK]
        cols, m, _, s = oa._row_block(Q, K, V, spec, mod, b, h, r, sc, True)
        if len(cols) == 0:
            continue
        mx = s.max(axis=1)
        live = np.isfinite(mx)
        mx0 = np.where(live, mx, 0.0)
        with np.errstate(invalid="ignore"):
            p = np.where(m, np.exp(s - mx0[:, None]), 0.0)
        ell = np.where(live, p.sum(axis=1), 1.0)
        out[a:a + len(r)] = np.where(live[:, None], rnd(rnd(p) @ V[cols] / ell[:, None]), 0.0)
        lse[a:a + len(r)] = np.where(live, mx0 + np.log(ell), -np.inf)
    return out, lse


def emulate_dkdv_cols(Q, K, V, dO, spec, mod, b, h, cols, scale=None, rnd=bf16):
    """dK, dV [C, D] for the key positions `cols` with the bf16 rounding
    points of the interface: Delta from the bf16 out, dS and P rounded to
    bf16 before their products, outputs rounded to bf16."""
    cols = np.asarray(cols, dtype=np.int64)
    D = Q.shape[1]
    sc = oa._scale(D, scale)
    rows = np.nonzero(visible(spec, b, np.arange(Q.shape[0])[:, None], cols[None, :]).any(axis=1))[0]
    dK = np.zeros((len(cols), D))
    dV = np.zeros((len(cols), V.shape[1]))
    if len(rows) == 0:
        return dK, dV
    out_e, lse = _emulated_rows(Q, K, V, spec, mod, b, h, rows, sc, rnd)
    for a in range(0, len(rows), oa.ROW_CHUNK):
        r = rows[a:a + oa.ROW_CHUNK]
        g, p = oa._grad_block(Q, K, V, dO, spec, mod, b, h, r, cols, out_e[a:a + len(r)], lse[a:a + len(r)], sc)
        dK += sc * (rnd(g).T @ Q[r])
        dV += rnd(p).T @ dO[r]
    return rnd(dK), rnd(dV)
