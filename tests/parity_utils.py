"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare.

Tolerances for bf16 outputs against the fp64 oracle:
  * the five workloads: max-abs 2e-2 and mean-abs 2e-3 (the fixed bar);
  * other cases (randomized edge cases, long prefixes with ALiBi), whose
    outputs can be large or sums of thousands of terms: per element
        |err| <= 2e-2 + half_ulp_bf16(|ref|) + 2^-8 * mass
    where half_ulp_bf16 is the rounding of the exact value to the bf16
    output and mass is the oracle's operand mass of the element (the sum it
    is made of, with absolute values): the first-order worst case of rounding
    the matrix-core operands P and dS, and the forward output that Delta is
    formed from, to bf16 (unit roundoff 2^-8); and mean-abs at most a tenth
    of the mean of that bound -- the ratio of the fixed bar (2e-3 to 2e-2),
    to which it reduces for outputs of unit scale, while an output summed
    from hundreds of terms (one key seen by every query) carries its own
    rounding scale into the mean too.
lse (fp32): max-abs 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from schedule_checks import check_schedule

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3

# The eight tile-list arrays: compared bit for bit with the oracle.
BM_NAMES = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices",
            "q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices")
# Scheduling data exported with them: checked by its properties
# (schedule_checks), not against the oracle.
SCHEDULE_NAMES = ("kv_order", "q_order", "doc_range")

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU visible")


def log(msg):
    print(msg, flush=True)


def oracle_block_mask(spec_data):
    return oracle.spec_block_mask_lists(spec_data)


def gpu_block_mask(spec_data):
    from block_sparse_masked_build_amd import api
    spec = api.from_spec_data(spec_data)
    bm = api.build_block_mask(spec)
    torch.cuda.synchronize()
    names = BM_NAMES + SCHEDULE_NAMES[:2] + (("doc_range",) if spec_data.document else ())
    return spec, bm, {n: getattr(bm, n).cpu().numpy() for n in names}


def assert_block_masks_equal(gpu, ref, ctx="", spec=None):
    """The tile lists bit for bit against the oracle's, then the exported
    schedule (work orders, document ranges) by its properties."""
    for n in BM_NAMES:
        a, b = gpu[n], ref[n]
        assert a.shape == b.shape, (ctx, n, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{ctx} {n} differs at {bad.tolist()}: "
                                 f"gpu {[a[tuple(x)] for x in bad]} oracle {[b[tuple(x)] for x in bad]}")
    if "kv_order" in gpu:
        docs = spec.doc_ids if spec is not None and spec.document else None
        check_schedule(gpu, docs, ctx)


def f64(t):
    return t.detach().float().cpu().double().numpy()


BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits, round to nearest)
F16_U = 2.0 ** -11  # unit roundoff of fp16 (11 significant bits)
# fp16 outputs: the fixed part of the bound.  fp16 carries three more bits
# than bf16 and the fp32 arithmetic around the products is far below either,
# so a tenth of the bf16 bar is still generous; a path that rounded its
# operands to bf16 would miss it.
F16_MAX_ABS = 2e-3


def half_ulp_bf16(x):
    """Half the bf16 spacing at |x|: 2^(e - 8) for |x| in [2^e, 2^(e+1))."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(x)  # x = m 2^E, m in [0.5, 1)
    return np.where(x > 0, np.ldexp(1.0, E - 9), 0.0)


def half_ulp_f16(x):
    """Half the fp16 spacing at |x|: 2^(e - 11) for |x| in [2^e, 2^(e+1)),
    and 2^-25 below 2^-14 (subnormals)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(x)
    return np.where(x > 0, np.maximum(np.ldexp(1.0, E - 12), 2.0 ** -25), 0.0)


FORMATS = {"bf16": (BF16_U, half_ulp_bf16, MAX_ABS), "f16": (F16_U, half_ulp_f16, F16_MAX_ABS)}


def operand_bound(ref, mass, max_abs=None, fmt="bf16"):
    """Per-element bound: max_abs + half_ulp(|ref|) + u * mass for the
    output format fmt (bf16 or f16), max_abs by default that format's."""
    u, half_ulp, fixed = FORMATS[fmt]
    return (fixed if max_abs is None else max_abs) + half_ulp(ref) + u * np.asarray(mass, dtype=np.float64)


def assert_within_bound(gpu, ref, mass, ctx="", mean_abs=MEAN_ABS, fmt="bf16"):
    """Every element within operand_bound, and mean-abs within
    mean_abs / MAX_ABS of the mean of that bound (mean_abs for outputs of
    unit scale in bf16)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape == np.shape(mass), (ctx, gpu.shape, ref.shape, np.shape(mass))
    assert np.all(np.isfinite(gpu)), f"{ctx}: non-finite values"
    err = np.abs(gpu - ref)
    if not err.size:
        return 0.0, 0.0
    bound = operand_bound(ref, mass, fmt=fmt)
    worst = int(np.argmax(err - bound))
    mx, mn = float(err.max()), float(err.mean())
    mean_bar = float(bound.mean()) * (mean_abs / MAX_ABS)
    assert err.flat[worst] <= bound.flat[worst] and mn <= mean_bar, (
        f"{ctx}: max-abs {mx:.3e}; worst element {worst} err {err.flat[worst]:.3e} (bound "
        f"{bound.flat[worst]:.3e}, ref {ref.flat[worst]:.3e}); mean-abs {mn:.3e} (bar {mean_bar:.3e})")
    return mx, mn


def assert_close(gpu, ref, ctx="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """The fixed bar: max-abs <= max_abs and mean-abs <= mean_abs."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (ctx, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{ctx}: non-finite values"
    err = np.abs(gpu - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, f"{ctx}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def assert_lse_close(gpu, ref, ctx=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{ctx}: -inf pattern differs"
    fin = ~ninf_r
    if fin.any():
        err = np.abs(gpu[fin] - ref[fin]).max()
        assert err <= LSE_MAX_ABS, f"{ctx}: lse max-abs {err:.3e}"


def to_device(tensors):
    return {k: v.cuda() for k, v in tensors.items()}


def per_head_f64(t, b, h):
    """[T, D] float64 numpy of a bf16 CPU tensor [B, H, T, D]."""
    return t[b, h].double().numpy()
