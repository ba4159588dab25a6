"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare.

Tolerances for bf16 outputs against the fp64 oracle:
  * the five workloads: max-abs 2e-2 and mean-abs 2e-3 (fixed bar);
  * randomized edge cases, whose outputs can reach |x| ~ 4 and more (tiny
    windows concentrate the softmax): |err| <= 2e-2 + 2^-8 |ref| per element
    and mean-abs 2e-3.  Rounding the exact value to bf16 alone costs up to
    |x| 2^-9, and the bf16 probabilities / score gradients fed to the matrix
    cores cost about as much again.
lse (fp32): max-abs 1e-3."""
import numpy as np
import pytest
import torch

import oracle

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3

BM_NAMES = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices",
            "q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices",
            "kv_order", "q_order")

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU visible")


def log(msg):
    print(msg, flush=True)


def oracle_block_mask(spec_data):
    ref = oracle.block_mask_lists(oracle.tile_counts(spec_data))
    if spec_data.document:
        ref["doc_range"] = oracle.document_ranges(spec_data)
    return ref


def gpu_block_mask(spec_data):
    from block_sparse_masked_build_amd import api
    spec = api.from_spec_data(spec_data)
    bm = api.build_block_mask(spec)
    torch.cuda.synchronize()
    names = BM_NAMES + (("doc_range",) if spec_data.document else ())
    return spec, bm, {n: getattr(bm, n).cpu().numpy() for n in names}


def assert_block_masks_equal(gpu, ref, ctx=""):
    for n in ref:
        a, b = gpu[n], ref[n]
        assert a.shape == b.shape, (ctx, n, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{ctx} {n} differs at {bad.tolist()}: "
                                 f"gpu {[a[tuple(x)] for x in bad]} oracle {[b[tuple(x)] for x in bad]}")


def f64(t):
    return t.detach().float().cpu().double().numpy()


EDGE_RTOL = 2.0 ** -8


def assert_close(gpu, ref, ctx="", max_abs=MAX_ABS, mean_abs=MEAN_ABS, rtol=0.0):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (ctx, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{ctx}: non-finite values"
    err = np.abs(gpu - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    if rtol == 0.0:
        assert mx <= max_abs and mn <= mean_abs, f"{ctx}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    else:
        excess = err - (max_abs + rtol * np.abs(ref))
        worst = float(excess.max()) if err.size else -1.0
        assert worst <= 0.0 and mn <= mean_abs, (
            f"{ctx}: max-abs {mx:.3e} (bound exceeded by {worst:.3e}) mean-abs {mn:.3e}")
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
