"""GPU parity of the decoding step (one query per (batch, head) at position
kv_len - 1; tutorial "FlexAttention in PyTorch", "Decoding and paged KV
caches") against the fp64 oracle: the oracle's forward row kv_len - 1 with the
decode query placed there, on the same bf16-rounded inputs.  Bounds as the
forward: max-abs 2e-2, mean-abs 2e-3 on out, 1e-3 on lse."""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_close, assert_lse_close, f64, log, needs_gpu
from workloads import MaskSpecData, ScoreModData, alibi_slopes, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _case(B, H, T, D, spec, mod, seed, heads=None, ctx=""):
    from block_sparse_masked_build_amd import api
    g = torch.Generator("cpu").manual_seed(seed)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, T, D), g)
    v = random_bf16((B, H, T, D), g)
    s = api.from_spec_data(spec)
    m = None
    if mod is not None and (mod.alibi_slopes is not None or mod.softcap is not None):
        m = api.score_mod(mod.alibi_slopes, mod.softcap)
    out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), s, m)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        for h in (heads if heads is not None else range(H)):
            Qf = np.zeros((T, D))
            Qf[T - 1] = q[b, h, 0].double().numpy()
            ro, rl = oracle.forward_rows(Qf, k[b, h].double().numpy(), v[b, h].double().numpy(), spec, mod, b, h,
                                         np.array([T - 1]))
            mx, mn = assert_close(f64(out[b, h]), ro, f"{ctx} b{b} h{h}")
            assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"{ctx} b{b} h{h}")
    log(f"  {ctx}: ok")


def test_documents_alibi_softcap():
    T, B, H = 1024, 2, 4
    rng = np.random.default_rng(51)
    docs = np.stack([np.cumsum(rng.random(T) < 1 / 200).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(T, causal=True, document=True, doc_ids=docs)
    log("[decode] B2 H4 T1024 D128, per-batch documents, ALiBi + soft-cap 30")
    _case(B, H, T, 128, spec, ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0), 52, ctx="docs+mods")


def test_window_with_sinks():
    T = 2048
    spec = MaskSpecData(T, causal=True, window=300, sinks=4)
    log("[decode] B1 H3 T2048 D64, window 300 + 4 sinks")
    _case(1, 3, T, 64, spec, None, 53, ctx="window+sinks")


def test_scattered_documents_no_causal():
    T = 1536
    rng = np.random.default_rng(54)
    docs = rng.integers(0, 3, size=(1, T)).astype(np.int32)
    spec = MaskSpecData(T, causal=False, document=True, doc_ids=docs)
    log("[decode] B2 H2 T1536 D128, scattered documents, no causal term, soft-cap 5")
    _case(2, 2, T, 128, spec, ScoreModData(softcap=5.0), 55, ctx="scattered docs")


def test_nothing_visible_gives_zero_and_neg_inf():
    from block_sparse_masked_build_amd import api
    T, D = 512, 64
    spec = api.mask_spec(T, causal=True, window=0)
    g = torch.Generator("cpu").manual_seed(56)
    q, k, v = (random_bf16(sh, g).cuda() for sh in ((1, 2, 1, D), (1, 2, T, D), (1, 2, T, D)))
    log("[decode] window 0: nothing visible")
    out, lse = api.flex_attention_decode(q, k, v, spec, None)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_sinks_32k_shape():
    """The sinks workload's shape (B1 H16 S32768 D64, window 1024 | 4 sinks):
    a decoding step over its whole cache, three heads checked."""
    T = 32768
    spec = MaskSpecData(T, causal=True, window=1024, sinks=4)
    log("[decode] B1 H16 T32768 D64, window 1024 + 4 sinks")
    _case(1, 16, T, 64, spec, None, 57, heads=[0, 7, 15], ctx="32K sinks")


def test_dense_causal_64k_alibi():
    """One 64K cache, plain causal with ALiBi (every key visible: 128 chunks
    merged), D = 128, two heads checked."""
    T, H = 65536, 2
    spec = MaskSpecData(T, causal=True)
    log("[decode] B1 H2 T65536 D128 causal, ALiBi")
    _case(1, H, T, 128, spec, ScoreModData(alibi_slopes=alibi_slopes(H)), 58, ctx="64K causal")
