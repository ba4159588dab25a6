"""GPU parity of the decoding step (tutorial "FlexAttention in PyTorch",
section "Decoding and paged KV caches"): one query per (batch, head) at
position kv_len - 1 of a cache whose live length kv_len is a device value
inside a bucketed allocation.  The oracle is its forward row kv_len - 1 over
the live keys (mask spec restricted to the first kv_len positions), on the
same bf16-rounded inputs; bounds as the forward (max-abs 2e-2, mean-abs 2e-3
on out, 1e-3 on lse)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_close, assert_lse_close, f64, log, needs_gpu
from workloads import MaskSpecData, ScoreModData, alibi_slopes, random_bf16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _live_spec(spec, L):
    """The predicate restricted to the first L positions."""
    docs = spec.doc_ids[:, :L] if spec.doc_ids is not None else None
    return dataclasses.replace(spec, T=L, doc_ids=docs)


def _oracle_row(q, k, v, spec, mod, b, h, L):
    if L == 0:
        return np.zeros((1, k.shape[-1])), np.array([-np.inf])
    D = k.shape[-1]
    Qf = np.zeros((L, D))
    Qf[L - 1] = q[b, h, 0].double().numpy()
    return oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                               _live_spec(spec, L), mod, b, h, np.array([L - 1]))


def _case(B, H, cap, D, spec, mod, seed, kv_lens, heads=None, ctx="", listed=False):
    """kv_lens: one live length for the batch (int) or one per batch element."""
    from block_sparse_masked_build_amd import api
    g = torch.Generator("cpu").manual_seed(seed)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    m = None
    if mod is not None and (mod.alibi_slopes is not None or mod.softcap is not None):
        m = api.score_mod(mod.alibi_slopes, mod.softcap)
    bm = api.build_block_mask(s) if listed else None
    kvl = kv_lens if isinstance(kv_lens, int) else torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), s, m, kv_len=kvl, block_mask=bm)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        L = kv_lens if isinstance(kv_lens, int) else kv_lens[b]
        for h in (heads if heads is not None else range(H)):
            ro, rl = _oracle_row(q, k, v, spec, mod, b, h, L)
            assert_close(f64(out[b, h]), ro, f"{ctx} b{b} h{h} L{L}")
            assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"{ctx} b{b} h{h} L{L}")
    log(f"  {ctx}: ok")


@pytest.mark.parametrize("L", [1, 127, 129, 32767, 32768])
def test_live_lengths_in_a_32k_cache(L):
    """A 32,768-position allocation, causal, live lengths at the edges of
    tiles and slots (1, 127, 129, 32,767, the full cache)."""
    log(f"[decode] B1 H2 cap 32768 D128 causal, live length {L}")
    _case(1, 2, 32768, 128, MaskSpecData(32768, causal=True), None, 60 + L % 7, L, ctx=f"L={L}")


def test_per_batch_live_lengths_documents_alibi_softcap():
    """Per-batch live lengths and per-batch documents, ALiBi + soft-cap 30,
    capacity 1000 (not a multiple of 128)."""
    cap, B, H = 1000, 3, 4
    rng = np.random.default_rng(51)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 200).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs)
    log("[decode] B3 H4 cap 1000 D128, live lengths 1000/513/64, documents, ALiBi + soft-cap 30")
    _case(B, H, cap, 128, spec, ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0), 52,
          [1000, 513, 64], ctx="docs+mods")


@pytest.mark.parametrize("listed", [False, True])
def test_document_decode_with_and_without_block_mask(listed):
    """Packed documents in a 16K cache: with the block mask the step reads
    only the tiles of the query's row; results equal the oracle either way."""
    cap, B, H = 16384, 2, 2
    rng = np.random.default_rng(57)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 700).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=1024)
    log(f"[decode] B2 H2 cap 16384 D64 documents + window 1024, block mask {listed}")
    _case(B, H, cap, 64, spec, ScoreModData(softcap=30.0), 58, [9000, 16384], ctx=f"docs listed={listed}",
          listed=listed)


def test_window_with_sinks():
    cap = 2048
    spec = MaskSpecData(cap, causal=True, window=300, sinks=4)
    log("[decode] B1 H3 cap 2048 D64, window 300 + 4 sinks, live 1999")
    _case(1, 3, cap, 64, spec, None, 53, 1999, ctx="window+sinks")


def test_window_with_sinks_listed():
    cap = 4096
    spec = MaskSpecData(cap, causal=True, window=300, sinks=4)
    log("[decode] B1 H3 cap 4096 D64, window 300 + 4 sinks, live 3001, block mask")
    _case(1, 3, cap, 64, spec, None, 54, 3001, ctx="window+sinks listed", listed=True)


def test_scattered_documents_no_causal():
    """Without the causal term every live key of the query's document is
    seen; keys beyond the live length never are."""
    cap = 1536
    rng = np.random.default_rng(54)
    docs = rng.integers(0, 3, size=(1, cap)).astype(np.int32)
    spec = MaskSpecData(cap, causal=False, document=True, doc_ids=docs)
    log("[decode] B2 H2 cap 1536 D128, scattered documents, no causal term, soft-cap 5, live 1400")
    _case(2, 2, cap, 128, spec, ScoreModData(softcap=5.0), 55, 1400, ctx="scattered docs")


def test_nothing_visible_gives_zero_and_neg_inf():
    from block_sparse_masked_build_amd import api
    cap, D = 512, 64
    spec = api.mask_spec(cap, causal=True, window=0)
    g = torch.Generator("cpu").manual_seed(56)
    q, k, v = (random_bf16(sh, g).cuda() for sh in ((1, 2, 1, D), (1, 2, cap, D), (1, 2, cap, D)))
    log("[decode] window 0: nothing visible; live length 0")
    for L in (cap, 0):
        out, lse = api.flex_attention_decode(q, k, v, spec, None, kv_len=L)
        torch.cuda.synchronize()
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_sinks_32k_shape():
    """The sinks workload's shape (B1 H16 S32768 D64, window 1024 | 4 sinks):
    a decoding step over the whole cache, three heads checked."""
    cap = 32768
    spec = MaskSpecData(cap, causal=True, window=1024, sinks=4)
    log("[decode] B1 H16 cap 32768 D64, window 1024 + 4 sinks")
    _case(1, 16, cap, 64, spec, None, 57, cap, heads=[0, 7, 15], ctx="32K sinks")


def test_dense_causal_64k_alibi():
    """One 64K cache, plain causal with ALiBi (every key visible: 64 slots
    merged), D = 128, two heads checked."""
    cap, H = 65536, 2
    spec = MaskSpecData(cap, causal=True)
    log("[decode] B1 H2 cap 65536 D128 causal, ALiBi")
    _case(1, H, cap, 128, spec, ScoreModData(alibi_slopes=alibi_slopes(H)), 58, cap, ctx="64K causal")


def test_graph_replay_as_the_cache_grows():
    """The step captured once in a HIP graph with the live length in device
    memory; replays at growing lengths equal eager calls bit for bit."""
    from block_sparse_masked_build_amd import api
    B, H, cap, D = 2, 4, 4096, 128
    rng = np.random.default_rng(59)
    docs = np.cumsum(rng.random(cap) < 1 / 300).astype(np.int32)[None]
    spec = api.mask_spec(cap, causal=True, doc_ids=docs, window=1024)
    bm = api.build_block_mask(spec)
    g = torch.Generator("cpu").manual_seed(59)
    q, k, v = (random_bf16(sh, g).cuda() for sh in ((B, H, 1, D), (B, H, cap, D), (B, H, cap, D)))
    kvl = torch.tensor([100, 100], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = api.decode_workspace(B, H, cap, D)

    def step():
        api.flex_attention_decode(q, k, v, spec, None, kv_len=kvl, block_mask=bm, out=out, lse=lse, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for L0 in (1, 129, 1500, 4095, 4096):
        log(f"[decode] graph replay at live length {L0}")
        kvl.copy_(torch.tensor([L0, max(1, L0 - 77)], dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref = api.flex_attention_decode(q, k, v, spec, None, kv_len=kvl.clone(), block_mask=bm)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), L0


@pytest.mark.parametrize("n,L", [(1, 1), (1, 1000), (4, 4), (4, 4096), (16, 2049), (130, 3000)])
def test_multi_query_decode_on_the_matrix_cores(n, L):
    """A block of n new queries at the end of a live cache (speculative or
    chunked decoding) runs as the rectangular forward over the live keys:
    parity with the oracle's rows L - n .. L - 1, documents + window 700,
    ALiBi + soft-cap 30, capacity 4,096."""
    from block_sparse_masked_build_amd import api
    cap, B, H, D = 4096, 2, 2, 128
    rng = np.random.default_rng(70 + n)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 600).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=700)
    mod = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0)
    log(f"[decode multi] n={n} L={L} cap {cap} B{B} H{H} D{D}")
    g = torch.Generator("cpu").manual_seed(80 + n)
    q = random_bf16((B, H, n, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    s = api.from_spec_data(spec)
    m = api.score_mod(mod.alibi_slopes, mod.softcap)
    out, lse = api.flex_attention_decode_multi(q.cuda(), k.cuda(), v.cuda(), s, L, m)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    rows = np.arange(L - n, L)
    for b in range(B):
        for h in range(H):
            Qf = np.zeros((L, D))
            Qf[rows] = q[b, h].double().numpy()
            ro, rl = oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                                         _live_spec(spec, L), mod, b, h, rows)
            assert_close(f64(out[b, h]), ro, f"multi n{n} L{L} b{b} h{h}")
            assert_lse_close(lse[b, h].double().numpy(), rl, f"multi n{n} L{L} b{b} h{h}")


def test_more_than_65535_batch_heads():
    """B x H = 66,000 (batch and head index the grid's first dimension, which
    takes more than 65,535 workgroups): sampled heads against the oracle."""
    from block_sparse_masked_build_amd import api
    B, H, cap, D, L = 2, 33000, 128, 64, 100
    log(f"[decode] B{B} H{H} cap {cap} D{D}, live length {L}")
    g = torch.Generator("cpu").manual_seed(61)
    q = random_bf16((B, H, 1, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    spec = MaskSpecData(cap, causal=True)
    out, lse = api.flex_attention_decode(q.cuda(), k.cuda(), v.cuda(), api.from_spec_data(spec), None, kv_len=L)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    for b, h in ((0, 0), (0, 32999), (1, 0), (1, 17001), (1, 32999)):
        ro, rl = _oracle_row(q, k, v, spec, None, b, h, L)
        assert_close(f64(out[b, h]), ro, f"b{b} h{h}")
        assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"b{b} h{h}")
