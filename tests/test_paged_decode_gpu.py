"""GPU parity of the decoding step over a paged key/value cache (tutorial
"FlexAttention in PyTorch", section "Decoding and paged KV caches": the
cache of every sequence is a list of fixed-size pages in a shared pool, a
block table mapping each logical page to its physical one).

Each case scatters a contiguous cache into a shuffled pool (with spare
pages) and checks that the paged step gives the contiguous step's results
bit for bit, and, for a few heads, the oracle's forward row kv_len - 1 over
the live keys within the forward's per-element operand bound.  Table
entries for pages past the live length hold out-of-range values: they must
never be read."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_lse_close, assert_within_bound, f64, log, needs_gpu
from workloads import MaskSpecData, ScoreModData, alibi_slopes, bias_table, random_bf16, random_f16

pytestmark = [pytest.mark.gpu, needs_gpu]


def _page(k, v, page, kv_lens, spare, seed):
    """Scatter k, v [B, H, cap, D] into pools of B * cap / page + spare pages
    in a shuffled order; logical pages at or past each live length get a
    table entry outside the pool."""
    B, H, cap, D = k.shape
    nl = cap // page
    npool = B * nl + spare
    perm = np.random.default_rng(seed).permutation(npool)
    table = perm[:B * nl].reshape(B, nl).astype(np.int32)
    kp = torch.zeros((npool, H, page, D), dtype=k.dtype)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for j in range(nl):
            kp[table[b, j]] = k[b, :, j * page:(j + 1) * page]
            vp[table[b, j]] = v[b, :, j * page:(j + 1) * page]
        L = kv_lens if isinstance(kv_lens, int) else kv_lens[b]
        first_dead = -(-L // page)
        table[b, first_dead:] = np.where(np.arange(nl - first_dead) % 2 == 0, -7, npool + 3)
    return kp, vp, torch.from_numpy(table)


def _oracle_row(q, k, v, spec, mod, b, h, L):
    D = k.shape[-1]
    Qf = np.zeros((L, D))
    Qf[L - 1] = q[b, h, 0].double().numpy()
    docs = spec.doc_ids[:, :L] if spec.doc_ids is not None else None
    return oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                               dataclasses.replace(spec, T=L, doc_ids=docs), mod, b, h, np.array([L - 1]),
                               with_mass=True)


def _case(B, H, cap, D, page, spec, mod, seed, kv_lens, heads=(0,), listed=False, dtype="bf16", ctx=""):
    from block_sparse_masked_build_amd import api
    log(f"[paged decode] {ctx}: B{B} H{H} cap {cap} D{D} page {page} {dtype} live {kv_lens} listed {listed}")
    rand = random_f16 if dtype == "f16" else random_bf16
    g = torch.Generator("cpu").manual_seed(seed)
    q = rand((B, H, 1, D), g)
    k = rand((B, H, cap, D), g)
    v = rand((B, H, cap, D), g)
    kp, vp, table = _page(k, v, page, kv_lens, spare=3, seed=seed + 1)
    s = api.from_spec_data(spec)
    m = None
    if mod is not None:
        m = api.score_mod(mod.alibi_slopes, mod.softcap,
                          bias=None if mod.bias_table is None else torch.from_numpy(mod.bias_table).cuda())
    bm = api.build_block_mask(s) if listed else None
    kvl = kv_lens if isinstance(kv_lens, int) else torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    qd = q.cuda()
    ref_o, ref_l = api.flex_attention_decode(qd, k.cuda(), v.cuda(), s, m, kv_len=kvl, block_mask=bm)
    out, lse = api.flex_attention_decode_paged(qd, kp.cuda(), vp.cuda(), table.cuda(), s, m, kv_len=kvl,
                                               block_mask=bm)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref_o.cpu()), f"{ctx}: paged out differs from the contiguous step"
    assert torch.equal(lse.cpu(), ref_l.cpu()), f"{ctx}: paged lse differs from the contiguous step"
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        L = kv_lens if isinstance(kv_lens, int) else kv_lens[b]
        for h in heads:
            ro, rl, rm = _oracle_row(q, k, v, spec, mod, b, h, L)
            assert_within_bound(f64(out[b, h]), ro, rm, f"{ctx} b{b} h{h} L{L}", fmt=dtype)
            assert_lse_close(lse[b, h:h + 1].double().numpy(), rl, f"{ctx} b{b} h{h} L{L}")
    log(f"  {ctx}: ok")


@pytest.mark.parametrize("page", [64, 128, 256, 1024])
def test_page_sizes_causal(page):
    """Page sizes from one 64-key block to a whole slot of 8 tiles; live
    lengths that end inside a page and on its edge."""
    _case(2, 3, 8192, 128, page, MaskSpecData(8192, causal=True), None, 70 + page // 64,
          [8192 - page // 2 - 1, 3 * page], heads=(0, 2), ctx=f"causal page {page}")


def test_documents_window_listed():
    """Packed documents + window with the block mask: listed tiles map to
    pages through the table."""
    cap, B, H = 16384, 2, 2
    rng = np.random.default_rng(71)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 700).astype(np.int32) for _ in range(B)])
    spec = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=1024)
    _case(B, H, cap, 64, 128, spec, ScoreModData(softcap=30.0), 72, [9000, 16384], heads=(1,), listed=True,
          ctx="docs+window listed")


def test_sinks_alibi_softcap_ragged_capacity():
    """Window + sinks, ALiBi + soft-cap, a capacity of 1,536 keys in pages of
    192 (a multiple of 64 that is not a power of two)."""
    H = 4
    spec = MaskSpecData(1536, causal=True, window=300, sinks=4)
    _case(3, H, 1536, 128, 192, spec, ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0), 73,
          [1536, 1, 700], heads=(0, 3), ctx="sinks+alibi page 192")


def test_bias_table_fp16():
    """A relative-position bias table in fp16."""
    H = 2
    spec = MaskSpecData(4096, causal=True)
    _case(2, H, 4096, 128, 256, spec, ScoreModData(bias_table=bias_table(H, 300, 74)), 75, [4000, 2049],
          heads=(0, 1), dtype="f16", ctx="bias fp16")


def test_head_dim_256():
    _case(1, 2, 2048, 256, 128, MaskSpecData(2048, causal=True), None, 76, 1999, heads=(0, 1), ctx="D256")


def test_single_page_pool_and_empty_live_length():
    """A pool of one page (every table entry clamps to it) and live length 0."""
    from block_sparse_masked_build_amd import api
    log("[paged decode] one-page pool, live lengths 64 and 0")
    g = torch.Generator("cpu").manual_seed(77)
    q = random_bf16((1, 2, 1, 64), g).cuda()
    kp = random_bf16((1, 2, 64, 64), g).cuda()
    vp = random_bf16((1, 2, 64, 64), g).cuda()
    table = torch.tensor([[0, 5, -2, 9]], dtype=torch.int32, device="cuda")
    spec = api.mask_spec(256, causal=True)
    out, lse = api.flex_attention_decode_paged(q, kp, vp, table, spec, kv_len=64)
    ref_o, ref_l = api.flex_attention_decode(q, kp, vp, api.mask_spec(64, causal=True), kv_len=64)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    out, lse = api.flex_attention_decode_paged(q, kp, vp, table, spec, kv_len=0)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_graph_replay_serving_loop():
    """A serving loop: the paged step captured once in a HIP graph; between
    replays new tokens are written into their pages, a page is taken from a
    free list whenever a sequence enters a new one (its table entry written
    in device memory), and the live lengths grow.  Every replay equals the
    eager contiguous step on the same keys bit for bit."""
    from block_sparse_masked_build_amd import api
    B, H, D, page, nl, npool = 2, 4, 128, 64, 16, 40
    cap = page * nl
    g = torch.Generator("cpu").manual_seed(78)
    q = random_bf16((B, H, 1, D), g).cuda()
    k_full = random_bf16((B, H, cap, D), g).cuda()
    v_full = random_bf16((B, H, cap, D), g).cuda()
    kp = torch.zeros((npool, H, page, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    table = torch.full((B, nl), -1, dtype=torch.int32, device="cuda")
    free = [int(x) for x in np.random.default_rng(78).permutation(npool)]
    kvl = torch.ones(B, dtype=torch.int32, device="cuda")
    spec = api.mask_spec(cap, causal=True, window=300, sinks=4)
    out = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = api.decode_workspace(B, H, cap, D)
    host_table = [[-1] * nl for _ in range(B)]
    filled = [0] * B

    def append(b, upto):
        # write keys filled[b] .. upto - 1 of sequence b into its pages
        while filled[b] < upto:
            pos = filled[b]
            j, r = divmod(pos, page)
            if host_table[b][j] < 0:
                host_table[b][j] = free.pop()
                table[b, j] = host_table[b][j]
            n = min(page - r, upto - pos)
            kp[host_table[b][j], :, r:r + n] = k_full[b, :, pos:pos + n]
            vp[host_table[b][j], :, r:r + n] = v_full[b, :, pos:pos + n]
            filled[b] += n

    def step():
        api.flex_attention_decode_paged(q, kp, vp, table, spec, None, kv_len=kvl, out=out, lse=lse, workspace=ws)

    for b in range(B):
        append(b, 1)
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
    for L0 in (1, 63, 64, 65, 300, 777, 1024):
        lens = [L0, max(1, L0 - 30)]
        log(f"[paged decode] graph replay at live lengths {lens}")
        for b in range(B):
            append(b, lens[b])
        kvl.copy_(torch.tensor(lens, dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref = api.flex_attention_decode(q, k_full, v_full, spec, None, kv_len=kvl.clone())
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), lens
    assert len(free) == npool - sum(-(-n // page) for n in filled)


@pytest.mark.parametrize("D,page,n_keys,dtype", [(64, 64, 1, "bf16"), (128, 192, 1000, "f16"), (128, 256, 4096, "bf16"),
                                                 (256, 128, 777, "bf16")])
def test_gather_pages_copies_exactly(D, page, n_keys, dtype):
    """The gather kernel's contiguous rows equal the keys and values they came
    from, bit for bit (ragged last block, table entries past n_keys out of
    range)."""
    from block_sparse_masked_build_amd import api
    B, H, cap = 3, 2, 4096 if page != 192 else 3840
    log(f"[gather] B{B} H{H} cap {cap} D{D} page {page} n_keys {n_keys} {dtype}")
    rand = random_f16 if dtype == "f16" else random_bf16
    g = torch.Generator("cpu").manual_seed(79 + D + page)
    k = rand((B, H, cap, D), g)
    v = rand((B, H, cap, D), g)
    kp, vp, table = _page(k, v, page, n_keys, spare=2, seed=80)
    kc, vc = api.gather_kv_pages(kp.cuda(), vp.cuda(), table.cuda(), n_keys)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), k[:, :, :n_keys]) and torch.equal(vc.cpu(), v[:, :, :n_keys])


@pytest.mark.parametrize("n,L", [(1, 1), (4, 777), (130, 3000)])
def test_multi_query_decode_over_pages(n, L):
    """A block of n new queries over a paged cache (gather, then the
    rectangular forward) equals the same block over the contiguous cache bit
    for bit, and the oracle on its first and last rows."""
    from block_sparse_masked_build_amd import api
    B, H, cap, D, page = 2, 2, 4096, 128, 128
    log(f"[paged multi-query decode] n {n} live {L}")
    rng = np.random.default_rng(81)
    docs = np.stack([np.cumsum(rng.random(cap) < 1 / 600).astype(np.int32) for _ in range(B)])
    spec_d = MaskSpecData(cap, causal=True, document=True, doc_ids=docs, window=700)
    mod_d = ScoreModData(alibi_slopes=alibi_slopes(H), softcap=30.0)
    g = torch.Generator("cpu").manual_seed(82 + n)
    q = random_bf16((B, H, n, D), g)
    k = random_bf16((B, H, cap, D), g)
    v = random_bf16((B, H, cap, D), g)
    kp, vp, table = _page(k, v, page, L, spare=3, seed=83)
    spec = api.from_spec_data(spec_d)
    m = api.score_mod(mod_d.alibi_slopes, mod_d.softcap)
    ref_o, ref_l = api.flex_attention_decode_multi(q.cuda(), k.cuda(), v.cuda(), spec, L, m)
    out, lse = api.flex_attention_decode_multi_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), spec, L, m)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref_o.cpu()) and torch.equal(lse.cpu(), ref_l.cpu())
    out, lse = out.cpu(), lse.cpu()
    live = dataclasses.replace(spec_d, T=L, doc_ids=docs[:, :L])  # queries at positions L - n .. L - 1
    sel = np.unique([0, n - 1])
    rows = L - n + sel
    for b in range(B):
        for h in range(H):
            Qf = np.zeros((L, D))
            Qf[rows] = q[b, h, sel].double().numpy()
            ro, rl, rm = oracle.forward_rows(Qf, k[b, h, :L].double().numpy(), v[b, h, :L].double().numpy(),
                                             live, mod_d, b, h, rows, with_mass=True)
            assert_within_bound(f64(out[b, h, sel]), ro, rm, f"b{b} h{h}")
            assert_lse_close(lse[b, h, sel].double().numpy(), rl, f"b{b} h{h}")
