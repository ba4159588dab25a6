"""The whole path captured once in a HIP graph and replayed across sliding
windows, the window-sweep workload's use.

* Captured: block-mask build, forward and backward on the current stream,
  every buffer preallocated.
* Between replays a new window is written to the device window scalar.
* The library makes no allocation, memset or host synchronisation, so the
  graph holds exactly its kernels.
* Every replay equals an eager run bit for bit (the kernels are
  deterministic), with eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

from parity_utils import log, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_graph_replays_match_eager_runs():
    from block_sparse_masked_build_amd import api
    B, H, T, D = 1, 2, 4096, 128
    rng = np.random.default_rng(11)
    docs = np.cumsum(rng.random(T) < 1 / 300).astype(np.int32)[None]
    spec = api.mask_spec(T, causal=True, doc_ids=docs, window=64)
    g = torch.Generator("cpu").manual_seed(5)
    q, k, v, do = (torch.randn((B, H, T, D), generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    bm = api.empty_block_mask(T, spec.mask_b)
    ws = api.block_mask_workspace(spec)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    wsb = api.bwd_workspace(B, H, T, D)

    def path():
        api.build_block_mask(spec, out=bm, workspace=ws)
        api.flex_attention_fwd(q, k, v, bm, spec, None, out=out, lse=lse)
        api.flex_attention_bwd(q, k, v, out, lse, do, bm, spec, None, dq=dq, dk=dk, dv=dv, workspace=wsb)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()  # warm-up off the default stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    names = [*bm._fields, "out", "lse", "dq", "dk", "dv"]
    for w in (64, 640, 1024, 1792, 300, 64):
        log(f"[graph] replay at window {w}")
        spec.set_window(w)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (*bm, out, lse, dq, dk, dv)]
        bm_e = api.build_block_mask(spec)  # eager run, fresh outputs
        out_e, lse_e = api.flex_attention_fwd(q, k, v, bm_e, spec, None)
        dq_e, dk_e, dv_e = api.flex_attention_bwd(q, k, v, out_e, lse_e, do, bm_e, spec, None)
        torch.cuda.synchronize()
        ref = [*bm_e, out_e, lse_e, dq_e, dk_e, dv_e]
        for name, a, b in zip(names, got, ref):
            assert torch.equal(a, b), f"window {w}: {name} differs between replay and eager run"
        assert int((bm_e.kv_num_blocks + bm_e.full_kv_num_blocks).sum()) > 0
