#!/usr/bin/env python3
"""Benchmark of the block-sparse masked attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = one pass of the whole path over one batch already resident in HBM:
build the block mask, run the forward, and (when the workload has it, or by
default on the 64K packed-document workload) the backward.  Each call is
bracketed by HIP events on the stream it is launched on, and each is preceded
(outside its events) by a 512 MiB device write that evicts the L2 and the
256 MiB last-level cache, so every call starts cold.  The reported value is
the forward throughput counted over visible tiles at the median cold time:

    TFLOP/s = sum_{b,h} visible_tiles(b) * 4 * 128 * 128 * D / t_fwd

(4*128*128*D = the two 128x128xD products of one tile; a partial tile costs
as much as a full one -- speedrun notes, tile-summary paragraph).  The
minimum and a warm back-to-back median go to `detail`, with every other
workload of the suite timed the same way (`detail.configs`).  Prints one
JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd TFLOP/s over visible tiles (% bf16 MFMA peak), 64K doc+window mask"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
TILE = 128
FWD_KERNEL_SOURCES = ["block_sparse_masked_build_amd/csrc/attn_fwd.hip",
                      "block_sparse_masked_build_amd/csrc/attn_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_64k_doc_window_traffic.json")
DECODE_SOURCES = ["block_sparse_masked_build_amd/csrc/attn_decode.hip"]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b8h32_32k_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="2",
                    help="1, 2, 2-causal, 2-window, 2-chunks, 3, 4a, 4b, 5, decode, decode-docs")
    ap.add_argument("--fwd-only", action="store_true", help="leave the backward out of the step")
    ap.add_argument("--page-size", type=int, default=0,
                    help="decode workload: read K/V from a shuffled pool of pages of this many keys "
                         "through a block table (0: one contiguous cache)")
    ap.add_argument("--slopes", action="store_true",
                    help="the backward also returns dL/dslope (workloads with ALiBi)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="leave out the timing of the other workloads (detail.configs)")
    ap.add_argument("--config-reps", type=int, default=8, help="cold reps per other workload")
    ap.add_argument("--configs", default=",".join(CONFIG_KEYS),
                    help="comma-separated workloads timed for detail.configs")
    return ap.parse_args()


# Workloads of detail.configs ("-block64": 128 x 64 blocks; "-bias": with a
# relative-position bias table and its gradient; "-f16": fp16 tensors;
# "-d256": head dimension 256).
CONFIG_KEYS = ("1", "2", "2-block64", "2-bias", "2-f16", "2-d256", "2-causal", "2-window", "2-chunks", "3", "4a",
               "4b", "5", "5-block64")

FLUSH_BYTES = 512 << 20
_flush_buf = None


def flush_caches():
    """Writes 512 MiB on the current stream: larger than the 8 x 4 MiB of L2
    and the 256 MiB last-level cache, so the next call reads its inputs from
    HBM."""
    import torch
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    _flush_buf.fill_(1)


def timed(fn, flush=True):
    """(start, end) events around fn() on the current stream, after a cache
    flush outside them."""
    import torch
    if flush:
        flush_caches()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    return e0, e1


def us(evs):
    import numpy as np
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def fwd_source_hash() -> str:
    h = hashlib.sha256()
    for p in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_traffic():
    """HBM bytes per decoding step from the committed counter summary, or
    None when the decode kernels have changed since."""
    try:
        with open(DECODE_TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_source_hash") != source_hash(DECODE_SOURCES):
        return None
    return t.get("bytes_per_launch")


def measured_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, or None when the forward kernel has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("fwd_source_hash") != fwd_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, tensors, budget_s: float):
    """Times the oracle (fp64 numpy, mode R: the predicate over every pair of
    a row block, arithmetic on the columns some row of the block sees) on
    whole query tiles, 256 per head spread over the sequence, head after
    head, until the time budget is used; BLAS may use every core the process
    is allowed on.  The full-workload time is extrapolated from the sampled
    visible-tile FLOPs."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    host_cpus = os.cpu_count()
    allowed = len(os.sched_getaffinity(0))
    # the machine's CPU share is set through OMP_NUM_THREADS there
    threads = min(allowed, int(os.environ.get("OMP_NUM_THREADS", allowed) or allowed))
    counts = oracle.tile_counts(w.spec)
    vis_per_row = (counts > 0).sum(axis=2)  # [mask_b, QT]
    nt = w.T // TILE
    order = [int(x) for x in np.linspace(0, nt - 1, num=min(nt, 256)).round()]
    done, flops = 0, 0.0
    heads = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=threads):
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        for h in range(w.H):
            Q, K, V = (tensors[n][0, h].double().numpy() for n in ("q", "k", "v"))
            heads += 1
            for i in order:
                rows = np.arange(i * TILE, (i + 1) * TILE)
                oracle.forward_rows(Q, K, V, w.spec, w.mod, 0, h, rows)
                done += 1
                flops += float(vis_per_row[0, i]) * 4 * TILE * TILE * w.D
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    rate = flops / dt
    total = float(sum(int(vis_per_row[b if w.spec.mask_b > 1 else 0].sum()) for b in range(w.B))) * w.H \
        * 4 * TILE * TILE * w.D
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": blas_threads, "kind": "oracle",
            "host_cpu_count": host_cpus, "affinity_cpus": allowed, "blas_threads": blas_threads,
            "mode": "R", "extrapolated_full_forward_s": round(total / rate, 1),
            "sample": (f"{done} query tiles (128 rows each) over {heads} head(s) of batch 0, "
                       f"{len(order)} per head spread over the sequence; fp64 numpy, mode R, "
                       f"BLAS on up to {blas_threads} threads; {dt:.1f} s; visible-tile FLOPs "
                       f"counted as for the GPU")}


def decode_bench(args, w):
    """Decoding step: one query per (b, h) at the last cache position against
    the whole K/V cache; HBM-bound, so the roofline is bytes of K and V of the
    visible keys (every key under the causal mask) over the kernel time."""
    import torch
    from block_sparse_masked_build_amd import api
    t = w.tensors()
    q = t["q"][:, :, -1:].contiguous().cuda()
    k, v = t["k"].cuda(), t["v"].cuda()
    spec = api.from_spec_data(w.spec)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = api.decode_workspace(w.B, w.H, w.T, w.D)
    kvl = torch.tensor([w.T], dtype=torch.int32, device="cuda")  # live length: the whole cache
    import numpy as np
    page = args.page_size
    # with documents the step reads the tiles its block-mask row lists: K and
    # V of those tiles are the algorithmic bytes (every tile is below the
    # live length, the whole cache)
    bm = api.build_block_mask(spec) if w.spec.document else None
    if bm is not None:
        nt, row = w.T // 128, (w.T - 1) // 128
        tiles = (bm.kv_num_blocks + bm.full_kv_num_blocks).view(-1, nt)[:, row].cpu().numpy()
        tiles = np.broadcast_to(tiles, (w.B,)) if tiles.size == 1 else tiles
        kv_bytes = int(tiles.sum()) * w.H * 128 * w.D * 2 * 2
    else:
        kv_bytes = 2 * w.B * w.H * w.T * w.D * 2

    if page:
        # the same cache as pages of `page` keys in a shuffled pool, one
        # block-table row per batch element
        if page % 64 or w.T % page:
            sys.exit(f"--page-size {page} must be a multiple of 64 that divides {w.T}")
        nl = w.T // page
        gen = torch.Generator("cpu").manual_seed(w.seed)
        table = torch.randperm(w.B * nl, generator=gen).to(torch.int32).view(w.B, nl).cuda()

        def to_pages(x):
            blocks = x.view(w.B, w.H, nl, page, w.D).permute(0, 2, 1, 3, 4).reshape(w.B * nl, w.H, page, w.D)
            pool = torch.empty_like(blocks)
            pool[table.flatten().long()] = blocks
            return pool

        kp, vp = to_pages(k), to_pages(v)
        del k, v

        def call():
            api.flex_attention_decode_paged(q, kp, vp, table, spec, None, kv_len=kvl, block_mask=bm, out=out,
                                            lse=lse, workspace=ws)
    else:
        def call():
            api.flex_attention_decode(q, k, v, spec, None, kv_len=kvl, block_mask=bm, out=out, lse=lse,
                                      workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    evs = [timed(call) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm = [timed(call, flush=False) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_us = float(np.median(us(evs)))
    gbs = kv_bytes / (t_us * 1e-6) / 1e9
    what = "the tiles of the query's document" if bm is not None else "whole cache"
    print(json.dumps({
        "metric": f"decode K/V GB/s (one query per batch and head, {what})", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D, "page_size": page or None},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if page or bm is not None else decode_traffic(),
                     "kernel": "decode_partial_kernel<%d> + decode_combine_kernel" % w.D},
        "detail": {"decode_us_median_cold": t_us, "decode_us_min_cold": float(us(evs).min()),
                   "decode_us_median_warm": float(np.median(us(warm))), "kv_bytes": kv_bytes,
                   "timing": "HIP events per call, 512 MiB device write before each (outside the events)"}}),
          flush=True)
    if args.copy_calibration_mib:  # one device copy of known size for the HBM counters
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    return 0


def tiles_per_bh(api, spec, bm, ws, w, win=None):
    """Visible tiles summed over (b, h), full and partial tiles of the mask
    (read once, outside any timed region)."""
    import torch
    if win is not None:
        spec.set_window(win)
    api.build_block_mask(spec, out=bm, workspace=ws)
    torch.cuda.synchronize()
    per_b = (bm.kv_num_blocks + bm.full_kv_num_blocks).sum(dim=(1, 2)).cpu().numpy()
    full = int(bm.full_kv_num_blocks.sum().item())
    part = int(bm.kv_num_blocks.sum().item())
    return sum(int(per_b[b if spec.mask_b > 1 else 0]) for b in range(w.B)) * w.H, full, part


class Path:
    """Device buffers of one workload and its three calls."""

    def __init__(self, api, w, backward, slopes=False):
        import torch
        self.api, self.w, self.backward = api, w, backward
        t = w.tensors(with_dout=backward)
        self.dev = {k: v.cuda() for k, v in t.items()}
        self.host = t
        self.spec = api.from_spec_data(w.spec)
        self.mod = None
        bias = getattr(w.mod, "bias_table", None)
        if w.mod.alibi_slopes is not None or w.mod.softcap is not None or bias is not None:
            self.mod = api.score_mod(w.mod.alibi_slopes, w.mod.softcap, bias=bias)
        self.bm = api.empty_block_mask(self.spec)
        self.ws = api.block_mask_workspace(self.spec)
        self.out = torch.empty_like(self.dev["q"])
        self.lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
        self.dslopes = self.dbias = None
        if backward:
            self.grads = [torch.empty_like(self.dev["q"]) for _ in range(3)]
            self.bws = api.bwd_workspace(w.B, w.H, w.T, w.D, mod=self.mod)
            if bias is not None:
                self.dbias = torch.empty(self.mod.bias.shape, dtype=torch.float32, device="cuda")
            if slopes:
                self.dslopes = torch.empty(w.H, dtype=torch.float32, device="cuda")

    def build(self):
        self.api.build_block_mask(self.spec, out=self.bm, workspace=self.ws)

    def fwd(self):
        d = self.dev
        self.api.flex_attention_fwd(d["q"], d["k"], d["v"], self.bm, self.spec, self.mod, out=self.out,
                                    lse=self.lse)

    def bwd(self):
        d = self.dev
        dq, dk, dv = self.grads
        self.api.flex_attention_bwd(d["q"], d["k"], d["v"], self.out, self.lse, d["dout"], self.bm, self.spec,
                                    self.mod, dq=dq, dk=dk, dv=dv, workspace=self.bws, dslopes=self.dslopes,
                                    dbias=self.dbias)


def config_detail(api, key, reps):
    """Cold timings of one other workload: mask build, forward and (with a
    backward) backward medians, and the throughput over visible tiles.  A
    key ending in "-block64" is that workload with 128 x 64 blocks: its
    throughput counts the listed 64-key blocks (4 * 128 * 64 * D flops
    each), the work the kernels do there.  A key ending in "-bias" adds a
    relative-position bias table of radius 1024 (N(0, 0.25) entries) and
    runs the backward with its gradient; "-f16" runs the workload on fp16
    tensors, forward and backward; "-d256" at head dimension 256."""
    import dataclasses
    import numpy as np
    import torch
    from workloads import bias_table, make_config
    with_bias = key.endswith("-bias")
    if with_bias:
        key = key[:-len("-bias")]
    f16 = key.endswith("-f16")
    if f16:
        key = key[:-len("-f16")]
    d256 = key.endswith("-d256")
    if d256:
        key = key[:-len("-d256")]
    base, _, variant = key.partition("-block")
    w = make_config(base if variant else key)
    if f16:
        w = dataclasses.replace(w, name=w.name + ", fp16", backward=True, dtype="f16")
    if d256:
        w = dataclasses.replace(w, name=w.name.replace("D128", "D256"), D=256, backward=True)
    if with_bias:
        w = dataclasses.replace(w, name=w.name + ", bias table R 1024", backward=True,
                                mod=dataclasses.replace(w.mod, bias_table=bias_table(w.H, 1024, seed=2, sd=0.5)))
    kb = TILE
    if variant:
        kb = int(variant)
        w = dataclasses.replace(w, name=w.name + f", 128 x {kb} blocks", spec=dataclasses.replace(w.spec, kv_block=kb))
    path = Path(api, w, w.backward)
    windows = w.windows or [None]
    res = {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D, "mask_b": path.spec.mask_b}
    per_win = {}
    for win in windows:
        vis, full, part = tiles_per_bh(api, path.spec, path.bm, path.ws, w, win)
        for _ in range(3):  # warm-up: a lighter workload just ran, let the clocks settle
            path.fwd()
            if w.backward:
                path.bwd()
        ev = {"mask": [], "fwd": [], "bwd": []}
        for _ in range(reps):
            ev["mask"].append(timed(path.build))
            ev["fwd"].append(timed(path.fwd))
            if w.backward:
                ev["bwd"].append(timed(path.bwd))
        torch.cuda.synchronize()
        fl = vis * 4 * TILE * kb * w.D
        r = {"visible_tiles_per_head": vis // w.H, "full_tiles": full, "partial_tiles": part,
             "mask_build_us": round(float(np.median(us(ev["mask"]))), 1),
             "fwd_us": round(float(np.median(us(ev["fwd"]))), 1)}
        r["fwd_tflops"] = round(fl / (r["fwd_us"] * 1e-6) / 1e12, 1)
        r["fwd_pct_bf16_peak"] = round(100 * r["fwd_tflops"] / PEAK_BF16_TFLOPS, 1)
        if w.backward:
            r["bwd_us"] = round(float(np.median(us(ev["bwd"]))), 1)
            r["bwd_tflops"] = round(2.5 * fl / (r["bwd_us"] * 1e-6) / 1e12, 1)
            r["bwd_pct_bf16_peak"] = round(100 * r["bwd_tflops"] / PEAK_BF16_TFLOPS, 1)
        per_win[win] = r
    if w.windows:
        res["per_window"] = {str(k): v for k, v in per_win.items()}
        fwd_tot = sum(v["fwd_us"] for v in per_win.values())
        fl_tot = sum(v["visible_tiles_per_head"] * w.H * 4 * TILE * TILE * w.D for v in per_win.values())
        res["sweep_fwd_us_total"] = round(fwd_tot, 1)
        res["sweep_mask_build_us_total"] = round(sum(v["mask_build_us"] for v in per_win.values()), 1)
        res["sweep_fwd_tflops"] = round(fl_tot / (fwd_tot * 1e-6) / 1e12, 1)
        res["sweep_fwd_pct_bf16_peak"] = round(100 * res["sweep_fwd_tflops"] / PEAK_BF16_TFLOPS, 1)
    else:
        res.update(per_win[None])
    del path
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU sharding "
              "(every batch/head/query-tile unit is independent; see the sharding note "
              "in the design document). Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from block_sparse_masked_build_amd import api
    from workloads import make_config

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    w = make_config(args.workload)
    if str(args.workload) in ("decode", "decode-docs"):
        return decode_bench(args, w)
    backward = w.backward or (str(args.workload) == "2" and not args.fwd_only)
    if args.fwd_only:
        backward = False
    if args.slopes and (w.mod.alibi_slopes is None):
        sys.exit("--slopes needs a workload with ALiBi (5)")
    path = Path(api, w, backward, args.slopes)
    windows = w.windows or [None]
    vis = {win: tiles_per_bh(api, path.spec, path.bm, path.ws, w, win) for win in windows}

    def step(s, flush=True):
        win = windows[s % len(windows)]
        if win is not None:
            path.spec.set_window(win)
        ev = [timed(path.build, flush), timed(path.fwd, flush)]
        if backward:
            ev.append(timed(path.bwd, flush))
        return ev, win

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [step(s) for s in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # warm reference: the same forward calls back to back, no flush
    warm = []
    for s in range(args.steps):
        win = windows[s % len(windows)]
        if win is not None:
            path.spec.set_window(win)
            path.build()
        warm.append((timed(path.fwd, flush=False), win))
    torch.cuda.synchronize()

    mask_us = us([r[0][0] for r in recs])
    fwd_us = us([r[0][1] for r in recs])
    bwd_us = us([r[0][2] for r in recs]) if backward else None
    warm_us = us([r[0] for r in warm])
    fl = np.array([vis[r[1]][0] * 4 * TILE * TILE * w.D for r in recs], dtype=np.float64)
    tflops = fl / (fwd_us * 1e-6) / 1e12          # per cold call
    warm_tflops = np.array([vis[r[1]][0] * 4 * TILE * TILE * w.D for r in warm]) / (warm_us * 1e-6) / 1e12
    achieved = float(np.median(tflops))           # the median cold call
    cfg = {
        "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
        "mask_b": path.spec.mask_b,
        "visible_tiles_per_head": vis[windows[0]][0] // w.H,
        "full_tiles": vis[windows[0]][1], "partial_tiles": vis[windows[0]][2],
        "tiles_per_side": w.T // TILE,
        "backward_in_step": backward,
        "documents": int(w.spec.doc_ids.max() + 1) if w.spec.doc_ids is not None else None,
    }
    if w.windows:
        cfg["windows"] = f"{w.windows[0]}..{w.windows[-1]} step {w.windows[1] - w.windows[0]}"
    extra = {
        "timing": "HIP events per call; 512 MiB device write before each call (outside the events); "
                  "value = median cold call",
        "mask_build_us_median": float(np.median(mask_us)),
        "fwd_us_median_cold": float(np.median(fwd_us)),
        "fwd_us_min_cold": float(fwd_us.min()),
        "fwd_us_median_warm": float(np.median(warm_us)),
        "fwd_tflops_median_cold": achieved,
        "fwd_tflops_best_cold": float(tflops.max()),
        "fwd_tflops_median_warm": float(np.median(warm_tflops)),
        "pct_bf16_peak": 100.0 * achieved / PEAK_BF16_TFLOPS,
        "ms_per_step_includes": "three 512 MiB cache flushes per step",
    }
    if backward:
        extra["bwd_us_median_cold"] = float(np.median(bwd_us))
        extra["bwd_tflops_median_cold"] = float(np.median(2.5 * fl / (bwd_us * 1e-6) / 1e12))
        extra["bwd_pct_bf16_peak"] = 100.0 * extra["bwd_tflops_median_cold"] / PEAK_BF16_TFLOPS
        extra["bwd_slope_grad"] = path.dslopes is not None
    line = {
        "metric": METRIC,
        "value": round(achieved, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic() if args.workload == "2" else None,
            "kernel": "fwd_kernel<%d,%s,%s,false,%s>" % (
                w.D, str(w.mod.alibi_slopes is not None).lower(), str(w.mod.softcap is not None).lower(),
                str(w.T % TILE != 0).lower()),
        },
        "detail": extra,
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["detail"]["copy_calibration_bytes"] = n
    host = path.host
    del path
    torch.cuda.empty_cache()
    if not args.no_configs:
        confs = {}
        for key in [k for k in args.configs.split(",") if k]:
            if key not in CONFIG_KEYS:
                sys.exit(f"unknown config {key!r}: one of {', '.join(CONFIG_KEYS)}")
            print(f"[bench] timing workload {key}", file=sys.stderr, flush=True)
            confs[key] = config_detail(api, key, args.config_reps)
        line["detail"]["configs"] = confs
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
