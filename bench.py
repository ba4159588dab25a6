#!/usr/bin/env python3
"""Benchmark of the block-sparse masked attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = one pass of the whole path over one batch already resident in HBM:
build the block mask, run the forward, and (when the workload has it, or by
default on the 64K packed-document workload) the backward.  Each kernel call
is bracketed by HIP events on the stream it is launched on; the reported
value is the forward throughput counted over visible tiles:

    TFLOP/s = sum_{b,h} visible_tiles(b) * 4 * 128 * 128 * D / t_fwd

(4*128*128*D = the two 128x128xD products of one tile; a partial tile counts
in full, as the speedrun notes state a tile with one visible score costs a
full tile).  Prints one JSON line.
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
                    help="1, 2, 2-causal, 2-window, 2-chunks, 3, 4a, 4b, 5, decode")
    ap.add_argument("--fwd-only", action="store_true", help="leave the backward out of the step")
    ap.add_argument("--slopes", action="store_true",
                    help="the backward also returns dL/dslope (workloads with ALiBi)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


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
    """Times the oracle (fp64, single thread) on whole query tiles, 256 per
    head spread over the sequence, head after head, until the time budget is
    used."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits

    counts = oracle.tile_counts(w.spec)
    vis_per_row = (counts > 0).sum(axis=2)  # [mask_b, QT]
    nt = w.T // TILE
    order = [int(x) for x in np.linspace(0, nt - 1, num=min(nt, 256)).round()]
    done, flops = 0, 0.0
    heads = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": (f"{done} query tiles (128 rows each) over {heads} head(s) of batch 0, "
                       f"{len(order)} per head spread over the sequence; fp64 numpy on one "
                       f"thread; {dt:.1f} s; visible-tile FLOPs counted as for the GPU")}


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
    ws = torch.empty(api.lib.bsm_decode_workspace_bytes(w.B, w.H, w.T, w.D), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        api.flex_attention_decode(q, k, v, spec, None, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        api.flex_attention_decode(q, k, v, spec, None, out=out, lse=lse, workspace=ws)
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)[len(evs) // 2]
    kv_bytes = 2 * w.B * w.H * w.T * w.D * 2
    gbs = kv_bytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "decode K/V GB/s (one query per batch and head, whole cache)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": decode_traffic(),
                     "kernel": "decode_partial_kernel<%d> + decode_combine_kernel" % w.D},
        "detail": {"decode_us_median": us, "kv_bytes": kv_bytes}}), flush=True)
    if args.copy_calibration_mib:  # one device copy of known size for the HBM counters
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    return 0


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
    if str(args.workload) == "decode":
        return decode_bench(args, w)
    backward = w.backward or (str(args.workload) == "2" and not args.fwd_only)
    if args.fwd_only:
        backward = False
    tensors = w.tensors(with_dout=backward)
    dev = {k: v.cuda() for k, v in tensors.items()}
    spec = api.from_spec_data(w.spec)
    mod = None
    if w.mod.alibi_slopes is not None or w.mod.softcap is not None:
        mod = api.score_mod(w.mod.alibi_slopes, w.mod.softcap)
    bm = api.empty_block_mask(w.T, spec.mask_b)
    ws = api.block_mask_workspace(spec)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
    dslopes = None
    if backward:
        dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
        bws = api.bwd_workspace(w.B, w.H, w.T, w.D)
        if args.slopes:
            if mod is None or mod.alibi_slopes is None:
                sys.exit("--slopes needs a workload with ALiBi (5)")
            dslopes = torch.empty(w.H, dtype=torch.float32, device="cuda")
    windows = w.windows or [None]

    def step(s):
        win = windows[s % len(windows)]
        if win is not None:
            spec.set_window(win)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        api.build_block_mask(spec, out=bm, workspace=ws)
        ev[1].record()
        api.flex_attention_fwd(dev["q"], dev["k"], dev["v"], bm, spec, mod, out=out, lse=lse)
        ev[2].record()
        if backward:
            api.flex_attention_bwd(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], bm, spec, mod,
                                   dq=dq, dk=dk, dv=dv, workspace=bws, dslopes=dslopes)
        ev[3].record()
        return ev, win

    # visible tiles per window (read once, outside the timed region)
    vis = {}
    for win in windows:
        if win is not None:
            spec.set_window(win)
        api.build_block_mask(spec, out=bm, workspace=ws)
        torch.cuda.synchronize()
        per_b = (bm.kv_num_blocks + bm.full_kv_num_blocks).sum(dim=(1, 2)).cpu().numpy()
        full = int(bm.full_kv_num_blocks.sum().item())
        part = int(bm.kv_num_blocks.sum().item())
        tiles_bh = sum(int(per_b[b if spec.mask_b > 1 else 0]) for b in range(w.B)) * w.H
        vis[win] = (tiles_bh, full, part)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [step(s) for s in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    mask_ms = np.array([r[0][0].elapsed_time(r[0][1]) for r in recs])
    fwd_ms = np.array([r[0][1].elapsed_time(r[0][2]) for r in recs])
    bwd_ms = np.array([r[0][2].elapsed_time(r[0][3]) for r in recs]) if backward else None
    fwd_flops = np.array([vis[r[1]][0] * 4 * TILE * TILE * w.D for r in recs], dtype=np.float64)
    fwd_tflops_total = fwd_flops.sum() / (fwd_ms.sum() * 1e-3) / 1e12
    achieved = fwd_tflops_total
    cfg = {
        "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
        "mask_b": spec.mask_b,
        "visible_tiles_per_head": vis[windows[0]][0] // w.H,
        "full_tiles": vis[windows[0]][1], "partial_tiles": vis[windows[0]][2],
        "tiles_per_side": w.T // TILE,
        "backward_in_step": backward,
        "documents": int(w.spec.doc_ids.max() + 1) if w.spec.doc_ids is not None else None,
    }
    if w.windows:
        cfg["windows"] = f"{w.windows[0]}..{w.windows[-1]} step {w.windows[1] - w.windows[0]}"
        cfg["per_window"] = {str(win): {"visible_tiles_per_head": vis[win][0] // w.H}
                             for win in w.windows}
    extra = {
        "mask_build_us_median": float(np.median(mask_ms) * 1e3),
        "fwd_us_median": float(np.median(fwd_ms) * 1e3),
        "fwd_us_mean": float(fwd_ms.mean() * 1e3),
        "pct_bf16_peak": 100.0 * achieved / PEAK_BF16_TFLOPS,
    }
    if backward:
        bwd_flops = fwd_flops * 2.5
        extra["bwd_us_median"] = float(np.median(bwd_ms) * 1e3)
        extra["bwd_tflops"] = float(bwd_flops.sum() / (bwd_ms.sum() * 1e-3) / 1e12)
        extra["bwd_slope_grad"] = dslopes is not None
    line = {
        "metric": METRIC,
        "value": round(float(achieved), 3),
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
            "achieved": round(float(achieved), 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(float(achieved / PEAK_BF16_TFLOPS), 4),
            "traffic": measured_traffic() if args.workload == "2" else None,
            "kernel": "fwd_kernel<%d,%s,%s>" % (w.D, str(w.mod.alibi_slopes is not None).lower(),
                                                str(w.mod.softcap is not None).lower()),
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
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, tensors, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
