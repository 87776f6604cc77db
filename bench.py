#!/usr/bin/env python3
"""Benchmark of the tile-overlapped GEMM-ReduceScatter on one MI355X.

One step = one entwine_gemm_rs call: the rank's whole share of the operation
(the GEMM producing every tile with its ready flag, and the concurrent
reduction of the rank's partition) on inputs already resident in HBM.

Default workload: the MLP down-projection slice, M = N = 4096, K_local =
1792, P = 8 simulated ranks, rank 0, bf16 inputs, fp32 accumulation, bf16
output, with the tuning table's choice of order, budget and block shape.

Reported (one JSON line on stdout):
  value        TFLOP/s of the overlapped step (2*M*N*K_local / latency)
  ms_per_step  mean step time over the timed steps
  latency_us_median   median per-step latency (the pages' protocol: 120
               warm-up and 200 timed iterations, median)
  sequential   the same kernels run back to back (budget 0) and the
               speedup of the overlapped schedule over it
  roofline     the GEMM kernel (the dominant kernel) against the bf16 MFMA
               dense peak, its duration timed with HIP events on the stream
               it runs on
  reducer      the reduction kernel alone (sequential schedule), GB/s of
               algorithmic bytes against HBM peak
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM+RS latency (µs) & TFLOP/s, % bf16 MFMA peak, reducer HBM GB/s"
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tile_overlapped_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(f"{kernel}/{workload}")
    if not e or e.get("sources") != kernel_sources_digest():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, X, W, peers, target_s: float):
    """Time the CPU oracle on the first S rows of the partition (S chosen so
    the run takes about target_s seconds), scaled to TFLOP/s."""
    from oracle import oracle as orc

    threads = orc.num_threads(0)
    t0 = time.perf_counter()
    orc.gemm_rs(X, W, peers, w.P, w.rank, row_begin=0, row_end=1, threads=threads)
    one = max(time.perf_counter() - t0, 1e-4)
    rows = int(max(1, min(w.rows, target_s / one)))
    t0 = time.perf_counter()
    orc.gemm_rs(X, W, peers, w.P, w.rank, row_begin=0, row_end=rows, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the rank's {w.rows}-row partition, all {w.N} columns, "
                      f"full K_local={w.K}, plus the {w.P - 1} peer adds; fp64 plain loops; "
                      f"{dt:.1f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=120)
    ap.add_argument("--workload", default="mlp")
    ap.add_argument("--order", default="auto", help="auto|row|partition|interleaved|col")
    ap.add_argument("--budget", type=int, default=-1)
    ap.add_argument("--block", default="", help="BMxBN, e.g. 128x256 (default: tuning table)")
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-seq", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the operation is built "
              "at one GPU's share of the work, with peer contributions as seeded buffers; "
              "no multi-GPU path exists.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tile_overlapped_gemm_amd as tog
    import workloads as wl

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    dev = torch.device("cuda:0")
    tog.load()
    tog.entwine_load_tuning(os.path.join(ROOT, "tile_overlapped_gemm_amd", "tuning.txt"))
    w = wl.BY_NAME[args.workload]
    log(f"workload {w.name}: M={w.M} N={w.N} K={w.K} P={w.P} rank={w.rank}; generating inputs")
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    Xd, Wd = up(X), up(W)
    pd = [None if p is None else up(p) for p in peers]
    out = torch.empty((w.rows, w.N), dtype=torch.float32 if w.fp32_io else torch.bfloat16,
                      device=dev)
    cfg_kw = dict(tile_m=w.tile, tile_n=w.tile, reducer_threads=args.threads)
    if w.fp32_io:
        cfg_kw.update(peer_dtype=tog.F32, out_dtype=tog.F32)
    if args.block:
        bm, bn = (int(v) for v in args.block.lower().split("x"))
        cfg_kw.update(block_m=bm, block_n=bn)
    cfg = tog.config(**cfg_kw)
    order = tog.ORDER_AUTO if args.order == "auto" else tog.ORDERS[args.order]
    stream = torch.cuda.current_stream(dev)

    def step(budget):
        tog.gemm_rs(Xd, Wd, pd, out, w.P, w.rank, order, budget, cfg=cfg, stream=stream)

    def timed(budget, steps, warmup):
        for _ in range(warmup):
            step(budget)
        torch.cuda.synchronize()
        st = tog.entwine_device_status(stream.cuda_stream)
        if st != tog.ENTWINE_OK:
            raise RuntimeError(f"device status {st} after warm-up")
        tog.entwine_timing_read()
        tog.entwine_timing(True)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(steps):
            step(budget)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        tog.entwine_timing(False)
        gemm_ms, red_ms, calls = tog.entwine_timing_read()
        st = tog.entwine_device_status(stream.cuda_stream)
        if st != tog.ENTWINE_OK:
            raise RuntimeError(f"device status {st} in the timed region")
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        total = evs[0].elapsed_time(evs[-1])
        return dict(ms_per_step=total / steps, median_ms=statistics.median(per),
                    p10_ms=sorted(per)[len(per) // 10], p90_ms=sorted(per)[(9 * len(per)) // 10],
                    gemm_ms=gemm_ms / calls, reduce_ms=red_ms / calls, wall_s=wall)

    budget = args.budget
    log(f"overlapped: {args.warmup} warm-up + {args.steps} timed steps")
    ov = timed(budget, args.steps, args.warmup)
    flops = float(w.flops)
    red_bytes = float(w.rows) * w.N * ((4 + 4 * (w.P - 1) + 4) if w.fp32_io
                                       else (4 + 2 * (w.P - 1) + 2))
    res = {
        "metric": METRIC,
        "value": flops / (ov["ms_per_step"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ov["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K_local": w.K, "P": w.P,
                   "rank": w.rank, "tile_order": args.order, "comm_budget": budget,
                   "block": args.block or "tuning table", "tile": w.tile,
                   "reducer_threads": args.threads or "tuning table",
                   "peer_ready": "preseeded"},
        "latency_us": ov["ms_per_step"] * 1e3,
        "latency_us_median": ov["median_ms"] * 1e3,
        "latency_us_p10_p90": [ov["p10_ms"] * 1e3, ov["p90_ms"] * 1e3],
        "pct_bf16_peak": 100.0 * flops / (ov["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "gemm_in_overlap_us": ov["gemm_ms"] * 1e3,
        "reduce_kernel_in_overlap_us": ov["reduce_ms"] * 1e3,
    }
    gemm_ms = ov["gemm_ms"]
    if not args.no_seq:
        log("sequential (budget 0): same steps")
        sq = timed(0, args.steps, args.warmup)
        res["sequential"] = {
            "latency_us": sq["ms_per_step"] * 1e3,
            "latency_us_median": sq["median_ms"] * 1e3,
            "gemm_us": sq["gemm_ms"] * 1e3,
            "reduce_us": sq["reduce_ms"] * 1e3,
        }
        res["speedup_vs_sequential"] = sq["ms_per_step"] / ov["ms_per_step"]
        res["overlap_efficiency"] = sq["gemm_ms"] / ov["ms_per_step"]
        res["reducer"] = {
            "bytes": red_bytes,
            "standalone_gbps": red_bytes / (sq["reduce_ms"] * 1e-3) / 1e9,
            "pct_hbm_peak": 100.0 * red_bytes / (sq["reduce_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "in_overlap_gbps_incl_waits": red_bytes / (ov["reduce_ms"] * 1e-3) / 1e9,
        }
        res["gemm_standalone_tflops"] = flops / (sq["gemm_ms"] * 1e-3) / 1e12
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    res["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                       "traffic": traffic_for(w.name, "gemm_publish"),
                       "kernel": "gemm_publish (in the overlapped step)",
                       "algorithmic_flops_per_launch": flops}
    if not args.no_cpu:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(w, X, W, peers, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
