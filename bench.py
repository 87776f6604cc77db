#!/usr/bin/env python3
"""Benchmark of the tile-overlapped GEMM-ReduceScatter on one MI355X.

A step is one entwine_gemm_rs call: the rank's whole share of the operation
(the GEMM producing every output tile, and the reduction of the rank's
partition with the peers' contributions) on inputs already resident in HBM.
Steps are replayed from a captured HIP graph, as the pages' prototype does with
CUDA Graphs, so the timed loop measures device time rather than host launch
overhead.

Default workload: the large MLP slice, M = N = 8192, K_local = 3584, P = 8
simulated ranks, rank 0, bf16 inputs, fp32 accumulation, bf16 output, in the
configuration the offline tuning table picks for the shape (block shape,
order, budget -- 0 when no overlapped schedule beat the sequential one --,
schedule).  Timing follows the pages' protocol (Sec. 5.1): warm-up
iterations, then timed iterations each bracketed by HIP events, the median
reported.

One JSON line on stdout:
  value, ms_per_step   TFLOP/s (2*M*N*K_local / step time) and the median
                       per-replay step time of the tuned step
  sequential           the non-overlapped schedule (GEMM, then reduction)
  overlapped           both overlapped schedules (two streams, fused)
  ablations            Sec. 5.3.1 production order, Sec. 5.3.2 release
                       granularity and the communication budget's response
                       (Sec. 2.2, 5.4.2): end-to-end median and the device
                       trace's GEMM end and communication tail
  symmetric_all_ranks  the tuned step for every rank under symmetric peer
                       readiness; the slowest rank bounds a P-GPU step
  roofline             the step's dominant kernel against the bf16 MFMA
                       dense peak; its duration comes from HIP events
                       recorded on the stream the kernel runs on
  reducer              the reduction kernel alone against HBM peak, warm and
                       with the caches scrubbed, and the Eq. (4) comparison
  cpu_baseline         the CPU oracle on a bounded row sample of the workload
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


# The source files each measured kernel is built from: its counters stay valid
# while these are unchanged.
KERNEL_SOURCES = {
    "gemm_publish": ["kernels.h", "gemm_block.h", "gemm_publish.hip"],
    "gemm_rs_fused": ["kernels.h", "gemm_block.h", "reduce_task.h", "gemm_rs_fused.hip"],
    "flat_reduce": ["kernels.h", "reduce_task.h", "tile_reduce.hip"],
    "rmsnorm_rows": ["kernels.h", "rmsnorm.hip"],
}


def kernel_sources_digest(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tile_overlapped_gemm_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel's current sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(f"{kernel}/{workload}")
    if not e or e.get("sources") != kernel_sources_digest(kernel):
        return None
    return e.get("bytes_per_launch")


def tuned_entry(w):
    """The tuning table's entry for the workload's shape as a dict, or None."""
    names = ["order", "budget", "bm", "bn", "threads", "slabs", "schedule", "variant"]
    with open(os.path.join(ROOT, "tile_overlapped_gemm_amd", "tuning.txt")) as f:
        for line in f:
            v = line.split()
            if not v or v[0].startswith("#"):
                continue
            if [int(x) for x in v[:4]] == [w.M, w.N, w.K, w.P]:
                vals = [int(x) for x in v[4:]] + [1, 0, 0][len(v) - 9:]
                return dict(zip(names, vals))
    return None


def cpu_baseline(w, X, W, target_s: float):
    """The CPU oracle's fp64 partial GEMM on the first S rows of the M-row
    product (S sized so that three runs take about target_s seconds), median
    of the three, as TFLOP/s."""
    from oracle import oracle as orc

    threads = orc.num_threads(0)
    probe = max(1, min(w.M, 32))
    t0 = time.perf_counter()
    orc.partial_gemm(X, W, row_begin=0, row_end=probe, threads=threads)
    per_row = max((time.perf_counter() - t0) / probe, 1e-6)
    rows = int(max(1, min(w.M, target_s / 3.0 / per_row)))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        orc.partial_gemm(X, W, row_begin=0, row_end=rows, threads=threads)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {w.M}-row partial product X*W (N={w.N}, "
                      f"K_local={w.K}) in fp64 plain loops on {threads} threads, median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in times)} s); the reduction's adds are "
                      f"negligible next to it"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=120)
    ap.add_argument("--workload", default="large_mlp")
    ap.add_argument("--order", default="auto", help="auto|row|partition|interleaved|col")
    ap.add_argument("--budget", type=int, default=-1, help="comm budget x (-1: tuning table)")
    ap.add_argument("--block", default="", help="BMxBN, e.g. 256x256 (default: tuning table)")
    ap.add_argument("--threads", type=int, default=0, help="reduction threads (0: tuning table)")
    ap.add_argument("--slabs", type=int, default=0, help="row slabs per task (0: tuning table)")
    ap.add_argument("--gemm-variant", type=int, default=0,
                    help="GEMM pipeline (0: the tuning table's for its block shape, else 5 = "
                         "base, 4 = ping-pong, ...)")
    ap.add_argument("--peers", default="preseeded", help="preseeded|symmetric")
    ap.add_argument("--w-layout", default="kn", choices=["kn", "nk"],
                    help="W handed over [K_local][N] (the library's default) or [N][K_local]")
    ap.add_argument("--schedule", default="auto", choices=["auto", "streams", "fused", "assisted"],
                    help="overlapped schedule: two streams, one fused kernel, the fused kernel "
                         "with helper workgroups on a second stream, or the tuning table's")
    ap.add_argument("--static-cus", type=int, default=32,
                    help="CUs reserved for the reduction in the CU-policy leg (Sec. 5.3.3)")
    ap.add_argument("--reducer-cus", type=int, default=0,
                    help="with --profile: reserve this many CUs for the reduction (two streams; "
                         "--budget must match)")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ablations", action="store_true",
                    help="skip the order / release-granularity / budget sweeps")
    ap.add_argument("--profile", action="store_true",
                    help="only run --warmup + --steps eager calls (for rocprofv3), print nothing")
    ap.add_argument("--chain", action="store_true",
                    help="with --profile: the calls run the layer chain (residual + RMSNorm)")
    ap.add_argument("--scrub", type=int, default=0, metavar="MIB",
                    help="with --profile: fill a MIB-sized buffer before each call, so that the "
                         "call starts from cold caches (L2 and the 256 MB MALL)")
    ap.add_argument("--scrub-mode", default="fill", choices=["fill", "read"],
                    help="with --scrub: write the buffer (a fill) or only read it (a sum), so "
                         "that the evicted lines are dirty or clean")
    ap.add_argument("--stage", default="all", choices=["all", "gemm", "reduce", "copy", "library"],
                    help="with --profile: run one kernel of the step alone (the reduction alone "
                         "with --budget x runs x workgroups without waits), or, for scale, the "
                         "runtime's device copy moving the reduction's bytes (half read, half "
                         "written), or a library GEMM of the same shape (torch.matmul, X [M][K] "
                         "times W [K][N])")
    ap.add_argument("--lib", default="", metavar="PATH",
                    help="load the HIP library from PATH instead of the in-tree build (to "
                         "compare build options, e.g. one built by "
                         "tile_overlapped_gemm_amd._build.build(out=PATH, "
                         "extra=['-DENTWINE_MFMA_EDGE=32']))")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer --steps times (the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the operation is built "
              "at one GPU's share of the work, with the peers' contributions as seeded device "
              "buffers; there is no multi-GPU path to launch.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tile_overlapped_gemm_amd as tog
    import workloads as wl

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB x {args.steps}")
        return 0
    if args.lib:
        tog.load(os.path.abspath(args.lib))
    else:
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

    wkn = args.w_layout == "kn"
    W_kn = wl.w_as_kn(W)
    Xd, Wd = up(X), up(W_kn if wkn else W)
    pd = [None if p is None else up(p) for p in peers]
    out = torch.empty((w.rows, w.N), dtype=torch.float32 if w.fp32_io else torch.bfloat16,
                      device=dev)
    # The step's configuration, every field explicit: flags first, then the
    # tuning table's entry for the shape, then the library's defaults.
    tuned = tuned_entry(w) or {}
    _, _, q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    cus = tog.entwine_device_cus()
    if args.block:
        bm, bn = (int(v) for v in args.block.lower().split("x"))
    else:
        bm, bn = tuned.get("bm", 256), tuned.get("bn", 256)
    order = (tog.ORDERS[args.order] if args.order != "auto"
             else tuned.get("order", tog.ORDER_INTERLEAVED))
    budget = args.budget if args.budget >= 0 else tuned.get("budget", 32)
    threads = args.threads or tuned.get("threads", 256)
    slabs = args.slabs or tuned.get("slabs", 1)
    schedule = ({"streams": tog.SCHEDULE_STREAMS, "fused": tog.SCHEDULE_FUSED,
                 "assisted": tog.SCHEDULE_ASSISTED}[args.schedule]
                if args.schedule != "auto" else (tuned.get("schedule") or tog.SCHEDULE_STREAMS))
    # The overlapped schedules are also timed when the tuned step is sequential:
    # then at the largest budget below the CU count with four row slabs per
    # tile, where the fused schedule measured best (every CU reduces a share).
    ov_budget = budget if budget > 0 else min(q * 4, cus - 1)
    ov_slabs = slabs if budget > 0 else (4 if w.tile % 4 == 0 else 1)
    kind = "sequential" if budget == 0 else ("fused" if schedule == tog.SCHEDULE_FUSED
                                             else "streams")
    # The pipeline the step's GEMM runs (tuning-table numbering, 0 = base).
    if args.gemm_variant:
        pipeline = 0 if args.gemm_variant == tog.GEMM_BASE else args.gemm_variant
    else:
        pipeline = tuned.get("variant", 0) if (tuned.get("bm"), tuned.get("bn")) == (bm, bn) else 0
        if wkn:
            pipeline = 0  # the base pipeline is the one built for W [K][N]
    cfg_kw = dict(w_layout=tog.W_KN if wkn else tog.W_NK,
                  tile_m=w.tile, tile_n=w.tile, block_m=bm, block_n=bn, reducer_threads=threads,
                  task_slabs=slabs, schedule=schedule, gemm_variant=args.gemm_variant,
                  peer_ready=tog.PEERS_SYMMETRIC if args.peers == "symmetric" else tog.PEERS_PRESEEDED)
    if w.fp32_io:
        cfg_kw.update(peer_dtype=tog.F32, out_dtype=tog.F32)
    cfg = tog.config(**cfg_kw)
    cfg_gemm = tog.config(**cfg_kw, stages=tog.STAGES_GEMM)
    cfg_red = tog.config(**cfg_kw, stages=tog.STAGES_REDUCE)
    cfg_streams = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_STREAMS, task_slabs=ov_slabs))
    cfg_fused = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_FUSED, task_slabs=ov_slabs))
    # CU policy (Sec. 5.3.3): n reduction workgroups in the shared pool against
    # the same n on n CUs reserved for them.
    n_static = max(1, min(args.static_cus, cus - 8))
    # Each policy with its own reduction workgroup size: the shared pool's must
    # fit beside a GEMM block; a reserved CU takes the library's choice (512).
    cfg_static = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_STREAMS, task_slabs=ov_slabs,
                                   reducer_cus=n_static, reducer_threads=0))
    stream = torch.cuda.Stream(dev)

    def call(b, c=cfg, rank=w.rank, peers=pd):
        tog.gemm_rs(Xd, Wd, peers, out, w.P, rank, order, b, cfg=c, stream=stream)

    def check_status(where):
        st = tog.entwine_device_status(stream.cuda_stream)
        if st != tog.ENTWINE_OK:
            raise RuntimeError(f"device status {st} {where}")

    # The layer chain's inputs (residual stream rows and norm weight).
    res_h, gamma_h = wl.chain_inputs(w)
    res_d, gamma_d = up(res_h), up(gamma_h)
    h_buf, y_buf = torch.empty_like(out), torch.empty_like(out)

    def chain(b):
        tog.gemm_rs_rmsnorm(Xd, Wd, pd, res_d, gamma_d, 1e-5, h_buf, y_buf, w.P, w.rank, order, b,
                            cfg=cfg, stream=stream)

    def settle_clocks(seconds=1.0):
        """About a second of a library bf16 GEMM (kernels of other names in a
        trace), so that the GPU's clocks have ramped before what is measured."""
        a = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(4):
                torch.matmul(a, a)
            torch.cuda.synchronize()

    if args.profile:
        settle_clocks()
        pc = (tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_STREAMS,
                                reducer_cus=args.reducer_cus,
                                reducer_threads=args.threads)) if args.reducer_cus else cfg)
        if args.stage in ("gemm", "reduce"):
            pc = tog.config(**dict(cfg_kw, stages=tog.STAGES_GEMM if args.stage == "gemm"
                                   else tog.STAGES_REDUCE))
        scrub_buf = (torch.empty(args.scrub << 20, dtype=torch.uint8, device=dev).fill_(1)
                     if args.scrub else None)
        scrub_sum = torch.zeros((), dtype=torch.float32, device=dev)
        if args.stage == "copy":
            n_red = w.rows * w.N * ((4 + 4 * (w.P - 1) + 4) if w.fp32_io
                                    else (4 + 2 * (w.P - 1) + 2))
            cp_src = torch.ones(n_red // 2, dtype=torch.uint8, device=dev)
            cp_dst = torch.empty_like(cp_src)
        if args.stage == "library":
            W_lib = Wd if wkn else Wd.t().contiguous()
            lib_out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup + args.steps):
            if scrub_buf is not None:
                with torch.cuda.stream(stream):
                    if args.scrub_mode == "fill":
                        scrub_buf.fill_(1)
                    else:
                        torch.sum(scrub_buf.view(torch.float32), 0, out=scrub_sum)
            if args.stage == "copy":
                with torch.cuda.stream(stream):
                    cp_dst.copy_(cp_src)
            elif args.stage == "library":
                with torch.cuda.stream(stream):
                    torch.matmul(Xd, W_lib, out=lib_out)
            else:
                chain(budget) if args.chain else call(budget, pc)
        stream.synchronize()
        check_status("in the profiled calls")
        log(f"profiled {args.warmup + args.steps} calls: {kind}, block {bm}x{bn}, order {order}, "
            f"budget {budget}, stage {args.stage}")
        return 0

    def graph_of(body):
        with torch.cuda.stream(stream):
            body()  # workspace and schedule exist before the capture
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            body()
        return g

    def timed_graph(body, steps, warmup, per_step=True):
        """Graph replays of `body` after `warmup` untimed ones.  per_step: the
        pages' protocol (Sec. 5.1), `steps` replays each bracketed by HIP
        events, the median (ms_per_step) and the 10th / 90th percentiles;
        then, as a second figure, the mean over `steps` back-to-back replays
        between two events (an event between replays serializes them, which
        the back-to-back figure leaves out).  Without per_step only the
        back-to-back mean (kernel timings of many launches per replay)."""
        g = graph_of(body)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                g.replay()
        stream.synchronize()
        check_status("after warm-up")
        res = {}
        if per_step:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                evs[0].record(stream)
                for i in range(steps):
                    g.replay()
                    evs[i + 1].record(stream)
            torch.cuda.synchronize()
            check_status("in the per-replay pass")
            per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
            res.update(ms_per_step=statistics.median(per), p10_ms=per[len(per) // 10],
                       p90_ms=per[(9 * len(per)) // 10])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(steps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        check_status("in the timed region")
        res["back_to_back_ms"] = e0.elapsed_time(e1) / steps
        if not per_step:
            res["ms_per_step"] = res["back_to_back_ms"]
        return res

    def timed_eager(body, steps, warmup):
        """The same per-step protocol as timed_graph, with the calls issued
        eagerly (the library's own launches, no graph): the median of `steps`
        calls each bracketed by HIP events, and the back-to-back mean."""
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                body()
        stream.synchronize()
        check_status("after the eager warm-up")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        with torch.cuda.stream(stream):
            evs[0].record(stream)
            for i in range(steps):
                body()
                evs[i + 1].record(stream)
        stream.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(steps):
                body()
            e1.record(stream)
        stream.synchronize()
        check_status("in the eager timed region")
        return {"ms_per_step": statistics.median(per), "p10_ms": per[len(per) // 10],
                "p90_ms": per[(9 * len(per)) // 10], "back_to_back_ms": e0.elapsed_time(e1) / steps}

    def lat(r):
        return {"latency_us": r["ms_per_step"] * 1e3,
                "latency_us_back_to_back": r["back_to_back_ms"] * 1e3}

    # The GPU's clocks ramp over the first fraction of a second of work: about
    # one second of untimed replays of the step settles them before any of
    # the timed legs (each still runs its own W warm-up replays).
    settle = graph_of(lambda: call(budget))
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        with torch.cuda.stream(stream):
            for _ in range(20):
                settle.replay()
        stream.synchronize()
    check_status("while the clocks settle")
    del settle
    log(f"step ({kind}, block {bm}x{bn}, order {order}, budget {budget}): {args.warmup} warm-up "
        f"+ {args.steps} timed graph replays")
    st = timed_graph(lambda: call(budget), args.steps, args.warmup)
    log("sequential step (budget 0): same protocol")
    sq = timed_graph(lambda: call(0), args.steps, args.warmup)
    log(f"overlapped steps at budget {ov_budget}, {ov_slabs} slab(s) per tile, two streams and "
        "fused: same protocol")
    ov_s = timed_graph(lambda: call(ov_budget, cfg_streams), args.steps, args.warmup)
    ov_f = timed_graph(lambda: call(ov_budget, cfg_fused), args.steps, args.warmup)
    log("the same with every peer-bound tile also pushed to the staging buffer")
    cfg_push_s = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_STREAMS, task_slabs=ov_slabs,
                                   push_outgoing=1))
    cfg_push_f = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_FUSED, task_slabs=ov_slabs,
                                   push_outgoing=1))
    pu_s = timed_graph(lambda: call(ov_budget, cfg_push_s), args.steps, args.warmup)
    pu_f = timed_graph(lambda: call(ov_budget, cfg_push_f), args.steps, args.warmup)
    log(f"CU policy at {n_static} reduction workgroups, two streams: shared pool, then "
        f"{n_static} CUs reserved for the reduction: same protocol")
    cp_sh = timed_graph(lambda: call(n_static, cfg_streams), args.steps, args.warmup)
    cp_st = timed_graph(lambda: call(n_static, cfg_static), args.steps, args.warmup)
    # Eager calls (no graph), where the assisted schedule's helpers run: the
    # sequential step and the three overlapped schedules at the same budget.
    log(f"eager calls: sequential, two streams, fused and assisted at budget {ov_budget}")
    cfg_assist = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_ASSISTED, task_slabs=ov_slabs))
    eg = {"sequential": timed_eager(lambda: call(0), args.steps, args.warmup),
          "streams": timed_eager(lambda: call(ov_budget, cfg_streams), args.steps, args.warmup),
          "fused": timed_eager(lambda: call(ov_budget, cfg_fused), args.steps, args.warmup),
          "assisted": timed_eager(lambda: call(ov_budget, cfg_assist), args.steps, args.warmup)}

    # Every rank's step under symmetric peer readiness (each peer's tile counts
    # as ready once this GPU has produced the block at the position where the
    # peer produces it): the slowest rank bounds the step of the P-GPU operation.
    log("every rank, symmetric peer readiness: same protocol")
    sym_cfg = tog.config(**dict(cfg_kw, peer_ready=tog.PEERS_SYMMETRIC))
    seeded = [p for p in pd if p is not None]
    per_rank = []
    for r in range(w.P):
        it = iter(seeded)
        pr = [None if k == r else next(it) for k in range(w.P)]
        body = (lambda r=r, pr=pr: call(budget, sym_cfg, r, pr))
        per_rank.append(timed_graph(body, args.steps, args.warmup)["ms_per_step"] * 1e3)

    # The layer chain (Sec. 5.2.2): the same step followed by the residual
    # addition (in the reduction's store) and an RMSNorm of the rank's rows.
    log("layer chain (residual + RMSNorm): tuned step and sequential, same protocol")
    ch = timed_graph(lambda: chain(budget), args.steps, args.warmup)
    ch_sq = timed_graph(lambda: chain(0), args.steps, args.warmup)

    # Kernels alone: GEMM without flags; the reduction of the workspace's
    # partial, flat (sequential schedule) and tiled at the overlapped budget.
    # Ten launches per graph replay amortize the replay's launch latency; the
    # cold reduction subtracts a graph holding only the cache scrub.
    reps, ksteps = 10, max(10, min(args.steps, 50))
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    # The reduction's algorithmic bytes: the local fp32 partial and P-1 peer
    # contributions read, the output written.
    red_bytes = float(w.rows) * w.N * ((4 + 4 * (w.P - 1) + 4) if w.fp32_io
                                       else (4 + 2 * (w.P - 1) + 2))

    def rep(body):
        def f():
            for _ in range(reps):
                body()
        return f

    log("kernels alone")
    g_alone = timed_graph(rep(lambda: call(0, cfg_gemm)), ksteps, 3, False)["ms_per_step"] / reps
    # The same GEMM with W in the other layout (base pipeline), for the layout
    # comparison.
    other = not wkn
    Wd_other = up(W_kn if other else W)
    cfg_gemm_other = tog.config(**dict(cfg_kw, stages=tog.STAGES_GEMM,
                                       w_layout=tog.W_KN if other else tog.W_NK,
                                       gemm_variant=tog.GEMM_BASE if other else args.gemm_variant))

    def call_other():
        tog.gemm_rs(Xd, Wd_other, pd, out, w.P, w.rank, order, 0, cfg=cfg_gemm_other,
                    stream=stream)
    g_alone_other = timed_graph(rep(call_other), ksteps, 3, False)["ms_per_step"] / reps
    del Wd_other
    r_flat = timed_graph(rep(lambda: call(0, cfg_red)), ksteps, 3, False)["ms_per_step"] / reps
    r_tile = timed_graph(rep(lambda: call(ov_budget, cfg_red)), ksteps, 3,
                         False)["ms_per_step"] / reps
    t_scrub = timed_graph(lambda: scrub.fill_(1), ksteps, 3, False)["ms_per_step"]
    t_both = timed_graph(lambda: (scrub.fill_(1), call(0, cfg_red)), ksteps, 3,
                         False)["ms_per_step"]
    r_cold = max(t_both - t_scrub, 1e-6)
    # For scale, the runtime's device-to-device copy moving the same bytes
    # (half read, half written), warm and after the same scrub: what a plain
    # streaming kernel reaches at this size.
    cp_src = torch.ones(int(red_bytes) // 2, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    c_warm = timed_graph(rep(lambda: cp_dst.copy_(cp_src)), ksteps, 3,
                         False)["ms_per_step"] / reps
    c_both = timed_graph(lambda: (scrub.fill_(1), cp_dst.copy_(cp_src)), ksteps, 3,
                         False)["ms_per_step"]
    c_cold = max(c_both - t_scrub, 1e-6)
    del scrub, cp_src, cp_dst
    # The Fig. 12 analogue (Sec. 5.4.2): the tiled reduction alone (no waits,
    # warm caches) with x workgroups, x from 1 to the largest budget: how its
    # bandwidth grows with the resources given to communication.
    cfg_red_x = tog.config(**dict(cfg_kw, stages=tog.STAGES_REDUCE, task_slabs=ov_slabs))
    red_by_x = {}
    for x in (1, 2, 4, 8, 16, 32, 64, 128, 192, cus - 1):
        n = 1 if x < 32 else reps
        red_by_x[x] = timed_graph(lambda x=x, n=n: [call(x, cfg_red_x) for _ in range(n)],
                                  4 if x < 32 else ksteps, 1, False)["ms_per_step"] / n
    # ... and at the largest x with each workgroup size b (Sec. 4.3).
    red_by_b = {}
    for b_thr in (128, 256, 512):
        cb = tog.config(**dict(cfg_kw, stages=tog.STAGES_REDUCE, task_slabs=ov_slabs,
                               reducer_threads=b_thr))
        red_by_b[b_thr] = timed_graph(rep(lambda cb=cb: call(cus - 1, cb)), ksteps, 3,
                                      False)["ms_per_step"] / reps
    check_status("in the reduction-bandwidth legs")
    # For scale: a library GEMM of the same shape (hipBLASLt through
    # torch.matmul; X [M][K] times W [K][N], bf16 out), which does only the
    # GEMM part of the step.
    Wt = Wd if wkn else Wd.t().contiguous()
    lib_out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    lib_gemm = timed_graph(rep(lambda: torch.matmul(Xd, Wt, out=lib_out)), ksteps, 3,
                           False)["ms_per_step"] / reps
    del Wt, lib_out

    # The step's kernels, from HIP events recorded on each kernel's own stream
    # around eager calls: GEMM and reduction (sequential: one after the other;
    # two streams: concurrently), or the fused kernel twice.
    for _ in range(3):
        call(budget)
    stream.synchronize()
    tog.entwine_timing_read()
    tog.entwine_timing(True)
    for _ in range(ksteps):
        call(budget)
    stream.synchronize()
    tog.entwine_timing(False)
    gm, rm, n = tog.entwine_timing_read()
    check_status("in the kernel timing loop")
    k_gemm, k_red = gm / n, rm / n

    # The communication tail (Sec. 3.2, 5.3) from the device trace: the last
    # reduction's end past the last GEMM block's end, and the reduction's span
    # (first task loop entered to last store issued, waits included), median
    # over replays of a graph of the tuned step and of both overlapped legs,
    # captured with tracing on (each replay resets and records the stamps).
    def traced(body, n=21):
        tog.entwine_trace(True)
        try:
            g = graph_of(body)
            rows = []
            for _ in range(n):
                with torch.cuda.stream(stream):
                    g.replay()
                rows.append(tog.entwine_trace_read())
            del g
        finally:
            tog.entwine_trace(False)
        check_status("in the traced calls")
        med = lambda i: statistics.median(r[i] for r in rows)  # noqa: E731
        return {"gemm_end_us": med(0), "reduce_start_us": med(1), "reduce_end_us": med(2),
                "tail_us": med(3),
                "reduce_span_us": statistics.median(r[2] - r[1] for r in rows)}

    log("device trace of the communication tail: tuned step and both overlapped legs")
    tr_step = traced(lambda: call(budget))
    tr_streams = traced(lambda: call(ov_budget, cfg_streams))
    tr_fused = traced(lambda: call(ov_budget, cfg_fused))
    tr_cp_sh = traced(lambda: call(n_static, cfg_streams))
    tr_cp_st = traced(lambda: call(n_static, cfg_static))

    def traced_eager(body, n=21):
        """The device trace of eager calls (synchronized one by one)."""
        tog.entwine_trace(True)
        try:
            rows = []
            for _ in range(n):
                with torch.cuda.stream(stream):
                    body()
                stream.synchronize()
                rows.append(tog.entwine_trace_read())
        finally:
            tog.entwine_trace(False)
        check_status("in the traced eager calls")
        med = lambda i: statistics.median(r[i] for r in rows)  # noqa: E731
        return {"gemm_end_us": med(0), "reduce_start_us": med(1), "reduce_end_us": med(2),
                "tail_us": med(3),
                "reduce_span_us": statistics.median(r[2] - r[1] for r in rows)}

    tr_eager = {"sequential": traced_eager(lambda: call(0)),
                "assisted": traced_eager(lambda: call(ov_budget, cfg_assist))}

    # Ablations on the paper's two-stream schedule, each leg with the pages'
    # timing protocol (end-to-end median) and the device trace (GEMM end and
    # the communication tail, median of 21 replays).
    #  * order (Sec. 5.3.1, Fig. 7(a)): the four production orders under
    #    symmetric peer readiness, at rank 0 and rank P-1 (a rank-dependent
    #    order ranks its partitions differently; the slower of the two bounds
    #    the step);
    #  * release granularity (Sec. 5.3.2, Fig. 7(c)): tiles released alone, in
    #    groups of 4, per partition and once for the whole output;
    #  * budget response (Sec. 2.2, Fig. 2; Sec. 5.4.2): the reduction's
    #    workgroup count x, 0 being the sequential schedule.
    ablations = None
    if not args.no_ablations:
        def ablation_leg(b, o, rank=w.rank, peers=pd, **extra):
            c = tog.config(**dict(cfg_kw, schedule=tog.SCHEDULE_STREAMS, task_slabs=ov_slabs,
                                  **extra))

            def body():
                tog.gemm_rs(Xd, Wd, peers, out, w.P, rank, o, b, cfg=c, stream=stream)
            t = timed_graph(body, args.steps, args.warmup)
            tr = traced(body)
            return {"latency_us": t["ms_per_step"] * 1e3, "gemm_end_us": tr["gemm_end_us"],
                    "reduce_end_us": tr["reduce_end_us"], "tail_us": tr["tail_us"]}

        last = w.P - 1
        it = iter(seeded)
        peers_last = [None if k == last else next(it) for k in range(w.P)]
        log(f"ablation: production order, symmetric readiness, ranks 0 and {last}, budget "
            f"{ov_budget}")
        by_order = {}
        for name in ("interleaved", "col", "partition", "row"):
            o = tog.ORDERS[name]
            r0 = ablation_leg(ov_budget, o, peer_ready=tog.PEERS_SYMMETRIC)
            rl = ablation_leg(ov_budget, o, rank=last, peers=peers_last,
                              peer_ready=tog.PEERS_SYMMETRIC)
            by_order[name] = {f"rank{w.rank}": r0, f"rank{last}": rl,
                              "latency_us_max": max(r0["latency_us"], rl["latency_us"]),
                              "tail_us_max": max(r0["tail_us"], rl["tail_us"])}
        log("ablation: release granularity (interleaved order, preseeded peers)")
        by_group = {}
        for name, grp in (("tile", tog.RELEASE_TILE), ("4_tiles", 4),
                          ("partition", tog.RELEASE_PARTITION), ("output", tog.RELEASE_OUTPUT)):
            by_group[name] = ablation_leg(ov_budget, tog.ORDER_INTERLEAVED, release_group=grp)
        budgets = (list(range(0, 33)) if w.name == "ragged"
                   else [0, 1, 2, 4, 8, 16, 32, 64, 128, 192, cus - 1])
        log(f"ablation: budget response over x in {budgets}")
        by_budget = {}
        for b in budgets:
            if b >= cus:
                continue
            by_budget[str(b)] = ablation_leg(b, tog.ORDER_INTERLEAVED)
        ablations = {"schedule": "streams", "budget": ov_budget, "task_slabs": ov_slabs,
                     "order_symmetric": by_order, "release_group": by_group,
                     "budget_response": by_budget}

    flops = float(w.flops)
    # Eq. (4) (Sec. 3.3, 5.4.1): the bandwidth the reduction must sustain to
    # keep up with the GEMM is the remote volume, the P-1 peers'
    # contributions to the rank's partition, over the GEMM's time.
    remote_bytes = float(w.P - 1) * w.rows * w.N * (4 if w.fp32_io else 2)
    tflops = flops / (st["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (k_gemm * 1e-3) / 1e12
    gbps = lambda ms: red_bytes / (ms * 1e-3) / 1e9
    kernel = {"sequential": "gemm_publish_kernel (the step's GEMM)",
              "streams": "gemm_publish_kernel (inside the overlapped step)",
              "fused": "gemm_rs_fused_kernel (the whole step: GEMM and reduction)"}[kind]
    traffic_key = "gemm_rs_fused" if kind == "fused" else "gemm_publish"
    res = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K_local": w.K, "P": w.P,
                   "rank": w.rank, "schedule": kind, "block": f"{bm}x{bn}", "tile": w.tile,
                   "tile_order": order, "comm_budget": budget, "reducer_threads": threads,
                   "task_slabs": slabs, "gemm_pipeline": pipeline, "peer_ready": args.peers,
                   "w_layout": "[K_local][N]" if wkn else "[N][K_local]",
                   "source": "tuning table" if tuned and args.budget < 0 else "flags",
                   "launch": "HIP graph replay"},
        "latency_us": st["ms_per_step"] * 1e3,
        "latency_us_p10_p90": [st["p10_ms"] * 1e3, st["p90_ms"] * 1e3],
        "latency_us_back_to_back": st["back_to_back_ms"] * 1e3,
        "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS,
        # the end-to-end roofline: every workload here is MFMA-bound, so the
        # lower bound is the GEMM's FLOP at the bf16 peak
        "fraction_of_roofline": (flops / (BF16_PEAK_TFLOPS * 1e12)) / (st["ms_per_step"] * 1e-3),
        "sequential": lat(sq),
        "speedup_vs_sequential": sq["ms_per_step"] / st["ms_per_step"],
        "overlapped": {"budget": ov_budget, "task_slabs": ov_slabs,
                       "streams": lat(ov_s), "fused": lat(ov_f),
                       "best_speedup_vs_sequential":
                           sq["ms_per_step"] / min(ov_s["ms_per_step"], ov_f["ms_per_step"]),
                       # the sender's side of a push-based transfer: every
                       # peer-bound tile also copied, (M - M/P) * N * 2 * 2 bytes more
                       "push_outgoing": {"streams": lat(pu_s), "fused": lat(pu_f)},
                       # eager calls, with the assisted schedule (fused kernel
                       # plus helpers, no join); same budget and slabs
                       "eager": {**{k: lat(v) for k, v in eg.items()},
                                 "assisted_speedup_vs_sequential":
                                     eg["sequential"]["ms_per_step"] / eg["assisted"]["ms_per_step"],
                                 "trace": tr_eager}},
        # Sec. 5.3.3: shared pool against static CU partitioning, same budget
        "cu_policy": {"reduction_workgroups": n_static, "task_slabs": ov_slabs,
                      "threads": {"shared_pool": threads, "static": 512},
                      "shared_pool": lat(cp_sh), "static": lat(cp_st),
                      "shared_speedup_vs_static": cp_st["ms_per_step"] / cp_sh["ms_per_step"],
                      "trace": {"shared_pool": tr_cp_sh, "static": tr_cp_st}},
        "layer_chain": {"step": lat(ch), "sequential": lat(ch_sq),
                        "speedup_vs_sequential": ch_sq["ms_per_step"] / ch["ms_per_step"],
                        # beyond the plain step: the residual read and the norm's
                        # h read + y write, (M/P)*N*3*2 bytes
                        "extra_over_step_us": (ch["ms_per_step"] - st["ms_per_step"]) * 1e3},
        "symmetric_all_ranks": {"latency_us_max": max(per_rank),
                                "latency_us_per_rank": per_rank,
                                "speedup_vs_sequential": sq["ms_per_step"] * 1e3 / max(per_rank)},
        "gemm_alone_us": g_alone * 1e3,
        "library_gemm_us": lib_gemm * 1e3,
        "gemm_alone_us_by_w_layout": {("[K_local][N]" if wkn else "[N][K_local]"): g_alone * 1e3,
                                      ("[N][K_local]" if wkn else "[K_local][N]"):
                                          g_alone_other * 1e3},
        "gemm_alone_tflops": flops / (g_alone * 1e-3) / 1e12,
        # the GEMM inside the two-stream overlapped step (device trace: first
        # block's start to the last block's end)
        "gemm_in_overlap_tflops": flops / (max(tr_streams["gemm_end_us"], 1e-3) * 1e-6) / 1e12,
        "step_kernels_us": ({"fused": k_gemm * 1e3} if kind == "fused"
                            else {"gemm": k_gemm * 1e3, "reduction": k_red * 1e3}),
        "overlap_efficiency": g_alone / st["ms_per_step"],
        # the reduction's end past the GEMM's last block, from the device trace
        "tail_us": tr_step["tail_us"],
        "trace": {"step": tr_step, "overlapped_streams": tr_streams, "overlapped_fused": tr_fused},
        "reducer": {
            "bytes": red_bytes,
            "flat_warm_us": r_flat * 1e3,
            "flat_warm_gbps": gbps(r_flat),
            "flat_cold_us": r_cold * 1e3,
            "flat_cold_gbps": gbps(r_cold),
            "pct_hbm_peak_cold": 100.0 * gbps(r_cold) / HBM_PEAK_GBPS,
            # the runtime's device copy of the same byte count, same protocol
            "copy_same_bytes_warm_gbps": gbps(c_warm),
            "copy_same_bytes_cold_gbps": gbps(c_cold),
            "tiled_at_budget_us": r_tile * 1e3,
            "tiled_at_budget_gbps": gbps(r_tile),
            # Fig. 12 analogue: GB/s of the reduction alone against its
            # workgroup count x (task_slabs as in the overlapped legs)
            "gbps_by_workgroups": {str(x): gbps(t) for x, t in red_by_x.items()},
            f"gbps_by_threads_at_{cus - 1}_workgroups": {str(b): gbps(t)
                                                         for b, t in red_by_b.items()},
            # the reduction's HBM bytes over its traced span, waits included
            "hbm_gbps_step": gbps(max(tr_step["reduce_span_us"], 1e-3) * 1e-3),
            "hbm_gbps_overlapped_streams": gbps(max(tr_streams["reduce_span_us"], 1e-3) * 1e-3),
        },
        # Sec. 3.3 Eq. (4) and Sec. 5.4.1: required = remote volume / GEMM time
        # alone; measured = remote volume / the reduction's traced span
        "eq4": {"remote_bytes": remote_bytes,
                "required_gbps": remote_bytes / (g_alone * 1e-3) / 1e9,
                "measured_gbps_step": remote_bytes / (max(tr_step["reduce_span_us"], 1e-3) * 1e-6) / 1e9,
                "measured_gbps_overlapped_streams":
                    remote_bytes / (max(tr_streams["reduce_span_us"], 1e-3) * 1e-6) / 1e9},
        "ablations": ablations,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": traffic_for(w.name, traffic_key),
                     "kernel": kernel,
                     "kernel_us": k_gemm * 1e3,
                     "algorithmic_flops_per_launch": flops},
    }
    if not args.no_cpu:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(w, X, W, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
