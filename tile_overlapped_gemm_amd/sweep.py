"""Offline sweep that writes the tuning table read by entwine_load_tuning().

Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
Communication across GPUs" (paperpeel.com/paper/2609.11562).  Sec. 3.2 and
Sec. 5.3: the production order and the communication budget x are chosen
offline, per GEMM shape, by the measured end-to-end latency of the whole
GEMM + ReduceScatter step; x = 0 (no overlap) is one of the candidates.

Objective.  A step of the real P-GPU operation ends when the slowest rank
ends, and each rank's reduction waits for tiles that its peers produce in
their own order.  By default every candidate is therefore timed for every
rank r = 0..P-1 under SYMMETRIC peer readiness (each peer's tile counts as
ready when this GPU has produced the block at the position where the peer
produces it) and scored by the maximum over ranks.  `--objective preseeded`
scores one rank with the peers' contributions ready from the start instead.

The search is staged rather than exhaustive:
  A. every GEMM block shape and main-loop pipeline without overlap (x = 0,
     the order does not matter), and every block shape x production order
     with the two-stream schedule (base pipeline) and the fused schedule
     (every pipeline) at budget min(128, Q); and both schedules per block
     shape at the largest budget below the CU count with four slabs;
  B. for the best two overlapped (block, order, schedule) points of A: every
     budget of the list x task slabs;
  C. at the best two-stream point: reduction threads 128 / 256 / 512 (the
     fused kernel's workgroups are the GEMM's).
Each measurement is one call captured in a HIP graph and replayed; a rank's
latency is the median per-replay time (for the candidates without overlap, the
better of two passes in opposite orders).  Scores within `tie` of the best count
as equal, and the tie goes to the smaller budget, then the smaller reduction
thread count, then the smaller order enum (then the base pipeline).

Usage (one GPU):
    python -m tile_overlapped_gemm_amd.sweep --workloads mlp,large_mlp --out tuning.txt
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

BLOCKS = [(128, 128), (128, 256), (256, 128), (256, 256), (128, 384)]
BUDGETS = [0, 1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 255]
SLABS = [1, 2, 4]
THREADS = [128, 256, 512]


class Candidate:
    """One configuration; `variant` is the GEMM pipeline as the tuning table
    numbers it (0 = the base pipeline, 4 = ping-pong)."""
    __slots__ = ("bm", "bn", "order", "budget", "threads", "slabs", "schedule", "variant", "us")

    def __init__(self, bm, bn, order, budget, threads=256, slabs=1, schedule=1, variant=0,
                 us=None):
        self.bm, self.bn, self.order, self.budget = bm, bn, order, budget
        self.threads, self.slabs, self.schedule, self.us = threads, slabs, schedule, us
        self.variant = variant

    def key(self):
        return (self.bm, self.bn, self.order, self.budget, self.threads, self.slabs, self.schedule,
                self.variant)

    def __repr__(self):
        return (f"Candidate(block={self.bm}x{self.bn}, order={self.order}, x={self.budget}, "
                f"b={self.threads}, slabs={self.slabs}, schedule={self.schedule}, "
                f"variant={self.variant}, us={self.us})")


def pick(cands: list[Candidate], tie: float = 0.01) -> Candidate:
    """The best measured candidate: the lowest latency, where latencies within
    a factor (1 + tie) of the lowest count as equal and the tie goes to the
    smaller budget, then fewer reduction threads, then the smaller order enum
    (then fewer slabs, the two-stream schedule and the base pipeline)."""
    done = [c for c in cands if c.us is not None]
    if not done:
        raise ValueError("no candidate was measured")
    best = min(c.us for c in done)
    close = [c for c in done if c.us <= best * (1.0 + tie)]
    return min(close, key=lambda c: (c.budget, c.threads, c.order, c.slabs, c.schedule, c.variant,
                                     c.us))


def table_line(w, c: Candidate) -> str:
    """One tuning-table entry: M N K_local P order budget bm bn threads slabs schedule
    variant."""
    return (f"{w.M} {w.N} {w.K} {w.P} {c.order} {c.budget} {c.bm} {c.bn} {c.threads} "
            f"{c.slabs} {c.schedule} {c.variant}")


def pipelines_for(bm: int, bn: int, wkn: bool = False) -> list[int]:
    """GEMM pipelines worth timing for a block shape (tuning-table numbering);
    with W [K][N] the base pipeline only."""
    return [0, 4] if (bm, bn) == (256, 256) and not wkn else [0]


def budgets_for(q: int, cus: int) -> list[int]:
    """The budget list, without values past Q (they behave as x = Q) and below
    the CU count."""
    out = []
    for x in BUDGETS:
        if x >= cus:
            continue
        x = min(x, q)
        if x not in out:
            out.append(x)
    return out


def measure_workload(w, tog, torch, steps: int, warmup: int, objective: str, log=print,
                     w_layout: str = "kn"):
    """Run stages A-C for one workload on cuda:0, with W handed over [K][N]
    ("kn", the library's default) or [N][K] ("nk"); returns the chosen
    Candidate."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import workloads as wl

    dev = torch.device("cuda:0")
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    wkn = w_layout == "kn"
    Xd, Wd = up(X), up(wl.w_as_kn(W) if wkn else W)
    # Peer buffers for every rank's view: the values do not change the timing,
    # so the same P - 1 seeded partials serve whichever rank is local.
    seeded = [up(p) for p in peers if p is not None]
    out = torch.empty((w.rows, w.N), dtype=torch.float32 if w.fp32_io else torch.bfloat16,
                      device=dev)
    stream = torch.cuda.Stream(dev)
    cus = tog.entwine_device_cus()
    if objective == "symmetric":
        ranks, mode = list(range(w.P)), tog.PEERS_SYMMETRIC
    else:
        ranks, mode = [w.rank], tog.PEERS_PRESEEDED
    cache = {}

    def time_rank(c: Candidate, rank: int):
        kw = dict(block_m=c.bm, block_n=c.bn, tile_m=w.tile, tile_n=w.tile,
                  reducer_threads=c.threads, task_slabs=c.slabs, schedule=c.schedule,
                  peer_ready=mode, gemm_variant=c.variant or tog.GEMM_BASE,
                  w_layout=tog.W_KN if wkn else tog.W_NK)
        if w.fp32_io:
            kw.update(peer_dtype=tog.F32, out_dtype=tog.F32)
        cfg = tog.config(**kw)
        it = iter(seeded)
        pd = [None if r == rank else next(it) for r in range(w.P)]

        def body():
            tog.gemm_rs(Xd, Wd, pd, out, w.P, rank, c.order, c.budget, cfg=cfg, stream=stream)

        with torch.cuda.stream(stream):
            body()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            body()
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                g.replay()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        with torch.cuda.stream(stream):
            evs[0].record(stream)
            for i in range(steps):
                g.replay()
                evs[i + 1].record(stream)
        torch.cuda.synchronize()
        st = tog.entwine_device_status(stream.cuda_stream)
        if st != tog.ENTWINE_OK:
            raise RuntimeError(f"device status {st} for {c} at rank {rank}")
        return 1e3 * statistics.median(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))

    def run(c: Candidate, all_ranks: bool = True):
        if c.key() in cache:
            c.us = cache[c.key()]
            return c
        try:
            c.us = max(time_rank(c, r) for r in (ranks if all_ranks else ranks[:1]))
        except tog.EntwineError as e:  # e.g. a reducer that cannot share a CU
            log(f"  skip {c}: {e}")
            c.us = None
        cache[c.key()] = c.us
        log(f"  {c}")
        return c

    _, _, q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    x0 = min(128, q, cus - 1)
    # The first timings of a process run slower while the GPU's clocks ramp:
    # a throwaway warm-up of about a second first.
    warm = Candidate(256 if w.tile == 128 else 128, 256 if w.tile == 128 else 128,
                     tog.ORDER_INTERLEAVED, 0)
    t_warm = time_rank(warm, ranks[0]) * 1e-6
    for _ in range(max(1, int(1.0 / max(t_warm * (steps + warmup), 1e-3)))):
        time_rank(warm, ranks[0])
    blocks = [(bm, bn) for bm, bn in BLOCKS if bm % w.tile == 0 and bn % w.tile == 0]
    orders = (tog.ORDER_ROW_MAJOR, tog.ORDER_PARTITION_MAJOR, tog.ORDER_INTERLEAVED,
              tog.ORDER_COL_MAJOR)
    # A: no overlap (every rank takes the same time), and the overlapped
    # schedules per block shape and order
    seq = [run(Candidate(bm, bn, tog.ORDER_INTERLEAVED, 0, variant=v), all_ranks=False)
           for bm, bn in blocks for v in pipelines_for(bm, bn, wkn)]
    # Candidates timed later in a run measure slightly faster: a second pass
    # in reverse order, keeping each candidate's better time, evens that out
    # between the block shapes and pipelines without overlap.
    for c in reversed(seq):
        if c.us is not None:
            c.us = min(c.us, time_rank(c, ranks[0]))
            cache[c.key()] = c.us
            log(f"  again {c}")
    stage_a = [run(Candidate(bm, bn, order, x0, schedule=s, variant=v))
               for bm, bn in blocks for order in orders
               for s in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED)
               for v in (pipelines_for(bm, bn, wkn) if s == tog.SCHEDULE_FUSED else [0])]
    # The overlapped schedules also at the largest budget with four slabs per
    # tile (every CU takes a share of the reduction), interleaved order.
    x_max = min(q * 4, cus - 1)
    if w.tile % 4 == 0:
        stage_a += [run(Candidate(bm, bn, tog.ORDER_INTERLEAVED, x_max, slabs=4, schedule=s))
                    for bm, bn in blocks for s in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED)]
    top = sorted((c for c in stage_a if c.us is not None), key=lambda c: c.us)[:2]
    log(f"stage A: no overlap {pick(seq)}; overlapped {top}")
    # B: budget x slabs at the two best overlapped points
    stage_b = list(top)
    for a in top:
        for x in budgets_for(q, cus):
            if x == 0:
                continue
            for slabs in SLABS:
                if w.tile % slabs == 0:
                    stage_b.append(run(Candidate(a.bm, a.bn, a.order, x, slabs=slabs,
                                                 schedule=a.schedule, variant=a.variant)))
    b = pick(stage_b)
    log(f"stage B: {b}")
    # C: reduction threads for the two-stream schedule
    stage_c = [b]
    if b.schedule == tog.SCHEDULE_STREAMS:
        for t in THREADS:
            stage_c.append(run(Candidate(b.bm, b.bn, b.order, b.budget, threads=t, slabs=b.slabs,
                                         schedule=b.schedule, variant=b.variant)))
    best = pick(seq + stage_c)
    log(f"chosen: {best}; best without overlap {pick(seq)}")
    return best


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", default="tiny,mlp,large_mlp,attn_out,ragged")
    ap.add_argument("--out", default=os.path.join(PKG, "tuning.txt"))
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--w-layout", default="kn", choices=["kn", "nk"],
                    help="W handed over [K_local][N] (the default) or [N][K_local]")
    ap.add_argument("--objective", default="symmetric", choices=["symmetric", "preseeded"],
                    help="max over ranks under symmetric peer readiness, or one rank with "
                         "preseeded peers")
    args = ap.parse_args(argv)

    import torch

    sys.path.insert(0, ROOT)
    import tile_overlapped_gemm_amd as tog
    import workloads as wl

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 1
    tog.load()
    lines = []
    for name in args.workloads.split(","):
        w = wl.BY_NAME[name]
        print(f"workload {w.name}: M={w.M} N={w.N} K={w.K} P={w.P}", flush=True)
        best = measure_workload(w, tog, torch, args.steps, args.warmup, args.objective,
                                log=lambda s: print(s, flush=True), w_layout=args.w_layout)
        lines.append(f"# {w.name}: median {best.us:.1f} us per step\n{table_line(w, best)}")
    header = [
        "# Offline tuning table read by entwine_load_tuning(): the AUTO choices per shape,",
        "# written by tile_overlapped_gemm_amd/sweep.py from the median latency of",
        f"# graph-replayed steps on one MI355X (objective: {args.objective}, W "
        f"{'[K_local][N]' if args.w_layout == 'kn' else '[N][K_local]'}).",
        "# M N K_local P tile_order comm_budget block_m block_n reducer_threads task_slabs schedule "
        "gemm_variant",
    ]
    with open(args.out, "w") as f:
        f.write("\n".join(header + lines) + "\n")
    print(f"wrote {args.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
