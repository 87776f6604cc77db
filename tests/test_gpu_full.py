"""Every workload at full size, in the launch configurations the benchmark
times (the tuning table's AUTO choices, and its overlapped legs): sampled rows
against the CPU oracle, and bit-identity with the sequential (non-overlapped)
schedule over the whole output."""
import os

import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import Case, device, down, err_ratio
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def sample_rows(R):
    """First, middle and last rows of the partition (the last tile row is the
    ragged one when R is not a multiple of the tile)."""
    rows = sorted({0, 1, 2, R // 2, R // 2 + 1, R - 3, R - 2, R - 1})
    return [r for r in rows if 0 <= r < R]


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=lambda w: w.name)
def test_full_size_sampled_parity(w):
    dev = device()
    tog.entwine_load_tuning(os.path.join(os.path.dirname(tog.__file__), "tuning.txt"))
    print(f"workload {w.name}: generating inputs", flush=True)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    print(f"workload {w.name}: overlapped run (AUTO)", flush=True)
    out = case.run(tog.ORDER_AUTO, tog.BUDGET_AUTO)
    print(f"workload {w.name}: sequential run", flush=True)
    seq = case.run(tog.ORDER_AUTO, tog.BUDGET_SEQUENTIAL)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t  # noqa: E731
    assert torch.equal(bits(out), bits(seq))
    # Both overlapped schedules as the benchmark's overlapped legs run them when
    # the tuned step is sequential (the largest budget below the CU count, four
    # slabs per tile), and at a budget of 128 with one task per tile.
    _, _, q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    x_max = min(q * 4, tog.entwine_device_cus() - 1)
    slabs = 4 if w.tile % 4 == 0 else 1
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED):
        for budget, sl in ((x_max, slabs), (128, 1)):
            print(f"workload {w.name}: overlapped run, budget {budget}, {sl} slab(s), "
                  f"schedule {sched}", flush=True)
            got = case.run(tog.ORDER_AUTO, budget, schedule=sched, task_slabs=sl)
            assert torch.equal(bits(got), bits(seq))
    # Static CU partitioning as the benchmark's static leg runs it (32 reserved
    # CUs, four slabs), and with a quarter of the CUs reserved.
    for n in (32, 64):
        print(f"workload {w.name}: static partition, {n} reduction CUs", flush=True)
        got = case.run(tog.ORDER_AUTO, n, schedule=tog.SCHEDULE_STREAMS, task_slabs=slabs,
                       reducer_cus=n)
        assert torch.equal(bits(got), bits(seq))
    got = down(out)
    worst = 0.0
    for r in sample_rows(w.rows):
        ref = orc.gemm_rs(X, W, peers, w.P, w.rank, row_begin=r, row_end=r + 1)
        worst = max(worst, err_ratio(got[r:r + 1], ref))
    print(f"workload {w.name}: max err/tol over sampled rows {worst:.3f}", flush=True)
    assert worst <= 1.0
    del case
    torch.cuda.empty_cache()
