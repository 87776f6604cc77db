"""Every workload at full size, in the launch configurations the benchmark
times (the tuning table's AUTO choices, its overlapped legs and the static CU
split): the whole partition of every leg against the CPU oracle, element by
element at the 1e-2 * max(1, |ref|) bar, and bit-identity with the sequential
(non-overlapped) schedule.  The library's workspace is overwritten with NaN
bytes before every call (gpu_util.poison_workspace), so a reduction that read
a tile before the GEMM had stored it would show."""
import os

import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import Case, device, down, err_ratio
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=lambda w: w.name)
def test_full_size_parity(w):
    dev = device()
    tog.entwine_load_tuning(os.path.join(os.path.dirname(tog.__file__), "tuning.txt"))
    print(f"workload {w.name}: generating inputs", flush=True)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    print(f"workload {w.name}: CPU oracle over the whole {w.rows}-row partition", flush=True)
    ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
    case = Case(w, X, W, peers, dev)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t  # noqa: E731
    worst = {}

    def leg(name, *args, **kw):
        print(f"workload {w.name}: {name}", flush=True)
        got = case.run(*args, **kw)
        worst[name] = err_ratio(down(got), ref)
        print(f"workload {w.name}: {name}: max err/tol {worst[name]:.3f}", flush=True)
        assert worst[name] <= 1.0, name
        return got

    # W handed over [K_local][N] (the default layout) in every leg, and once
    # [N][K_local]: both layouts give the same bits.
    seq = leg("sequential", tog.ORDER_AUTO, tog.BUDGET_SEQUENTIAL)
    out = leg("tuned step (AUTO)", tog.ORDER_AUTO, tog.BUDGET_AUTO)
    assert torch.equal(bits(out), bits(seq))
    got = leg("tuned step (AUTO), W [N][K]", tog.ORDER_AUTO, tog.BUDGET_AUTO, w_layout=tog.W_NK)
    assert torch.equal(bits(got), bits(seq))
    # The overlapped schedules as the benchmark's overlapped legs run them when
    # the tuned step is sequential (the largest budget below the CU count, four
    # slabs per tile), and at a budget of 128 with one task per tile.
    _, _, q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    x_max = min(q * 4, tog.entwine_device_cus() - 1)
    slabs = 4 if w.tile % 4 == 0 else 1
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED, tog.SCHEDULE_ASSISTED):
        for budget, sl in ((x_max, slabs), (128, 1)):
            got = leg(f"schedule {sched}, budget {budget}, {sl} slab(s)", tog.ORDER_AUTO, budget,
                      schedule=sched, task_slabs=sl)
            assert torch.equal(bits(got), bits(seq))
    # Static CU partitioning as the benchmark's static leg runs it (32 reserved
    # CUs, four slabs), and with a quarter of the CUs reserved.
    for n in (32, 64):
        got = leg(f"static partition, {n} reduction CUs", tog.ORDER_AUTO, n,
                  schedule=tog.SCHEDULE_STREAMS, task_slabs=slabs, reducer_cus=n)
        assert torch.equal(bits(got), bits(seq))
    print(f"workload {w.name}: worst err/tol {max(worst.values()):.3f}", flush=True)
    del case
    torch.cuda.empty_cache()
