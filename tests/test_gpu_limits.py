"""Shapes at the library's size limits.  The kernels address a block's
operand rows, an output strip and a reduction task's rows through buffer
descriptors with 32-bit byte offsets, so the largest shapes the boundary
accepts put those offsets just below 2^31:

* wide: N = 2^22 with a 128-row partition, so one reduction task's fp32 rows
  of the own partial span 2^31 - 32 bytes;
* deep: W [K_local][N] of N * K_local * 2 = 2^31 - 2 MiB bytes.

Every element of the partition against the oracle, and the sequential and
both overlapped schedules bit-identical (the workspace poisoned before each
call)."""
import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import Case, device, down, err_ratio
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

CASES = [
    wl.custom("limit_wide", 128, 1 << 22, 64, 1, rank=0, index=360),
    wl.custom("limit_deep", 16, 16384, 65472, 1, rank=0, index=361),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_size_limits(w):
    dev = device()
    print(f"case {w.name}: {w.M}x{w.N}x{w.K} P{w.P}: generating inputs", flush=True)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    print(f"case {w.name}: oracle", flush=True)
    ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
    case = Case(w, X, W, peers, dev)
    del W
    first = {}
    for bm, bn in ((128, 128), (256, 256)):
        for budget, sched in ((0, tog.SCHEDULE_AUTO), (64, tog.SCHEDULE_STREAMS),
                              (64, tog.SCHEDULE_FUSED)):
            print(f"case {w.name}: block {bm}x{bn} budget {budget} schedule {sched}", flush=True)
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, block_m=bm, block_n=bn,
                                schedule=sched))
            ratio = err_ratio(out, ref)
            print(f"case {w.name}: max err/tol {ratio:.3f}", flush=True)
            assert ratio <= 1.0
            np.testing.assert_array_equal(out, first.setdefault((bm, bn), out))
    torch.cuda.synchronize()
