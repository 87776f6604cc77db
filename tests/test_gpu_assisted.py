"""The assisted schedule (the fused kernel on the caller's stream and helper
reduction workgroups on the library's internal stream, forked from the
caller's stream and never joined back): outputs bit-identical to the
sequential step and within the oracle's bar, with the workspace poisoned
before each call and inputs that change from call to call, so that a helper
reading a tile of another call (or before its GEMM stored it) would show.
Calls are also queued back to back without host synchronization, mixed with
the other schedules on one workspace, and issued from two streams."""
import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import Case, device, down, err_ratio, poison_workspace, up
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

AS = tog.SCHEDULE_ASSISTED


@pytest.fixture(scope="module")
def dev():
    return device()


def two_cases(dev, name, M, N, K, P, rank, index):
    """Two workloads of one shape with different X (and the same W and peers):
    their outputs differ everywhere, so a stale tile cannot pass."""
    wa = wl.custom(name, M, N, K, P, rank=rank, index=index)
    Xa, W = wl.operands(wa)
    Xb, _ = wl.operands(wl.custom(name + "_b", M, N, K, P, rank=rank, index=index + 1))
    peers = wl.peer_partials(wa)
    ca, cb = Case(wa, Xa, W, peers, dev), Case(wa, Xb, W, peers, dev)
    ref = [orc.gemm_rs(Xa, W, peers, P, rank), orc.gemm_rs(Xb, W, peers, P, rank)]
    return wa, (ca, cb), ref


def test_assisted_alternating_inputs(dev):
    w, cases, ref = two_cases(dev, "assist_alt", 1024, 1536, 512, 4, 2, 330)
    seq = [down(c.run(tog.ORDER_INTERLEAVED, 0)) for c in cases]
    for i in range(2):
        assert err_ratio(seq[i], ref[i]) <= 1.0
    assert not np.array_equal(seq[0], seq[1])
    for blk in ((128, 128), (256, 256)):
        for order in (tog.ORDER_INTERLEAVED, tog.ORDER_COL_MAJOR, tog.ORDER_PARTITION_MAJOR):
            for budget, slabs in ((1, 1), (4, 2), (64, 4), (255, 4)):
                for mode in (tog.PEERS_PRESEEDED, tog.PEERS_SYMMETRIC):
                    for i in (0, 1, 0):
                        print(f"case blk {blk} order {order} budget {budget} slabs {slabs} "
                              f"mode {mode} input {i}", flush=True)
                        out = down(cases[i].run(order, budget, schedule=AS, task_slabs=slabs,
                                                peer_ready=mode, block_m=blk[0], block_n=blk[1]))
                        np.testing.assert_array_equal(out, seq[i])


def test_assisted_back_to_back(dev):
    """Twenty calls queued without synchronization, alternating inputs and
    outputs: helpers of one call may start after, or outlive, their fused
    kernel; every output must still be its own input's."""
    w, cases, ref = two_cases(dev, "assist_b2b", 2048, 1024, 768, 8, 5, 332)
    seq = [down(c.run(tog.ORDER_INTERLEAVED, 0)) for c in cases]
    cfg = cases[0].base_cfg(schedule=AS, task_slabs=4, block_m=256, block_n=256)
    outs = [torch.full((w.rows, w.N), float("nan"), dtype=torch.bfloat16, device=dev)
            for _ in range(20)]
    poison_workspace()
    for k, o in enumerate(outs):
        c = cases[k % 2]
        tog.gemm_rs(c.Xd, c.W_dev(cfg.w_layout), c.pd, o, w.P, w.rank, tog.ORDER_INTERLEAVED,
                    16 if k % 3 else 255, cfg=cfg)
    assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
    for k, o in enumerate(outs):
        np.testing.assert_array_equal(down(o), seq[k % 2])


def test_assisted_mixed_with_other_schedules_and_streams(dev):
    """One workspace, calls of every schedule in turn on two streams (the
    library orders a call after the previous one's kernels, but not after an
    assisted call's helpers, which never touch what a later call uses)."""
    w, cases, ref = two_cases(dev, "assist_mix", 1000, 1536, 512, 8, 3, 334)
    seq = [down(c.run(tog.ORDER_INTERLEAVED, 0, block_m=128, block_n=128)) for c in cases]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    plan = [(AS, 8), (tog.SCHEDULE_AUTO, 0), (AS, 200), (tog.SCHEDULE_STREAMS, 8),
            (AS, 3), (tog.SCHEDULE_FUSED, 8), (AS, 64), (AS, 1)]
    outs = []
    poison_workspace()
    for k, (sched, budget) in enumerate(plan):
        c = cases[k % 2]
        cfg = c.base_cfg(schedule=sched, block_m=128, block_n=128, task_slabs=2)
        o = torch.full((w.rows, w.N), float("nan"), dtype=torch.bfloat16, device=dev)
        s = s1 if k % 3 else s2
        with torch.cuda.stream(s):
            o.record_stream(s)
            tog.gemm_rs(c.Xd, c.W_dev(cfg.w_layout), c.pd, o, w.P, w.rank,
                        tog.ORDER_INTERLEAVED, budget, cfg=cfg, stream=s)
        outs.append((o, s))
    torch.cuda.synchronize()
    assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
    for k, (o, _) in enumerate(outs):
        np.testing.assert_array_equal(down(o), seq[k % 2])


def test_assisted_reaches_the_oracle_on_ragged_tiles(dev):
    """125-row partitions (edge tiles), fp32 peers and output, and 64 x 64 tiles."""
    for w in (wl.custom("assist_rag", 1000, 1160, 384, 8, rank=7, index=336),
              wl.BY_NAME["tiny"]):
        X, W = wl.operands(w)
        peers = wl.peer_partials(w)
        ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
        case = Case(w, X, W, peers, dev)
        base = down(case.run(tog.ORDER_INTERLEAVED, 0, block_m=128, block_n=128))
        assert err_ratio(base, ref) <= 1.0
        for budget, slabs in ((2, 1), (32, 2), (200, 4)):
            if w.tile % slabs:
                continue
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, schedule=AS, task_slabs=slabs,
                                block_m=128, block_n=128))
            np.testing.assert_array_equal(out, base)


def test_assisted_late_helpers_never_touch_a_later_call(dev):
    """Sixty calls queued back to back on the smallest shape, where the fused
    kernel reaches its tasks a few µs after it starts: helpers of one call
    may still be running when the next call's fused workgroups claim tasks
    whose flags still hold the earlier epoch.  A claim moves only from an
    older call's number, so every output must be its own input's."""
    w = wl.custom("assist_late", 512, 512, 128, 4, rank=1, index=338)
    Xa, W = wl.operands(w)
    Xb, _ = wl.operands(wl.custom("assist_late_b", 512, 512, 128, 4, rank=1, index=339))
    peers = wl.peer_partials(w)
    cases = (Case(w, Xa, W, peers, dev), Case(w, Xb, W, peers, dev))
    seq = [down(c.run(tog.ORDER_INTERLEAVED, 0, block_m=128, block_n=128)) for c in cases]
    assert err_ratio(seq[0], orc.gemm_rs(Xa, W, peers, w.P, w.rank)) <= 1.0
    assert not np.array_equal(seq[0], seq[1])
    cfg = cases[0].base_cfg(schedule=AS, task_slabs=2, block_m=128, block_n=128)
    outs = [torch.full((w.rows, w.N), float("nan"), dtype=torch.bfloat16, device=dev)
            for _ in range(60)]
    poison_workspace()
    for k, o in enumerate(outs):
        c = cases[k % 2]
        tog.gemm_rs(c.Xd, c.W_dev(cfg.w_layout), c.pd, o, w.P, w.rank, tog.ORDER_INTERLEAVED,
                    (1, 4, 16)[k % 3], cfg=cfg)
    assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
    for k, o in enumerate(outs):
        np.testing.assert_array_equal(down(o), seq[k % 2])
