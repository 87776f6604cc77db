"""Parity of the HIP path with the CPU oracle on multi-tile and ragged shapes.

Bar: |out - ref| <= 1e-2 * max(1, |ref|) element by element against the fp64
oracle; bit-identical output across production orders, budgets (sequential
included), schedules (two streams, one fused kernel, or the fused kernel
with helper workgroups on another stream), reducer thread
counts, peer-readiness modes and release groups; bit-exact on integer
inputs; bit-exact reduction given the device's own fp32 partial.
"""
import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import Case, as_f64, device, down, err_ratio, hip, read_workspace
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

ORDERS = [tog.ORDER_ROW_MAJOR, tog.ORDER_PARTITION_MAJOR, tog.ORDER_INTERLEAVED, tog.ORDER_COL_MAJOR]
SMALL = [
    wl.custom("multi", 1024, 768, 512, 4, rank=1, index=300),        # 256-row partitions
    wl.custom("ragged", 1000, 1536, 512, 8, rank=5, index=301),      # 125-row partitions
    wl.custom("odd_n", 512, 1160, 256, 2, rank=1, index=302),        # N = 9*128 + 8
    wl.BY_NAME["tiny"],                                              # fp32 peers/out, 64x64 tiles
]
BLOCKS = [(128, 128), (128, 256), (256, 128), (256, 256), (128, 384)]
SCHEDULES = [tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED, tog.SCHEDULE_ASSISTED]
FUSED_KERNEL = (tog.SCHEDULE_FUSED, tog.SCHEDULE_ASSISTED)


def fused_built(bm, bn, variant):
    """The fused kernel is built for the base pipeline of every shape and variants 3 and
    4 of 256x256."""
    return variant in (tog.GEMM_AUTO, tog.GEMM_BASE) or (bm, bn) == (256, 256)


@pytest.fixture(scope="module")
def dev():
    return device()


_cases = {}


def case_for(w, dev):
    if w.name not in _cases:
        X, W = wl.operands(w)
        peers = wl.peer_partials(w)
        ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
        _cases[w.name] = (Case(w, X, W, peers, dev), ref)
    return _cases[w.name]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_parity_and_schedule_invariance(dev, w):
    case, ref = case_for(w, dev)
    _, _, q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    first = {}
    runs = 0
    for (bm, bn), variant, layout in [(b, v, lay) for b in BLOCKS
                                      for v in (tog.GEMM_BASE, 3, tog.GEMM_PINGPONG)
                                      for lay in (tog.W_NK, tog.W_KN)]:
        if w.tile == 64 and bm == 256:
            continue
        if True:
            if variant == tog.GEMM_PINGPONG and (bm, bn) != (256, 256):
                continue  # the ping-pong pipeline is built for 256 x 256 blocks
            if variant != tog.GEMM_BASE and (bm, bn) == (128, 384):
                continue  # one pipeline for 128 x 384
            if layout == tog.W_KN and variant != tog.GEMM_BASE:
                continue  # W [K][N]: the base pipeline
            for order in ORDERS:
                for budget, sched in [(b, s) for b in (0, 1, 3, min(q, 64)) for s in SCHEDULES]:
                    if sched in FUSED_KERNEL and (budget == 0 or not fused_built(bm, bn, variant)):
                        continue
                    print(f"case {w.name} block {bm}x{bn} v{variant} W {layout} order {order} "
                          f"budget {budget} schedule {sched}", flush=True)
                    if sched != tog.SCHEDULE_FUSED and budget > 0 and (
                            variant == tog.GEMM_PINGPONG or (variant == 3 and (bm, bn) == (256, 256))):
                        # The ping-pong pipeline (235 registers per lane) and
                        # the four 128 x 128 waves (256 accumulator registers
                        # plus 214) leave no room for a reduction workgroup on
                        # the GEMM's CUs (two streams, or the assisted
                        # schedule's helpers): refused, nothing runs
                        with pytest.raises(tog.EntwineError) as e:
                            case.run(order, budget, block_m=bm, block_n=bn, gemm_variant=variant,
                                     schedule=sched, w_layout=layout)
                        assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED
                        continue
                    out = down(case.run(order, budget, block_m=bm, block_n=bn, gemm_variant=variant,
                                        schedule=sched, w_layout=layout))
                    runs += 1
                    r = err_ratio(out, ref)
                    assert r <= 1.0, f"max err/tol {r:.3f}"
                    # Every block shape and pipeline adds the K steps of an
                    # output element in the same order, and the reduction's
                    # sum order is fixed: one result for the whole workload.
                    if "out" not in first:
                        first["out"] = out
                    else:
                        np.testing.assert_array_equal(out, first["out"])
    assert runs >= 2 * len(ORDERS) * (4 + 3 + 4)  # two shapes: v0 both schedules, v3 streams
    # every W [K][N] run agreed with the [N][K] ones: one result per workload


@pytest.mark.parametrize("w", SMALL[:2], ids=lambda w: w.name)
def test_reducer_variants_bit_identical(dev, w):
    case, ref = case_for(w, dev)
    blk = dict(block_m=128, block_n=128)
    base = down(case.run(tog.ORDER_INTERLEAVED, 4, **blk))
    for threads in (128, 256, 512):
        for mode in (tog.PEERS_PRESEEDED, tog.PEERS_SYMMETRIC):
            for order in (tog.ORDER_INTERLEAVED, tog.ORDER_PARTITION_MAJOR):
                for group in (tog.RELEASE_TILE, 3, tog.RELEASE_PARTITION, tog.RELEASE_OUTPUT):
                    print(f"case {w.name} b={threads} mode={mode} order={order} g={group}", flush=True)
                    out = down(case.run(order, 5, reducer_threads=threads, peer_ready=mode,
                                        release_group=group, **blk))
                    np.testing.assert_array_equal(out, base)
    for slabs in (1, 2, 8):
        for budget in (1, 5, 64):
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, task_slabs=slabs, **blk))
            np.testing.assert_array_equal(out, base)
    for publish_all in (0, 1):
        out = down(case.run(tog.ORDER_COL_MAJOR, 3, publish_all=publish_all, **blk))
        np.testing.assert_array_equal(out, base)
    out = down(case.run(tog.ORDER_INTERLEAVED, 0, **blk))
    np.testing.assert_array_equal(out, base)


@pytest.mark.parametrize("w", SMALL[:2], ids=lambda w: w.name)
def test_fused_schedule_variants_bit_identical(dev, w):
    """The fused kernel under every peer-readiness mode, release group, slab
    count, budget and publication setting gives the two-stream result."""
    case, ref = case_for(w, dev)
    blk = dict(block_m=128, block_n=128)
    base = down(case.run(tog.ORDER_INTERLEAVED, 4, **blk))
    fused = dict(schedule=tog.SCHEDULE_FUSED, **blk)
    for mode in (tog.PEERS_PRESEEDED, tog.PEERS_SYMMETRIC):
        for order in (tog.ORDER_INTERLEAVED, tog.ORDER_PARTITION_MAJOR, tog.ORDER_COL_MAJOR):
            for group in (tog.RELEASE_TILE, 3, tog.RELEASE_PARTITION, tog.RELEASE_OUTPUT):
                print(f"case {w.name} fused mode={mode} order={order} g={group}", flush=True)
                out = down(case.run(order, 5, peer_ready=mode, release_group=group, **fused))
                np.testing.assert_array_equal(out, base)
    for slabs in (1, 2, 8):
        for budget in (1, 5, 64, 255):
            budget = min(budget, tog.entwine_device_cus() - 1)
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, task_slabs=slabs, **fused))
            np.testing.assert_array_equal(out, base)
    for publish_all in (0, 1):
        out = down(case.run(tog.ORDER_ROW_MAJOR, 3, publish_all=publish_all, **fused))
        np.testing.assert_array_equal(out, base)
    # 8-wave instances take four tasks per poll round (the 4-wave 128 x 128
    # instance above takes two): 256 x 256 blocks, both readiness modes,
    # batches cut short by the task count.
    wide = dict(block_m=256, block_n=256)
    ref256 = down(case.run(tog.ORDER_INTERLEAVED, 0, **wide))
    for mode in (tog.PEERS_PRESEEDED, tog.PEERS_SYMMETRIC):
        for slabs in (1, 4):
            for budget in (1, 3, 255):
                budget = min(budget, tog.entwine_device_cus() - 1)
                print(f"case {w.name} fused 256x256 mode={mode} slabs={slabs} x={budget}",
                      flush=True)
                out = down(case.run(tog.ORDER_INTERLEAVED, budget, peer_ready=mode,
                                    task_slabs=slabs, schedule=tog.SCHEDULE_FUSED, **wide))
                np.testing.assert_array_equal(out, ref256)
    # the two schedules alternating on one workspace
    for sched in SCHEDULES * 2:
        out = down(case.run(tog.ORDER_INTERLEAVED, 6, schedule=sched, **blk))
        np.testing.assert_array_equal(out, base)


def read_staging(M, N, f32):
    ptr, nbytes = tog.entwine_staging()
    st = np.empty((M, N), dtype=np.float32 if f32 else np.uint16)
    assert ptr and nbytes >= st.nbytes
    assert hip().hipMemcpy(st.ctypes.data, ptr, st.nbytes, 2) == 0
    return st


@pytest.mark.parametrize("w", [SMALL[1], SMALL[3]], ids=lambda w: w.name)
def test_push_outgoing_copies_every_peer_tile(dev, w):
    """With push_outgoing the reduction workgroups also copy every peer-bound
    tile into the staging buffer: the output is unchanged and the staging rows
    of every other partition equal the outgoing partials bit for bit."""
    case, ref = case_for(w, dev)
    blk = dict(block_m=128, block_n=128)
    base = down(case.run(tog.ORDER_INTERLEAVED, 4, **blk))
    rows = np.ones(w.M, dtype=bool)
    rows[w.rank * w.rows:(w.rank + 1) * w.rows] = False
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 4, push_outgoing=1, schedule=tog.SCHEDULE_ASSISTED, **blk)
    assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED):
        for order, budget, slabs, mode in ((tog.ORDER_INTERLEAVED, 4, 1, tog.PEERS_PRESEEDED),
                                           (tog.ORDER_PARTITION_MAJOR, 1, 2, tog.PEERS_SYMMETRIC),
                                           (tog.ORDER_COL_MAJOR, 64, 4, tog.PEERS_PRESEEDED)):
            print(f"case {w.name} push schedule {sched} order {order} budget {budget} "
                  f"slabs {slabs} mode {mode}", flush=True)
            # a stale staging buffer must be fully overwritten
            st_ptr, st_bytes = tog.entwine_staging()
            if st_ptr:
                torch.cuda.synchronize()
                assert hip().hipMemset(st_ptr, 0x7f, st_bytes) == 0
            out = down(case.run(order, budget, push_outgoing=1, schedule=sched, task_slabs=slabs,
                                peer_ready=mode, **blk))
            np.testing.assert_array_equal(out, base)
            _, outgoing = read_workspace(w.rows, w.N, w.M, w.fp32_io)
            staging = read_staging(w.M, w.N, w.fp32_io)
            np.testing.assert_array_equal(staging[rows], outgoing[rows])
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 0, push_outgoing=1, **blk)
    assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED


def _flags(P, Q):
    ptr, words, epoch = tog.entwine_flags()
    assert words >= P * Q + 1
    f = np.empty(P * Q, dtype=np.uint32)
    assert hip().hipMemcpy(f.ctypes.data, ptr, f.nbytes, 2) == 0
    return f.reshape(P, Q), epoch


def _next_epoch(e):
    return 1 if e == 0xFFFFFFFF else e + 1


def test_flags_hold_the_call_epoch(dev):
    """The publication protocol's end state (Sec. 4.2; epoch-valued flags):
    after an overlapped call every flag it publishes holds that call's epoch
    and the epoch has advanced by one; with publish_all every tile of every
    partition is flagged; the sequential schedule publishes nothing and
    leaves the epoch."""
    w = wl.custom("flags", 1024, 768, 256, 4, rank=1, index=350)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    blk = dict(block_m=128, block_n=128)
    _, _, Q = tog.entwine_plan_shape(w.M, w.N, w.P, 128, 128, w.tile, w.tile)
    seq = down(case.run(tog.ORDER_INTERLEAVED, 0, **blk))
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED):
        print(f"case flags: schedule {sched}", flush=True)
        _, e0 = _flags(w.P, Q)
        out = down(case.run(tog.ORDER_INTERLEAVED, 5, schedule=sched, **blk))
        np.testing.assert_array_equal(out, seq)
        f, e1 = _flags(w.P, Q)
        assert e1 == _next_epoch(e0)
        assert (f[w.rank] == e0).all(), f[w.rank]
        out = down(case.run(tog.ORDER_INTERLEAVED, 5, schedule=sched, publish_all=1, **blk))
        np.testing.assert_array_equal(out, seq)
        f, e2 = _flags(w.P, Q)
        assert e2 == _next_epoch(e1)
        assert (f == e1).all(), f
    print("case flags: sequential", flush=True)
    f0, e0 = _flags(w.P, Q)
    out = down(case.run(tog.ORDER_INTERLEAVED, 0, **blk))
    np.testing.assert_array_equal(out, seq)
    f1, e1 = _flags(w.P, Q)
    assert e1 == e0
    np.testing.assert_array_equal(f1, f0)


def test_calls_from_two_host_threads(dev):
    """Two host threads, each on a stream of its own, make calls of two
    shapes (the workspace grows between them and both share it), one thread
    with the two-stream schedule and one with the fused kernel.  The library
    orders every call after the previous one on the workspace, so every
    output equals its single-thread result."""
    import threading

    cases = []
    for w in (wl.custom("thr_a", 1024, 768, 256, 4, rank=1, index=370),
              wl.custom("thr_b", 2048, 1024, 512, 8, rank=6, index=371)):
        X, W = wl.operands(w)
        peers = wl.peer_partials(w)
        case = Case(w, X, W, peers, dev)
        ref = down(case.run(tog.ORDER_INTERLEAVED, 0, block_m=128, block_n=128))
        cases.append((w, case, ref))
    errors = []

    def worker(w, case, ref, sched, budget):
        try:
            s = torch.cuda.Stream(dev)
            cfg = case.base_cfg(block_m=128, block_n=128, schedule=sched)
            outs = []
            for _ in range(6):
                out = torch.full((w.rows, w.N), float("nan"), dtype=torch.bfloat16, device=dev)
                tog.gemm_rs(case.Xd, case.Wd, case.pd, out, w.P, w.rank, tog.ORDER_INTERLEAVED,
                            budget, cfg=cfg, stream=s)
                outs.append(out)
            s.synchronize()
            for o in outs:
                np.testing.assert_array_equal(down(o), ref)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    print("case two host threads: streams and fused schedules", flush=True)
    threads = [threading.Thread(target=worker, args=(*cases[0], tog.SCHEDULE_STREAMS, 5)),
               threading.Thread(target=worker, args=(*cases[1], tog.SCHEDULE_FUSED, 7))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
    assert not errors, errors


def test_late_flags_do_not_leak_into_the_next_call(dev):
    """Regression test for the epoch hand-over of the two-stream schedule.  A
    call that releases every tile (publish_all) with preseeded peers stores
    flags of peer-bound tiles that none of its own waits read.  Row-major
    order at rank 0 produces the local partition in the first of two rounds
    of blocks, so the reduction ends while the GEMM still stores those flags.
    The epoch advances only after both kernels' workgroups have checked out,
    so the flags carry this call's epoch.  The next call pushes every
    peer-bound tile, and its send tasks wait on exactly those flags.  With the
    workspace poisoned in between, its staging rows must equal the outgoing
    partials: a send task that took an old flag for its own would copy NaN
    bytes."""
    w = wl.custom("late_flags", 4096, 2048, 4096, 4, rank=0, index=307)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    blk = dict(block_m=128, block_n=128)
    seq = down(case.run(tog.ORDER_ROW_MAJOR, 0, **blk))
    rows = np.ones(w.M, dtype=bool)
    rows[w.rank * w.rows:(w.rank + 1) * w.rows] = False
    for it in range(3):
        print(f"case late_flags iteration {it}: publish_all, then push", flush=True)
        out = down(case.run(tog.ORDER_ROW_MAJOR, 128, publish_all=1,
                            schedule=tog.SCHEDULE_STREAMS, **blk))
        np.testing.assert_array_equal(out, seq)
        out = down(case.run(tog.ORDER_ROW_MAJOR, 128, push_outgoing=1,
                            schedule=tog.SCHEDULE_STREAMS, **blk))
        np.testing.assert_array_equal(out, seq)
        _, outgoing = read_workspace(w.rows, w.N, w.M, w.fp32_io)
        staging = read_staging(w.M, w.N, w.fp32_io)
        np.testing.assert_array_equal(staging[rows], outgoing[rows])


def test_fused_many_rounds_bit_identical(dev):
    """More GEMM blocks than resident workgroups: workgroups take several
    blocks each (and take blocks from other XCDs' lists) before reducing."""
    w = wl.custom("rounds", 8192, 4096, 128, 4, rank=3, index=306)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    blk = dict(block_m=128, block_n=128)
    seq = down(case.run(tog.ORDER_INTERLEAVED, 0, **blk))
    for order in ORDERS:
        for budget in (1, 16, 200):
            print(f"case rounds order {order} budget {budget}", flush=True)
            out = down(case.run(order, budget, schedule=tog.SCHEDULE_FUSED, **blk))
            np.testing.assert_array_equal(out, seq)
    out = down(case.run(tog.ORDER_INTERLEAVED, 128, schedule=tog.SCHEDULE_FUSED, push_outgoing=1,
                        **blk))
    np.testing.assert_array_equal(out, seq)
    got = seq
    for r in (0, w.rows // 2, w.rows - 1):
        ref = orc.gemm_rs(X, W, peers, w.P, w.rank, row_begin=r, row_end=r + 1)
        assert err_ratio(got[r:r + 1], ref) <= 1.0


def test_static_cu_partitioning(dev):
    """Static CU partitioning (Sec. 5.3.3): the reduction on n CUs of its own,
    the GEMM on the rest.  Same tasks and the same fp32 sum order as the shared
    pool, so the output is bit-identical for any n, order, readiness mode and
    slab count; the fused schedule and a budget other than n are refused before
    anything is enqueued, and the workspace stays usable."""
    w = SMALL[1]
    case, ref = case_for(w, dev)
    blk = dict(block_m=128, block_n=128)
    base = down(case.run(tog.ORDER_INTERLEAVED, 0, **blk))
    assert err_ratio(base, ref) <= 1.0
    cus = tog.entwine_device_cus()
    # reducer_threads 0 picks 512-thread workgroups for the static split
    for n, order, slabs, mode, th in ((8, tog.ORDER_INTERLEAVED, 1, tog.PEERS_PRESEEDED, 0),
                                      (16, tog.ORDER_PARTITION_MAJOR, 2, tog.PEERS_SYMMETRIC, 0),
                                      (3, tog.ORDER_ROW_MAJOR, 4, tog.PEERS_PRESEEDED, 256),
                                      (cus - 8, tog.ORDER_COL_MAJOR, 1, tog.PEERS_SYMMETRIC, 128)):
        print(f"static partition: {n} reduction CUs, order {order}, {slabs} slab(s), "
              f"readiness {mode}, threads {th}", flush=True)
        out = down(case.run(order, n, reducer_cus=n, task_slabs=slabs, peer_ready=mode,
                            reducer_threads=th, **blk))
        np.testing.assert_array_equal(out, base)
    # AUTO budget and schedule follow reducer_cus
    np.testing.assert_array_equal(
        down(case.run(tog.ORDER_INTERLEAVED, tog.BUDGET_AUTO, reducer_cus=24, **blk)), base)
    # with the push of every peer-bound tile, and with a release group
    np.testing.assert_array_equal(
        down(case.run(tog.ORDER_INTERLEAVED, 16, reducer_cus=16, push_outgoing=1, **blk)), base)
    np.testing.assert_array_equal(
        down(case.run(tog.ORDER_INTERLEAVED, 16, reducer_cus=16, task_slabs=2,
                      release_group=tog.RELEASE_PARTITION, **blk)), base)
    # fp32 peers and output, 64 x 64 tiles
    tiny, tiny_ref = case_for(SMALL[3], dev)
    tiny_seq = down(tiny.run(tog.ORDER_INTERLEAVED, 0))
    assert err_ratio(tiny_seq, tiny_ref) <= 1.0
    np.testing.assert_array_equal(down(tiny.run(tog.ORDER_INTERLEAVED, 8, reducer_cus=8)),
                                  tiny_seq)
    # 256x256 blocks: the pipeline's own LDS already exceeds half of the CU's
    big = dict(block_m=256, block_n=256)
    np.testing.assert_array_equal(
        down(case.run(tog.ORDER_INTERLEAVED, 32, reducer_cus=32, task_slabs=4, **big)), base)
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 8, reducer_cus=8, schedule=tog.SCHEDULE_FUSED, **blk)
    assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 8, reducer_cus=16, **blk)
    assert e.value.status == tog.ENTWINE_ERR_INVALID_ARGUMENT
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 8, reducer_cus=cus, **blk)
    assert e.value.status == tog.ENTWINE_ERR_INVALID_ARGUMENT
    # the sequential schedule has no second kernel to place and ignores it
    np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, 0, reducer_cus=16, **blk)),
                                  base)
    np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, 8, **blk)), base)


def test_fused_unbuilt_variant_rejected(dev):
    case, _ = case_for(SMALL[0], dev)
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 4, schedule=tog.SCHEDULE_FUSED, block_m=256, block_n=256,
                 gemm_variant=1, w_layout=tog.W_NK)
    assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED


def test_reducer_that_cannot_share_a_cu_is_rejected(dev):
    """A 512-thread reduction workgroup beside a 256x256 GEMM block would need
    more registers than a SIMD holds, so waiting reducers could starve the
    GEMM of CUs: the call is refused before anything is enqueued."""
    case, _ = case_for(SMALL[0], dev)
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, 4, reducer_threads=512, block_m=256, block_n=256,
                 w_layout=tog.W_NK)
    assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED
    # the sequential schedule has no waiting reducers and stays available
    case.run(tog.ORDER_INTERLEAVED, 0, reducer_threads=512, block_m=256, block_n=256)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_reduction_bit_exact_given_own_partial(dev, w):
    """The reduction's closed form: acc = own fp32, + peers in rank order in
    fp32, one round to the output type (oracle.reduce_f32 on the device's own
    partial, read back from the workspace)."""
    case, ref = case_for(w, dev)
    out = down(case.run(tog.ORDER_INTERLEAVED, 3))
    own, outgoing = read_workspace(w.rows, w.N, w.M, w.fp32_io)
    want = orc.reduce_f32(own, case.peers, w.P, w.rank, orc.F32 if w.fp32_io else orc.BF16)
    np.testing.assert_array_equal(out, want)
    # the own partial itself is the GEMM of the partition's rows in fp32
    C = orc.partial_gemm(case.X, case.W)
    R = w.rows
    own_ref = C[w.rank * R:(w.rank + 1) * R]
    gamma = w.K * 2.0 ** -23
    absxw = orc.partial_gemm(case.X & 0x7FFF, case.W & 0x7FFF)  # sum |x||w| (sign bits cleared)
    bound = 2 * gamma * absxw[w.rank * R:(w.rank + 1) * R] + 1e-30
    assert (np.abs(own - own_ref) <= bound).all()
    # outgoing contributions (every other partition) in the peer dtype
    og = as_f64(outgoing)
    rows = np.ones(w.M, dtype=bool)
    rows[w.rank * R:(w.rank + 1) * R] = False
    rel = 2.0 ** -23 if w.fp32_io else 2.0 ** -8
    bound = rel * np.abs(C[rows]) + 2 * gamma * absxw[rows] + 1e-30
    assert (np.abs(og[rows] - C[rows]) <= bound).all()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_exact_integer_inputs_bit_exact(dev, w):
    """Integer inputs keep every intermediate exact: the device output must
    equal the oracle's value exactly, for every order and budget."""
    X, W, peers = wl.exact_operands(w)
    case = Case(w, X, W, peers, dev)
    ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
    assert (np.abs(ref) < 256).all() and (ref == np.round(ref)).all()
    for order in ORDERS:
        for budget, sched in ((0, tog.SCHEDULE_STREAMS), (2, tog.SCHEDULE_STREAMS),
                              (2, tog.SCHEDULE_FUSED), (255, tog.SCHEDULE_FUSED)):
            budget = min(budget, tog.entwine_device_cus() - 1)
            out = down(case.run(order, budget, schedule=sched, task_slabs=2))
            np.testing.assert_array_equal(as_f64(out), ref)


@pytest.mark.parametrize("sched", SCHEDULES)
def test_special_cases(dev, sched):
    """P = 1 is a plain GEMM; W = 0 leaves the sum of the peers; X = I passes
    W's rows; under both overlapped schedules (and the fused kernel's batches
    with 256 x 256 blocks)."""
    kw = dict(schedule=sched)
    w = wl.custom("p1", 256, 512, 128, 1, index=303)
    X, W = wl.operands(w)
    case = Case(w, X, W, [None], dev)
    for blk in ((128, 128), (256, 256)):
        out = down(case.run(tog.ORDER_INTERLEAVED, 2, block_m=blk[0], block_n=blk[1], **kw))
        assert err_ratio(out, orc.partial_gemm(X, W)) <= 1.0
    w = wl.custom("w0", 512, 256, 128, 4, rank=3, index=304)
    X, W = wl.operands(w)
    W[:] = 0
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    zero = np.zeros((w.rows, w.N), dtype=np.float32)
    for blk in ((128, 128), (256, 256)):
        out = down(case.run(tog.ORDER_ROW_MAJOR, 3, block_m=blk[0], block_n=blk[1], **kw))
        np.testing.assert_array_equal(out, orc.reduce_f32(zero, peers, w.P, w.rank))
    w = wl.custom("eye", 256, 384, 256, 2, rank=1, index=305)
    X = wl.bf16_bits(np.eye(256, dtype=np.float32))
    _, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    own = wl.bf16_to_f32(W.T[128:256]).copy()  # rows of W (as K x N) of partition 1
    for blk in ((128, 128), (256, 256)):
        out = down(case.run(tog.ORDER_COL_MAJOR, 1, block_m=blk[0], block_n=blk[1], **kw))
        np.testing.assert_array_equal(out, orc.reduce_f32(own, peers, w.P, w.rank))


def test_repeated_calls_and_release(dev):
    w = SMALL[1]
    case, ref = case_for(w, dev)
    a = down(case.run(tog.ORDER_INTERLEAVED, 7))
    for _ in range(5):
        np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, 7)), a)
    tog.entwine_release()
    np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, 7)), a)


@pytest.mark.parametrize("sched", SCHEDULES)
def test_watchdog_reports_timeout_then_recovers(dev, sched):
    """A tile whose flag never arrives (forced from the host) makes its
    reduction workgroup give up after the poll timeout; the device status
    reports ENTWINE_ERR_TIMEOUT once, and the next call is correct."""
    w = SMALL[0]
    case, ref = case_for(w, dev)
    good = down(case.run(tog.ORDER_INTERLEAVED, 4, schedule=sched))
    case.run(tog.ORDER_INTERLEAVED, 4, check_status=False, withhold_tile=3, poll_timeout_ms=20,
             schedule=sched)
    st = tog.entwine_device_status(torch.cuda.current_stream().cuda_stream)
    assert st == tog.ENTWINE_ERR_TIMEOUT
    assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
    np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, 4, schedule=sched)), good)


def test_timing_api(dev):
    w = SMALL[0]
    case, _ = case_for(w, dev)
    tog.entwine_timing_read()
    tog.entwine_timing(True)
    for b in (0, 4):
        case.run(tog.ORDER_INTERLEAVED, b)
    case.run(tog.ORDER_INTERLEAVED, 4, schedule=tog.SCHEDULE_FUSED)
    tog.entwine_timing(False)
    g, r, n = tog.entwine_timing_read()
    assert n == 3 and g > 0 and r > 0


def test_budget_at_cu_count_rejected(dev):
    w = SMALL[0]
    case, _ = case_for(w, dev)
    cus = tog.entwine_device_cus()
    assert cus > 0
    with pytest.raises(tog.EntwineError) as e:
        case.run(tog.ORDER_INTERLEAVED, cus)
    assert e.value.status == tog.ENTWINE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("M,N,K,P,rank", [(4, 8, 64, 4, 2),      # one row per partition, one column chunk
                                          (8, 16, 64, 8, 7),     # P = 8, last rank
                                          (96, 264, 128, 3, 0),  # 32-row partitions, N = 33*8
                                          (512, 8, 192, 2, 1)])  # a single 8-wide column
def test_degenerate_shapes(dev, M, N, K, P, rank):
    """Shapes at the smallest legal sizes: every block and tile is mostly
    masked.  All schedules and both block extremes give the oracle's result,
    and one bit pattern per block shape."""
    w = wl.custom(f"deg_{M}_{N}_{K}_{P}", M, N, K, P, rank=rank, index=330 + M % 7 + N % 5)
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    case = Case(w, X, W, peers, dev)
    ref = orc.gemm_rs(X, W, peers, w.P, w.rank)
    for bm, bn in ((128, 128), (256, 256)):
        first = None
        for budget, sched in ((0, tog.SCHEDULE_STREAMS), (1, tog.SCHEDULE_STREAMS),
                              (3, tog.SCHEDULE_FUSED), (200, tog.SCHEDULE_FUSED)):
            print(f"case deg {M}x{N}x{K} P{P} r{rank} block {bm}x{bn} budget {budget} "
                  f"schedule {sched}", flush=True)
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, block_m=bm, block_n=bn,
                                schedule=sched))
            assert err_ratio(out, ref) <= 1.0
            if first is None:
                first = out
            np.testing.assert_array_equal(out, first)


@pytest.mark.parametrize("sched", ["sequential"] + SCHEDULES)
def test_trace_stamps(dev, sched):
    """The device trace: the output is unchanged with tracing on, the stamps
    are ordered (the GEMM ends after it starts, the reduction ends after it
    starts), the tail is the reduction's end past the GEMM's, and the
    sequential reduction starts only after the GEMM kernel has ended."""
    w = SMALL[0]
    case, ref = case_for(w, dev)
    kw = dict(block_m=256, block_n=256)
    budget = 0 if sched == "sequential" else 8
    if sched != "sequential":
        kw.update(schedule=sched, task_slabs=2)
    plain = down(case.run(tog.ORDER_INTERLEAVED, budget, **kw))
    tog.entwine_trace(True)
    try:
        for _ in range(3):
            out = down(case.run(tog.ORDER_INTERLEAVED, budget, **kw))
            np.testing.assert_array_equal(out, plain)
            gemm, r0, r1, tail = tog.entwine_trace_read()
            print(f"trace {sched}: gemm {gemm:.2f} red {r0:.2f}..{r1:.2f} tail {tail:.2f} us",
                  flush=True)
            assert 0.0 < gemm < 1e6
            assert r0 <= r1 and r1 > 0.0
            assert tail == pytest.approx(r1 - gemm, abs=1e-6)
            if sched == "sequential":
                assert r0 >= gemm
        # captured with tracing on: every replay resets and records the stamps
        stream = torch.cuda.Stream()
        out_d = torch.empty((w.rows, w.N), dtype=case.out_dtype, device=dev)
        cfg = case.base_cfg(**kw)

        def body():
            tog.gemm_rs(case.Xd, case.Wd, case.pd, out_d, w.P, w.rank, tog.ORDER_INTERLEAVED,
                        budget, cfg=cfg, stream=stream)

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            body()
        for _ in range(2):
            with torch.cuda.stream(stream):
                out_d.fill_(float("nan"))
                graph.replay()
            gemm, r0, r1, tail = tog.entwine_trace_read()
            assert 0.0 < gemm < 1e6 and r0 <= r1 and r1 > 0.0
            np.testing.assert_array_equal(down(out_d), plain)
    finally:
        tog.entwine_trace(False)
    np.testing.assert_array_equal(down(case.run(tog.ORDER_INTERLEAVED, budget, **kw)), plain)
