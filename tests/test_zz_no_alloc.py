"""entwine_gemm_rs_noalloc (for callers that cannot allocate device memory)
against entwine_gemm_rs_ex with the same arguments, through the C ABI: two
calls in a row, the second on a smaller input, each bit-identical to the
allocating entry point, for the sequential and the fused schedules; and the
refusals (a call beyond the scratch's maximum, the two-stream schedule); graph capture
of a repeated call, and the refusal of one that needs new tables."""
import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import device, down, up

pytestmark = pytest.mark.gpu

BIG = wl.custom("noalloc_big", 2048, 1536, 512, 4, rank=2, index=340)
SMALL = wl.custom("noalloc_small", 1000, 768, 256, 8, rank=5, index=341)   # 125-row partitions


def inputs(w, dev):
    X, W = wl.operands(w)
    peers = wl.peer_partials(w)
    pd = [None if p is None else up(p, dev) for p in peers]
    return up(X, dev), up(wl.w_as_kn(W), dev), pd  # W [K][N], the default layout


def call(fn, w, Xd, Wd, pd, budget, cfg):
    out = torch.full((w.rows, w.N), float("nan"), dtype=torch.bfloat16, device=Xd.device)
    ptrs = [None if p is None else p.data_ptr() for p in pd]
    stream = torch.cuda.current_stream().cuda_stream
    fn(Xd.data_ptr(), Wd.data_ptr(), ptrs, out.data_ptr(), w.M, w.N, w.K, w.P, w.rank,
       tog.ORDER_INTERLEAVED, budget, stream, cfg)
    assert tog.entwine_device_status(stream) == tog.ENTWINE_OK
    return down(out)


@pytest.mark.parametrize("budget,sched", [(0, tog.SCHEDULE_AUTO), (5, tog.SCHEDULE_FUSED),
                                          (64, tog.SCHEDULE_AUTO)])
def test_noalloc_matches_allocating_entry_point(budget, sched):
    dev = device()
    for w in (BIG, SMALL):  # the second call is on a smaller input
        print(f"no-alloc {w.name}: budget {budget} schedule {sched}", flush=True)
        Xd, Wd, pd = inputs(w, dev)
        cfg = tog.config(block_m=128, block_n=128, schedule=sched, task_slabs=2)
        got = call(tog.entwine_gemm_rs_noalloc, w, Xd, Wd, pd, budget, cfg)
        # the allocating entry point, fused schedule for overlapped budgets
        ref_cfg = tog.config(block_m=128, block_n=128, task_slabs=2,
                             schedule=tog.SCHEDULE_FUSED if budget else tog.SCHEDULE_AUTO)
        ref = call(tog.entwine_gemm_rs_ex, w, Xd, Wd, pd, budget, ref_cfg)
        assert np.isfinite(wl.bf16_to_f32(ref)).all()
        np.testing.assert_array_equal(got, ref)
        # and a repeat, on the scratch the previous call left
        again = call(tog.entwine_gemm_rs_noalloc, w, Xd, Wd, pd, budget, cfg)
        np.testing.assert_array_equal(again, ref)


def test_noalloc_refusals():
    dev = device()
    w = SMALL
    Xd, Wd, pd = inputs(w, dev)
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_ASSISTED):
        cfg = tog.config(block_m=128, block_n=128, schedule=sched)
        with pytest.raises(tog.EntwineError) as e:
            call(tog.entwine_gemm_rs_noalloc, w, Xd, Wd, pd, 4, cfg)
        assert e.value.status == tog.ENTWINE_ERR_UNSUPPORTED
    # 16384 x 8192 outputs at P = 1: a 512 MiB fp32 partial, beyond the
    # 256 MiB scratch (rejected before any launch; the buffers are not read)
    M, N, K = 16384, 8192, 64
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((K, N), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    with pytest.raises(tog.EntwineError) as e:
        tog.entwine_gemm_rs_noalloc(X.data_ptr(), W.data_ptr(), [None], out.data_ptr(), M, N, K,
                                    1, 0, tog.ORDER_INTERLEAVED, 0,
                                    torch.cuda.current_stream().cuda_stream,
                                    tog.config(block_m=128, block_n=128))
    assert e.value.status == tog.ENTWINE_ERR_OUT_OF_MEMORY


def test_noalloc_under_graph_capture():
    """A repeat of the previous no-alloc call's shape and schedule can be
    captured, and every replay equals the eager result; a call that would
    upload new schedule tables is refused while capturing, before anything
    is enqueued."""
    dev = device()
    cfg = tog.config(block_m=128, block_n=128, schedule=tog.SCHEDULE_FUSED)
    Xs, Ws, ps = inputs(SMALL, dev)
    Xb, Wb, pb = inputs(BIG, dev)
    ref = call(tog.entwine_gemm_rs_noalloc, SMALL, Xs, Ws, ps, 5, cfg)  # tables of SMALL
    stream = torch.cuda.Stream(dev)
    out = torch.full((SMALL.rows, SMALL.N), float("nan"), dtype=torch.bfloat16, device=dev)

    def enqueue(w, X, W, pd, o):
        tog.entwine_gemm_rs_noalloc(X.data_ptr(), W.data_ptr(),
                                    [None if p is None else p.data_ptr() for p in pd],
                                    o.data_ptr(), w.M, w.N, w.K, w.P, w.rank,
                                    tog.ORDER_INTERLEAVED, 5, stream.cuda_stream, cfg)

    print("case noalloc capture: refused table upload", flush=True)
    big_out = torch.empty((BIG.rows, BIG.N), dtype=torch.bfloat16, device=dev)
    g_bad = torch.cuda.CUDAGraph()
    with pytest.raises(tog.EntwineError) as e:
        with torch.cuda.graph(g_bad, stream=stream):
            enqueue(BIG, Xb, Wb, pb, big_out)
    assert e.value.status == tog.ENTWINE_ERR_INVALID_ARGUMENT
    del g_bad
    print("case noalloc capture: repeat of the previous shape, three replays", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        enqueue(SMALL, Xs, Ws, ps, out)
    for it in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        assert tog.entwine_device_status(stream.cuda_stream) == tog.ENTWINE_OK
        np.testing.assert_array_equal(down(out), ref, err_msg=f"replay {it}")
