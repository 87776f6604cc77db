"""The layer chain (Sec. 5.2.2): GEMM-ReduceScatter, residual addition and
RMSNorm in one call, against the oracle.

Bar: h (= RS + residual) bit-exact against the oracle's fp32 reduction with
the residual as the last term, given the device's own fp32 partial, and
within 1e-2 * max(1, |ref|) of the fp64 operation; y within the same bar of
the fp64 RMSNorm of the device's h; h and y bit-identical across schedules,
orders and budgets, and in place (h_out = residual) or not.
"""
import numpy as np
import pytest
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from gpu_util import as_f64, device, down, err_ratio, poison_workspace, read_workspace, up
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SMALL = [
    wl.custom("multi", 1024, 768, 512, 4, rank=1, index=300),
    wl.custom("ragged", 1000, 1536, 512, 8, rank=5, index=301),
    wl.BY_NAME["tiny"],
]
EPS = 1e-5


class Chain:
    def __init__(self, w, dev):
        self.w = w
        self.X, self.W = wl.operands(w)
        self.peers = wl.peer_partials(w)
        self.res, self.gamma = wl.chain_inputs(w)
        # W handed over [K][N], the library's default layout
        self.Xd, self.Wd = up(self.X, dev), up(wl.w_as_kn(self.W), dev)
        self.pd = [None if p is None else up(p, dev) for p in self.peers]
        self.resd, self.gd = up(self.res, dev), up(self.gamma, dev)
        self.dtype = torch.float32 if w.fp32_io else torch.bfloat16
        self.dev = dev

    def cfg(self, **kw):
        d = dict(tile_m=self.w.tile, tile_n=self.w.tile)
        if self.w.fp32_io:
            d.update(peer_dtype=tog.F32, out_dtype=tog.F32)
        d.update(kw)
        return tog.config(**d)

    def run(self, order, budget, in_place=False, **kw):
        w = self.w
        h = self.resd.clone() if in_place else torch.full((w.rows, w.N), float("nan"),
                                                          dtype=self.dtype, device=self.dev)
        res = h if in_place else self.resd
        y = torch.full((w.rows, w.N), float("nan"), dtype=self.dtype, device=self.dev)
        poison_workspace()
        tog.gemm_rs_rmsnorm(self.Xd, self.Wd, self.pd, res, self.gd, EPS, h, y, w.P, w.rank,
                            order, budget, cfg=self.cfg(**kw))
        assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
        return down(h), down(y)


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_chain_parity_and_invariance(dev, w):
    c = Chain(w, dev)
    blk = dict(block_m=128, block_n=128)
    h0, y0 = c.run(tog.ORDER_INTERLEAVED, 0, **blk)
    # h: the reduction with the residual as its last term, bit for bit
    own, _ = read_workspace(w.rows, w.N, w.M, w.fp32_io)
    want_h = orc.reduce_f32(own, c.peers, w.P, w.rank, orc.F32 if w.fp32_io else orc.BF16,
                            residual=c.res)
    np.testing.assert_array_equal(h0, want_h)
    # h against the fp64 operation
    ref_h = orc.gemm_rs(c.X, c.W, c.peers, w.P, w.rank) + as_f64(c.res)
    assert err_ratio(h0, ref_h) <= 1.0
    # y against the fp64 RMSNorm of the device's h
    ref_y = orc.rmsnorm(h0, c.gamma, EPS)
    r = err_ratio(y0, ref_y)
    print(f"case {w.name}: y max err/tol {r:.3f}", flush=True)
    assert r <= 1.0
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED, tog.SCHEDULE_ASSISTED):
        for order, budget in ((tog.ORDER_INTERLEAVED, 4), (tog.ORDER_COL_MAJOR, 1),
                              (tog.ORDER_ROW_MAJOR, 64)):
            for in_place in (False, True):
                print(f"case {w.name} schedule {sched} order {order} budget {budget} "
                      f"in_place {in_place}", flush=True)
                h, y = c.run(order, budget, in_place=in_place, schedule=sched, **blk)
                np.testing.assert_array_equal(h, h0)
                np.testing.assert_array_equal(y, y0)
    h, y = c.run(tog.ORDER_INTERLEAVED, 0, in_place=True, **blk)
    np.testing.assert_array_equal(h, h0)
    np.testing.assert_array_equal(y, y0)


def test_chain_full_size(dev):
    """The MLP slice in the benchmark's launch configurations: the whole
    partition of h and y against the fp64 oracle, and bit-identity across the
    tuned step and both overlapped schedules (workspace poisoned before each)."""
    import os
    w = wl.BY_NAME["mlp"]
    tog.entwine_load_tuning(os.path.join(os.path.dirname(tog.__file__), "tuning.txt"))
    c = Chain(w, dev)
    print("chain mlp: AUTO and both overlapped schedules", flush=True)
    h0, y0 = c.run(tog.ORDER_AUTO, tog.BUDGET_AUTO)
    for sched in (tog.SCHEDULE_STREAMS, tog.SCHEDULE_FUSED, tog.SCHEDULE_ASSISTED):
        for budget, slabs in ((128, 1), (255, 4)):
            h, y = c.run(tog.ORDER_AUTO, budget, schedule=sched, task_slabs=slabs)
            np.testing.assert_array_equal(h, h0)
            np.testing.assert_array_equal(y, y0)
    print("chain mlp: CPU oracle over the whole partition", flush=True)
    ref_h = orc.gemm_rs(c.X, c.W, c.peers, w.P, w.rank) + as_f64(c.res)
    rh = err_ratio(h0, ref_h)
    ref_y = orc.rmsnorm(h0, c.gamma, EPS)
    ry = err_ratio(y0, ref_y)
    print(f"chain mlp: h max err/tol {rh:.3f}, y max err/tol {ry:.3f}", flush=True)
    assert rh <= 1.0 and ry <= 1.0


def test_chain_graph_replays(dev):
    w = SMALL[0]
    c = Chain(w, dev)
    cfg = c.cfg(block_m=256, block_n=128)
    h_ref, y_ref = c.run(tog.ORDER_INTERLEAVED, 5, block_m=256, block_n=128)
    h = torch.empty((w.rows, w.N), dtype=c.dtype, device=dev)
    y = torch.empty_like(h)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tog.gemm_rs_rmsnorm(c.Xd, c.Wd, c.pd, c.resd, c.gd, EPS, h, y, w.P, w.rank,
                            tog.ORDER_INTERLEAVED, 5, cfg=cfg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tog.gemm_rs_rmsnorm(c.Xd, c.Wd, c.pd, c.resd, c.gd, EPS, h, y, w.P, w.rank,
                            tog.ORDER_INTERLEAVED, 5, cfg=cfg)
    for rep in range(4):
        print(f"chain replay {rep}", flush=True)
        h.fill_(float("nan"))
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert tog.entwine_device_status(torch.cuda.current_stream().cuda_stream) == tog.ENTWINE_OK
        np.testing.assert_array_equal(down(h), h_ref)
        np.testing.assert_array_equal(down(y), y_ref)
