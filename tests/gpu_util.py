"""Helpers for GPU tests: upload seeded inputs, call the library, read back."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import tile_overlapped_gemm_amd as tog
import workloads as wl
from libentwine import ensure_built

_hip = None


def hip():
    global _hip
    if _hip is None:
        # the HIP runtime already loaded by torch (and used by the library)
        torch.cuda.init()
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
        _hip.hipMemset.restype = ctypes.c_int
    return _hip


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()
    return torch.device("cuda:0")


def up(a: np.ndarray, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def down(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def poison_workspace() -> bool:
    """Overwrite the library's own-partial, outgoing and staging buffers with
    0xFF bytes (a NaN in fp32 and in bf16), with the device idle before and
    after.  A call that then read any of them before its own GEMM had stored
    and released the data would return NaN or differ from the reference, where
    without the poison it would read the identical values the previous call
    left behind.  Writes stay within the allocated sizes.  Returns False when
    the device has no workspace yet (the next call allocates it)."""
    torch.cuda.synchronize()
    try:
        own_p, og_p, _ = tog.entwine_workspace()
        own_b, og_b, st_b = tog.entwine_workspace_sizes()
    except tog.EntwineError:
        return False
    for p, n in ((own_p, own_b), (og_p, og_b)):
        if p and n:
            assert hip().hipMemset(p, 0xFF, n) == 0
    if st_b:
        st_p, _ = tog.entwine_staging()
        assert hip().hipMemset(st_p, 0xFF, st_b) == 0
    torch.cuda.synchronize()
    return True


def as_f64(a: np.ndarray) -> np.ndarray:
    return (wl.bf16_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


class Case:
    """Device copies of one workload's inputs plus an output buffer.  W (drawn
    [N][K] by workloads.operands) is handed over in the layout a call's
    configuration names: [K][N] by default (the library's default), [N][K]
    with w_layout=tog.W_NK."""

    def __init__(self, w: wl.Workload, X, W, peers, dev, w_layout=tog.W_KN):
        self.w = w
        self.X, self.W, self.peers = X, W, peers
        self.w_layout = w_layout
        self.Xd = up(X, dev)
        self._Wd = {}
        self.pd = [None if p is None else up(p, dev) for p in peers]
        self.out_dtype = torch.float32 if w.fp32_io else torch.bfloat16
        self.dev = dev

    def W_dev(self, layout):
        if layout not in self._Wd:
            self._Wd[layout] = up(wl.w_as_kn(self.W) if layout == tog.W_KN else self.W, self.dev)
        return self._Wd[layout]

    @property
    def Wd(self):
        return self.W_dev(self.w_layout)

    def base_cfg(self, **kw):
        d = dict(tile_m=self.w.tile, tile_n=self.w.tile, w_layout=self.w_layout)
        if self.w.fp32_io:
            d.update(peer_dtype=tog.F32, out_dtype=tog.F32)
        d.update(kw)
        return tog.config(**d)

    def run(self, order=tog.ORDER_INTERLEAVED, budget=4, check_status=True, poison=True, **kw):
        """One call into a NaN-filled output, after poisoning the workspace
        (poison_workspace) unless poison=False."""
        out = torch.full((self.w.rows, self.w.N), float("nan"), dtype=self.out_dtype, device=self.dev)
        if poison:
            poison_workspace()
        cfg = self.base_cfg(**kw)
        tog.gemm_rs(self.Xd, self.W_dev(cfg.w_layout), self.pd, out, self.w.P, self.w.rank, order,
                    budget, cfg=cfg)
        if check_status:
            st = tog.entwine_device_status(torch.cuda.current_stream().cuda_stream)
            assert st == tog.ENTWINE_OK, f"device status {st}"
        return out


def read_workspace(rows: int, N: int, M: int, outgoing_f32: bool):
    """(own fp32 [rows][N], outgoing [M][N]) as written by the last call."""
    own_p, out_p, _ = tog.entwine_workspace()
    own = np.empty((rows, N), dtype=np.float32)
    assert hip().hipMemcpy(own.ctypes.data, own_p, own.nbytes, 2) == 0
    og = np.empty((M, N), dtype=np.float32 if outgoing_f32 else np.uint16)
    assert hip().hipMemcpy(og.ctypes.data, out_p, og.nbytes, 2) == 0
    return own, og


def err_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / (1e-2 * max(1, |ref|)); <= 1 passes the parity bar."""
    g = as_f64(got)
    assert np.isfinite(g).all(), "non-finite output (an element was never written?)"
    return float((np.abs(g - ref) / (1e-2 * np.maximum(1.0, np.abs(ref)))).max())
