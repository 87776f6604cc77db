"""Python binding of libentwine.so: tile-overlapped GEMM-ReduceScatter on MI355X.

The functions below carry the C ABI's names (include/entwine.h) and only
marshal arguments: every step of the operation runs in the library's HIP
kernels.  PyTorch is used for device memory and streams.  If the library has
not been built, every call raises; there is no fallback path.

Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
Communication across GPUs" (paperpeel.com/paper/2609.11562), Sec. 2.1-4.3.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libentwine.so")

ENTWINE_OK = 0
ENTWINE_ERR_INVALID_ARGUMENT = 1
ENTWINE_ERR_UNSUPPORTED = 2
ENTWINE_ERR_OUT_OF_MEMORY = 3
ENTWINE_ERR_HIP = 4
ENTWINE_ERR_TIMEOUT = 5

ORDER_AUTO, ORDER_ROW_MAJOR, ORDER_PARTITION_MAJOR, ORDER_INTERLEAVED, ORDER_COL_MAJOR = -1, 0, 1, 2, 3
ORDERS = {"row": 0, "partition": 1, "interleaved": 2, "col": 3}
BUDGET_AUTO, BUDGET_SEQUENTIAL = -1, 0
BF16, F32 = 0, 1
PEERS_PRESEEDED, PEERS_SYMMETRIC = 0, 1
W_KN, W_NK = 0, 1
RELEASE_TILE, RELEASE_PARTITION, RELEASE_OUTPUT = 1, 0, -1
STAGES_ALL, STAGES_GEMM, STAGES_REDUCE = 0, 1, 2
SCHEDULE_AUTO, SCHEDULE_STREAMS, SCHEDULE_FUSED, SCHEDULE_ASSISTED = 0, 1, 2, 3
GEMM_AUTO, GEMM_PINGPONG, GEMM_BASE = 0, 4, 5

# Names exported by the library (one per declaration in include/entwine.h).
EXPORTS = [
    "entwine_gemm_rs", "entwine_config_init", "entwine_gemm_rs_ex", "entwine_gemm_rs_noalloc",
    "entwine_gemm_rs_rmsnorm",
    "entwine_plan_shape",
    "entwine_plan_blocks", "entwine_plan_dispatch", "entwine_plan_tiles", "entwine_plan_waits",
    "entwine_plan_task_order", "entwine_plan_tasks",
    "entwine_device_status", "entwine_status_string", "entwine_last_error_message",
    "entwine_workspace", "entwine_workspace_sizes", "entwine_flags", "entwine_staging",
    "entwine_timing",
    "entwine_timing_read",
    "entwine_trace", "entwine_trace_read", "entwine_load_tuning",
    "entwine_release", "entwine_device_cus",
]


class EntwineError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class entwine_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("reducer_threads", ctypes.c_int32),
        ("w_layout", ctypes.c_int32),
        ("peer_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("peer_ready", ctypes.c_int32),
        ("release_group", ctypes.c_int32),
        ("task_slabs", ctypes.c_int32),
        ("poll_timeout_ms", ctypes.c_uint32),
        ("withhold_tile", ctypes.c_int32),
        ("gemm_variant", ctypes.c_int32),
        ("publish_all", ctypes.c_int32),
        ("linear_dispatch", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("reducer_cus", ctypes.c_int32),
        ("push_outgoing", ctypes.c_int32),
        ("poll_backoff", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: the library then binds to the HIP runtime torch already
    # loaded (same soname), so the process holds a single HIP runtime.
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(the operation has no CPU fallback)")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    pcfg = ctypes.POINTER(entwine_config)
    sig = {
        "entwine_gemm_rs": ([vp, vp, ctypes.POINTER(vp), vp, i64, i64, i64, i32, i32, i32, i32, vp], i32),
        "entwine_gemm_rs_ex": ([vp, vp, ctypes.POINTER(vp), vp, i64, i64, i64, i32, i32, i32, i32, vp,
                                pcfg], i32),
        "entwine_gemm_rs_noalloc": ([vp, vp, ctypes.POINTER(vp), vp, i64, i64, i64, i32, i32, i32,
                                     i32, vp, pcfg], i32),
        "entwine_config_init": ([pcfg], None),
        "entwine_gemm_rs_rmsnorm": ([vp, vp, ctypes.POINTER(vp), vp, vp, ctypes.c_float, vp, vp,
                                     i64, i64, i64, i32, i32, i32, i32, vp, pcfg], i32),
        "entwine_plan_shape": ([i64, i64, i32, i32, i32, i32, i32, pi64, pi64, pi64], i32),
        "entwine_plan_blocks": ([i64, i64, i32, i32, i32, i32, i32, i32, i32, pi32, i64], i32),
        "entwine_plan_dispatch": ([i64, i64, i32, i32, i32, i32, i32, i32, i32, i64, pi32, i64], i32),
        "entwine_plan_tiles": ([i64, i64, i32, i32, i32, i32, i32, pi32, i64], i32),
        "entwine_plan_waits": ([i64, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32, pi32, i64], i32),
        "entwine_plan_task_order": ([i64, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32, i64,
                                     i32, pi32, i64], i32),
        "entwine_plan_tasks": ([i64, i32, i32, pi32, i64, pi64], i32),
        "entwine_device_status": ([vp], i32),
        "entwine_status_string": ([i32], ctypes.c_char_p),
        "entwine_last_error_message": ([], ctypes.c_char_p),
        "entwine_workspace": ([ctypes.POINTER(vp), ctypes.POINTER(vp), pi64], i32),
        "entwine_workspace_sizes": ([pi64, pi64, pi64], i32),
        "entwine_flags": ([ctypes.POINTER(vp), pi64, ctypes.POINTER(ctypes.c_uint32)], i32),
        "entwine_staging": ([ctypes.POINTER(vp), pi64], i32),
        "entwine_timing": ([i32], i32),
        "entwine_timing_read": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), pi64],
                                i32),
        "entwine_trace": ([i32], i32),
        "entwine_trace_read": ([ctypes.POINTER(ctypes.c_double)] * 4, i32),
        "entwine_load_tuning": ([ctypes.c_char_p], i32),
        "entwine_release": ([], i32),
        "entwine_device_cus": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc != ENTWINE_OK:
        lib = load()
        raise EntwineError(rc, f"{lib.entwine_status_string(rc).decode()}: "
                               f"{lib.entwine_last_error_message().decode()}")
    return rc


def config(**kw) -> entwine_config:
    """An entwine_config initialised by the library, with fields overridden."""
    c = entwine_config()
    load().entwine_config_init(ctypes.byref(c))
    for k, v in kw.items():
        if not hasattr(c, k):
            raise AttributeError(f"entwine_config has no field {k}")
        setattr(c, k, v)
    return c


# ---------------------------------------------------------------- raw ABI --

def entwine_gemm_rs(X: int, W: int, peer_partials: list, out: int, M: int, N: int, K_local: int,
                    P: int, rank: int, tile_order: int, comm_budget: int, stream: int,
                    cfg: entwine_config | None = None) -> int:
    """Raw pointers in, status out (raises EntwineError on failure)."""
    lib = load()
    arr = (ctypes.c_void_p * max(P, 1))(*[p or None for p in peer_partials])
    if cfg is None:
        rc = lib.entwine_gemm_rs(X, W, arr, out, M, N, K_local, P, rank, tile_order, comm_budget,
                                 stream)
    else:
        rc = lib.entwine_gemm_rs_ex(X, W, arr, out, M, N, K_local, P, rank, tile_order,
                                    comm_budget, stream, ctypes.byref(cfg))
    return _check(rc)


entwine_gemm_rs_ex = entwine_gemm_rs


def entwine_gemm_rs_noalloc(X: int, W: int, peer_partials: list, out: int, M: int, N: int,
                            K_local: int, P: int, rank: int, tile_order: int, comm_budget: int,
                            stream: int, cfg: entwine_config | None = None) -> int:
    """Raw pointers in, status out (raises EntwineError on failure): the
    operation on the library's fixed device scratch, allocating nothing."""
    lib = load()
    arr = (ctypes.c_void_p * max(P, 1))(*[p or None for p in peer_partials])
    rc = lib.entwine_gemm_rs_noalloc(X, W, arr, out, M, N, K_local, P, rank, tile_order,
                                     comm_budget, stream, ctypes.byref(cfg) if cfg else None)
    return _check(rc)


def entwine_device_status(stream: int = 0) -> int:
    return load().entwine_device_status(stream)


def entwine_timing(enable: bool) -> None:
    _check(load().entwine_timing(int(enable)))


def entwine_timing_read():
    """(summed GEMM ms, summed reduction ms, calls) since the last read."""
    g, r, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(load().entwine_timing_read(ctypes.byref(g), ctypes.byref(r), ctypes.byref(n)))
    return g.value, r.value, n.value


def entwine_trace(enable: bool) -> None:
    _check(load().entwine_trace(int(enable)))


def entwine_trace_read():
    """The last traced call's stamps in µs from its first GEMM block's start:
    (GEMM end, reduction start, reduction end, tail = reduction end - GEMM end)."""
    v = [ctypes.c_double() for _ in range(4)]
    _check(load().entwine_trace_read(*(ctypes.byref(x) for x in v)))
    return tuple(x.value for x in v)


def entwine_workspace():
    own, outg, nb = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int64()
    _check(load().entwine_workspace(ctypes.byref(own), ctypes.byref(outg), ctypes.byref(nb)))
    return own.value, outg.value, nb.value


def entwine_workspace_sizes():
    """(own partial, outgoing, staging) bytes allocated on the current device."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().entwine_workspace_sizes(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def entwine_flags():
    """(device pointer, words, next epoch) of the current device's tile flags."""
    fl, n, ep = ctypes.c_void_p(), ctypes.c_int64(), ctypes.c_uint32()
    _check(load().entwine_flags(ctypes.byref(fl), ctypes.byref(n), ctypes.byref(ep)))
    return fl.value, n.value, ep.value


def entwine_staging():
    """(device pointer, bytes) of the staging buffer that pushing calls fill."""
    st, nb = ctypes.c_void_p(), ctypes.c_int64()
    _check(load().entwine_staging(ctypes.byref(st), ctypes.byref(nb)))
    return st.value, nb.value


def entwine_load_tuning(path: str) -> None:
    _check(load().entwine_load_tuning(path.encode()))


def entwine_release() -> None:
    _check(load().entwine_release())


def entwine_device_cus() -> int:
    return load().entwine_device_cus()


def entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n):
    nb, bd, q = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n, ctypes.byref(nb),
                                     ctypes.byref(bd), ctypes.byref(q)))
    return nb.value, bd.value, q.value


def _i32_array(n):
    return (ctypes.c_int32 * max(n, 1))()


def entwine_plan_blocks(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n):
    """List of (partition, block row, block col, first tile) per logical position."""
    nb, _, _ = entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n)
    buf = _i32_array(4 * nb)
    _check(load().entwine_plan_blocks(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                                      buf, 4 * nb))
    return [tuple(buf[4 * p:4 * p + 4]) for p in range(nb)]


def entwine_plan_dispatch(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n, window):
    """Logical position computed by each GEMM workgroup (XCD-aware within windows)."""
    nb, _, _ = entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n)
    buf = _i32_array(nb)
    _check(load().entwine_plan_dispatch(M, N, P, rank, tile_order, block_m, block_n, tile_m,
                                        tile_n, window, buf, nb))
    return list(buf[:nb])


def entwine_plan_tiles(M, N, P, block_m, block_n, tile_m, tile_n):
    _, _, q = entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n)
    buf = _i32_array(2 * q)
    _check(load().entwine_plan_tiles(M, N, P, block_m, block_n, tile_m, tile_n, buf, 2 * q))
    return [tuple(buf[2 * t:2 * t + 2]) for t in range(q)]


def entwine_plan_waits(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                       peer_ready=PEERS_PRESEEDED, release_group=RELEASE_TILE):
    _, _, q = entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n)
    S = P + 1
    buf = _i32_array(q * S)
    _check(load().entwine_plan_waits(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                                     peer_ready, release_group, buf, q * S))
    return [list(buf[t * S:(t + 1) * S]) for t in range(q)]


def entwine_plan_task_order(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                            peer_ready=PEERS_PRESEEDED, release_group=RELEASE_TILE, window=0,
                            task_slabs=1):
    """The fused schedule's reduction tasks in the order workgroups take them."""
    _, _, q = entwine_plan_shape(M, N, P, block_m, block_n, tile_m, tile_n)
    n = q * task_slabs
    buf = _i32_array(n)
    _check(load().entwine_plan_task_order(M, N, P, rank, tile_order, block_m, block_n, tile_m,
                                          tile_n, peer_ready, release_group, window, task_slabs,
                                          buf, n))
    return list(buf[:n])


def entwine_plan_tasks(Q, comm_budget, consumer):
    n = ctypes.c_int64()
    load().entwine_plan_tasks(Q, comm_budget, consumer, None, 0, ctypes.byref(n))
    buf = _i32_array(n.value)
    _check(load().entwine_plan_tasks(Q, comm_budget, consumer, buf, n.value, ctypes.byref(n)))
    return list(buf[:n.value])


# ----------------------------------------------------------- torch helper --

def entwine_gemm_rs_rmsnorm(X: int, W: int, peer_partials: list, residual: int, gamma: int,
                            eps: float, h_out: int, y_out: int, M: int, N: int, K_local: int,
                            P: int, rank: int, tile_order: int, comm_budget: int, stream: int,
                            cfg: entwine_config | None = None) -> int:
    """Raw pointers in, status out (raises EntwineError on failure)."""
    lib = load()
    arr = (ctypes.c_void_p * max(P, 1))(*[p or None for p in peer_partials])
    rc = lib.entwine_gemm_rs_rmsnorm(X, W, arr, residual, gamma, eps, h_out, y_out, M, N,
                                     K_local, P, rank, tile_order, comm_budget, stream,
                                     ctypes.byref(cfg) if cfg is not None else None)
    return _check(rc)


def _check_operands(X, W, peers, out, P, rank, cfg):
    """Shapes, dtypes, devices and contiguity of the operation's operands;
    returns (M, N, K, peer pointers)."""
    import torch

    if not (X.is_cuda and W.is_cuda and out.is_cuda):
        raise ValueError("X, W and out must be device tensors")
    if W.device != X.device or out.device != X.device:
        raise ValueError("X, W and out must be on one device")
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("X and W must be bfloat16")
    for name, t in (("X", X), ("W", W), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    M, K = X.shape
    if cfg is not None and cfg.w_layout == W_NK:
        N = W.shape[0]
        if W.shape[1] != K:
            raise ValueError(f"W is {tuple(W.shape)}, expected [N][K_local] = ({N}, {K})")
    else:
        N = W.shape[1]
        if W.shape[0] != K:
            raise ValueError(f"W is {tuple(W.shape)}, expected [K_local][N] = ({K}, {N})")
    if out.shape != (M // P, N):
        raise ValueError(f"out is {tuple(out.shape)}, expected ({M // P}, {N})")
    want_out = torch.float32 if (cfg is not None and cfg.out_dtype == F32) else torch.bfloat16
    want_peer = torch.float32 if (cfg is not None and cfg.peer_dtype == F32) else torch.bfloat16
    if out.dtype != want_out:
        raise TypeError(f"out must be {want_out} for this configuration")
    ptrs = []
    for r in range(P):
        p = peers[r] if r < len(peers) else None
        if r == rank or p is None:
            ptrs.append(None)
            continue
        if not p.is_cuda or not p.is_contiguous() or p.shape != (M // P, N):
            raise ValueError(f"peer {r} must be a contiguous device tensor of shape {(M // P, N)}")
        if p.device != X.device:
            raise ValueError(f"peer {r} must be on X's device")
        if p.dtype != want_peer:
            raise TypeError(f"peer {r} must be {want_peer} for this configuration")
        ptrs.append(p.data_ptr())
    return M, N, K, ptrs


def gemm_rs(X, W, peers, out, P: int, rank: int, tile_order: int = ORDER_AUTO,
            comm_budget: int = BUDGET_AUTO, cfg: entwine_config | None = None, stream=None):
    """torch front end: checks devices, dtypes, shapes and contiguity, then
    calls entwine_gemm_rs(_ex) on the current (or given) stream.

    X [M][K] bf16, W [K][N] bf16 ([N][K] with cfg.w_layout = W_NK), peers[r]
    [M/P][N] (None at `rank`),
    out [M/P][N]; all CUDA tensors on one device.
    """
    import torch

    M, N, K, ptrs = _check_operands(X, W, peers, out, P, rank, cfg)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    return entwine_gemm_rs(X.data_ptr(), W.data_ptr(), ptrs, out.data_ptr(), M, N, K, P, rank,
                           tile_order, comm_budget, stream.cuda_stream, cfg)


def gemm_rs_noalloc(X, W, peers, out, P: int, rank: int, tile_order: int = ORDER_AUTO,
                    comm_budget: int = BUDGET_AUTO, cfg: entwine_config | None = None,
                    stream=None):
    """torch front end of entwine_gemm_rs_noalloc (same checks as gemm_rs)."""
    import torch

    M, N, K, ptrs = _check_operands(X, W, peers, out, P, rank, cfg)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    return entwine_gemm_rs_noalloc(X.data_ptr(), W.data_ptr(), ptrs, out.data_ptr(), M, N, K, P,
                                   rank, tile_order, comm_budget, stream.cuda_stream, cfg)


def gemm_rs_rmsnorm(X, W, peers, residual, gamma, eps: float, h_out, y_out, P: int, rank: int,
                    tile_order: int = ORDER_AUTO, comm_budget: int = BUDGET_AUTO,
                    cfg: entwine_config | None = None, stream=None):
    """torch front end of the layer chain: h_out = RS + residual, y_out =
    RMSNorm(h_out) * gamma.  residual and h_out [M/P][N] (may be the same
    tensor), gamma [N], y_out [M/P][N], all in the output dtype."""
    import torch

    M, N, K, ptrs = _check_operands(X, W, peers, h_out, P, rank, cfg)
    for name, t, shape in (("residual", residual, (M // P, N)), ("gamma", gamma, (N,)),
                           ("y_out", y_out, (M // P, N))):
        if not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a contiguous device tensor of shape {shape}")
        if t.dtype != h_out.dtype:
            raise TypeError(f"{name} must be {h_out.dtype}")
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    return entwine_gemm_rs_rmsnorm(X.data_ptr(), W.data_ptr(), ptrs, residual.data_ptr(),
                                   gamma.data_ptr(), eps, h_out.data_ptr(), y_out.data_ptr(), M,
                                   N, K, P, rank, tile_order, comm_budget, stream.cuda_stream,
                                   cfg)
