"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  Nothing on the product path imports this
module, and this module imports nothing from the product package.

The library is built by :func:`build` (gcc, no HIP) into ``oracle/liboracle.so``.
Every function takes numpy arrays holding the exact values that the device
receives (bf16 as uint16 bit patterns, or float32) and returns fp64 results,
except :func:`reduce_f32`, the bit-exact fp32 closed form of the reduction.

Source: "Entwine: Coordinating Tiled Computation and Fine-Grained
Communication across GPUs" (paperpeel.com/paper/2609.11562), Sec. 2.1, 3.1,
4.2 (ReduceTile) and 5.2.2 (the layer chain); see oracle.c for the
definitions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

W_NK = 0  # W stored [N][K]
W_KN = 1  # W stored [K][N]
BF16 = 0
F32 = 1

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math, no HIP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-o", out, src, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB):
    """Load (building first if absent) and declare the oracle's C entry points."""
    global _lib
    if _lib is not None and path == LIB:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_partial_gemm.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i32, vp]
    lib.oracle_partial_gemm.restype = i32
    lib.oracle_gemm_rs.argtypes = [vp, vp, i32, ctypes.POINTER(vp), i32, i64, i64, i64,
                                   i32, i32, i64, i64, i32, vp]
    lib.oracle_gemm_rs.restype = i32
    lib.oracle_reduce_f32.argtypes = [vp, ctypes.POINTER(vp), i32, i32, i32, i64, i64,
                                      vp, i32, i32, vp]
    lib.oracle_reduce_f32.restype = i32
    lib.oracle_rmsnorm.argtypes = [vp, i32, vp, i32, ctypes.c_double, i64, i64, vp]
    lib.oracle_rmsnorm.restype = i32
    lib.oracle_num_threads.argtypes = [i32]
    lib.oracle_num_threads.restype = i32
    if path == LIB:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what}: oracle returned status {rc}")


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"unsupported peer dtype {a.dtype}")


def num_threads(threads: int = 0, lib=None) -> int:
    return (lib or load()).oracle_num_threads(threads)


def partial_gemm(X: np.ndarray, W: np.ndarray, w_layout: int = W_NK,
                 row_begin: int = 0, row_end: int | None = None,
                 threads: int = 0, lib=None) -> np.ndarray:
    """fp64 C[row_begin:row_end] = X[rows] @ W for bf16-bit inputs."""
    lib = lib or load()
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    M, K = X.shape
    N = W.shape[0] if w_layout == W_NK else W.shape[1]
    row_end = M if row_end is None else row_end
    C = np.empty((row_end - row_begin, N), dtype=np.float64)
    _check(lib.oracle_partial_gemm(_ptr(X), _ptr(W), w_layout, M, N, K, row_begin,
                                   row_end, threads, _ptr(C)), "partial_gemm")
    return C


def gemm_rs(X: np.ndarray, W: np.ndarray, peers: list, P: int, rank: int,
            w_layout: int = W_NK, row_begin: int = 0, row_end: int | None = None,
            threads: int = 0, lib=None) -> np.ndarray:
    """fp64 rows [row_begin,row_end) of rank `rank`'s reduce-scattered output.

    `peers[r]` is peer r's [M/P][N] contribution to this rank's partition
    (uint16 bf16 bits or float32); `peers[rank]` is ignored and may be None.
    """
    lib = lib or load()
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    M, K = X.shape
    N = W.shape[0] if w_layout == W_NK else W.shape[1]
    R = M // P
    row_end = R if row_end is None else row_end
    keep = []
    arr = (ctypes.c_void_p * P)()
    pdt = None
    for r in range(P):
        if r == rank:
            arr[r] = None
            continue
        v = np.ascontiguousarray(peers[r])
        if v.shape != (R, N):
            raise ValueError(f"peer {r} has shape {v.shape}, expected {(R, N)}")
        code = _dtype_code(v)
        if pdt is not None and code != pdt:
            raise TypeError("all peers must share one dtype")
        pdt = code
        keep.append(v)
        arr[r] = _ptr(v)
    out = np.empty((row_end - row_begin, N), dtype=np.float64)
    _check(lib.oracle_gemm_rs(_ptr(X), _ptr(W), w_layout, arr,
                              BF16 if pdt is None else pdt, M, N, K, P, rank,
                              row_begin, row_end, threads, _ptr(out)), "gemm_rs")
    return out


def reduce_f32(own: np.ndarray, peers: list, P: int, rank: int,
               out_dtype: int = BF16, lib=None, residual: np.ndarray | None = None) -> np.ndarray:
    """Bit-exact fp32 reduction: acc = own, += peers ascending, += residual
    (if given), round to out."""
    lib = lib or load()
    own = np.ascontiguousarray(own, dtype=np.float32)
    rows, N = own.shape
    keep = []
    arr = (ctypes.c_void_p * P)()
    pdt = BF16
    for r in range(P):
        if r == rank:
            arr[r] = None
            continue
        v = np.ascontiguousarray(peers[r])
        if v.shape != (rows, N):
            raise ValueError(f"peer {r} has shape {v.shape}, expected {(rows, N)}")
        pdt = _dtype_code(v)
        keep.append(v)
        arr[r] = _ptr(v)
    out = np.empty((rows, N), dtype=np.uint16 if out_dtype == BF16 else np.float32)
    res_ptr, res_dt = None, BF16
    if residual is not None:
        residual = np.ascontiguousarray(residual)
        if residual.shape != (rows, N):
            raise ValueError(f"residual has shape {residual.shape}, expected {(rows, N)}")
        res_ptr, res_dt = _ptr(residual), _dtype_code(residual)
    _check(lib.oracle_reduce_f32(_ptr(own), arr, pdt, P, rank, rows, N, res_ptr, res_dt,
                                 out_dtype, _ptr(out)), "reduce_f32")
    return out


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float, lib=None) -> np.ndarray:
    """fp64 RMSNorm of each row: gamma * h / sqrt(mean(h^2) + eps)."""
    lib = lib or load()
    h = np.ascontiguousarray(h)
    gamma = np.ascontiguousarray(gamma)
    rows, N = h.shape
    if gamma.shape != (N,):
        raise ValueError(f"gamma has shape {gamma.shape}, expected {(N,)}")
    y = np.empty((rows, N), dtype=np.float64)
    _check(lib.oracle_rmsnorm(_ptr(h), _dtype_code(h), _ptr(gamma), _dtype_code(gamma),
                              float(eps), rows, N, _ptr(y)), "rmsnorm")
    return y
