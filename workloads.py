"""Seeded synthetic inputs for the GEMM-ReduceScatter hot path.

This module only draws and packs input tensors.  It holds none of the
operation's arithmetic: both the HIP library and the CPU oracle receive the
arrays produced here, and neither is imported by this module.

Workloads (one simulated rank's share of a tensor-parallel row-parallel GEMM
followed by a ReduceScatter; M x N output, K = the rank's reduction slice,
P ranks):

    tiny       256 x   256, K =  512, P = 4   64x64 tiles, fp32 peers/out
    mlp       4096 x  4096, K = 1792, P = 8   MLP down-projection slice (14336/8)
    large_mlp 8192 x  8192, K = 3584, P = 8   larger MLP slice (28672/8)
    attn_out 16384 x  5120, K = 1280, P = 4   attention out-projection (5120/4)
    ragged    1000 x 12288, K = 6144, P = 8   125-row partitions (edge tiles)

Value recipe.  X and W entries are N(0, 1/sqrt(K)) read with 1/sqrt(K) as
the variance, so each partial-product entry is ~N(0, 1); they are drawn in
fp32 and rounded to bf16 (round to nearest even).  Peer r's contribution to
the simulated rank's partition is the bf16 rounding of a seeded random GEMM of
the same shape, X_r[partition rows] @ W_r, evaluated in fp32 by numpy: it
stands in for what peer r would publish.  The tiny workload instead uses fp32
peers drawn from N(0, 1), as stated for it.

Seeds: numpy PCG64 over SeedSequence(20261202, spawn_key=(workload index,
rank, tensor id)) with tensor id 0 = X, 1 = W, 2 = peer noise, 3 = exact-case
draws, 4 = the layer chain's residual and norm weight.

Layer chain (residual addition and RMSNorm after the ReduceScatter): the
residual stream's rows of the rank's partition are N(0, 1), and the norm
weight is N(1, 0.1^2) per column; both in the output type (bf16, or fp32 for
fp32-I/O workloads).

W is handed over K-contiguous, [N][K] (element (k, n) at W[n*K + k]), the
layout in which a row-parallel linear layer keeps its weight; the [K][N]
layout is produced by :func:`w_as_kn` when a caller wants it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED = 20261202
X_ID, W_ID, PEER_ID, EXACT_ID, CHAIN_ID = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    P: int
    rank: int = 0
    tile: int = 128          # reduction tile edge (TM = TN)
    fp32_io: bool = False    # peers and output in fp32 instead of bf16
    index: int = 0           # position in WORKLOADS (seed component)

    @property
    def rows(self) -> int:
        return self.M // self.P

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = [
    Workload("tiny", 256, 256, 512, 4, tile=64, fp32_io=True, index=0),
    Workload("mlp", 4096, 4096, 1792, 8, index=1),
    Workload("large_mlp", 8192, 8192, 3584, 8, index=2),
    Workload("attn_out", 16384, 5120, 1280, 4, index=3),
    Workload("ragged", 1000, 12288, 6144, 8, index=4),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def custom(name: str, M: int, N: int, K: int, P: int, rank: int = 0, tile: int = 128,
           fp32_io: bool = False, index: int = 100) -> Workload:
    """A workload of any shape (tests use these for small multi-tile cases)."""
    return Workload(name, M, N, K, P, rank, tile, fp32_io, index)


def rng(index: int, r: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(index, r, tensor_id))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def w_as_kn(W_nk: np.ndarray) -> np.ndarray:
    """[N][K] -> [K][N] copy of the same matrix."""
    return np.ascontiguousarray(W_nk.T)


def operands(w: Workload, r: int | None = None):
    """(X [M][K], W [N][K]) bf16 bit patterns of simulated rank r."""
    r = w.rank if r is None else r
    std = np.float32(w.K ** -0.25)
    X = rng(w.index, r, X_ID).standard_normal((w.M, w.K), dtype=np.float32) * std
    W = rng(w.index, r, W_ID).standard_normal((w.N, w.K), dtype=np.float32) * std
    return bf16_bits(X), bf16_bits(W)


def peer_partials(w: Workload, rank: int | None = None) -> list:
    """Contributions V[r, rank, .] for r != rank, each [M/P][N]; None at `rank`.

    bf16 bit patterns (uint16), or float32 for fp32-I/O workloads.
    """
    rank = w.rank if rank is None else rank
    R = w.rows
    peers: list = []
    for r in range(w.P):
        if r == rank:
            peers.append(None)
            continue
        if w.fp32_io:
            peers.append(rng(w.index, r, PEER_ID).standard_normal((R, w.N), dtype=np.float32))
            continue
        Xr, Wr = operands(w, r)
        Xs = bf16_to_f32(Xr[rank * R:(rank + 1) * R])
        Wf = bf16_to_f32(Wr)
        peers.append(bf16_bits(Xs @ Wf.T))
    return peers


def exact_operands(w: Workload, r: int | None = None, nnz_per_row: int = 48,
                   peer_mag: int = 8):
    """Integer-valued inputs on which every intermediate is exact.

    X rows carry `nnz_per_row` entries of +-1 (the rest 0) and W entries are in
    {-1, 0, 1}, so every partial-product entry is an integer of magnitude
    <= nnz_per_row.  Peers are integers in [-peer_mag, peer_mag].  With the
    defaults and P <= 8 every sum is an integer below 256 in magnitude, which
    bf16, fp32 and fp64 all represent exactly.
    Returns (X bits, W bits [N][K], peers list).
    """
    r = w.rank if r is None else r
    g = rng(w.index, r, EXACT_ID)
    nnz = min(nnz_per_row, w.K)
    X = np.zeros((w.M, w.K), dtype=np.float32)
    cols = np.argsort(g.random((w.M, w.K)), axis=1)[:, :nnz]
    signs = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(w.M, nnz))
    np.put_along_axis(X, cols, signs, axis=1)
    W = g.integers(-1, 2, size=(w.N, w.K)).astype(np.float32)
    peers: list = []
    for q in range(w.P):
        if q == r:
            peers.append(None)
            continue
        v = g.integers(-peer_mag, peer_mag + 1, size=(w.rows, w.N)).astype(np.float32)
        peers.append(v if w.fp32_io else bf16_bits(v))
    return bf16_bits(X), bf16_bits(W), peers


def chain_inputs(w: Workload, rank: int | None = None):
    """(residual [M/P][N], gamma [N]) of the layer chain for rank `rank`: bf16
    bit patterns, or float32 for fp32-I/O workloads."""
    rank = w.rank if rank is None else rank
    g = rng(w.index, rank, CHAIN_ID)
    residual = g.standard_normal((w.rows, w.N), dtype=np.float32)
    gamma = (1.0 + 0.1 * g.standard_normal(w.N, dtype=np.float32)).astype(np.float32)
    if w.fp32_io:
        return residual, gamma
    return bf16_bits(residual), bf16_bits(gamma)
