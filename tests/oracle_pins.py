"""Pins for the CPU oracle: facts that hold independently of its code.

Each check takes a loaded oracle library and raises AssertionError when the
oracle disagrees with something fixed by mathematics, a library routine or a
hand-worked example.  test_oracle.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from oracle import oracle as orc
from workloads import bf16_bits, bf16_to_f32, custom, exact_operands, rng, w_as_kn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def _rand_bf16(g, shape, scale=1.0):
    return bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def pin_single_rank_is_matmul(lib):
    """P = 1: no peers, one partition, so the result is the plain product X @ W
    (numpy's fp64 matmul, a library routine).  Rectangular M != N != K so a
    transposed operand cannot pass; both W layouts."""
    g = rng(900, 0, 0)
    M, N, K = 24, 40, 16
    X = _rand_bf16(g, (M, K))
    W = _rand_bf16(g, (N, K))
    ref = _f64(X) @ _f64(W).T
    for layout, Wl in ((orc.W_NK, W), (orc.W_KN, w_as_kn(W))):
        got = orc.gemm_rs(X, Wl, [None], 1, 0, w_layout=layout, lib=lib)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        # a row sub-range is the same rows of the full result
        part = orc.gemm_rs(X, Wl, [None], 1, 0, w_layout=layout, row_begin=5,
                           row_end=17, lib=lib)
        np.testing.assert_allclose(part, ref[5:17], rtol=1e-12, atol=1e-12)


def pin_identity_X(lib):
    """X = I (M = K): the partial product is W itself, so rank d's output is
    W's rows of partition d plus the peers' contributions (exact in fp64)."""
    g = rng(901, 0, 0)
    P, N = 4, 24
    M = K = 32
    R = M // P
    X = bf16_bits(np.eye(M, dtype=np.float32))
    W = _rand_bf16(g, (N, K))
    Wkn = _f64(w_as_kn(W))  # [K][N]; row k of X@W is W(k, :)
    for rank in (0, 2, 3):
        peers = [None if r == rank else _rand_bf16(g, (R, N)) for r in range(P)]
        ref = Wkn[rank * R:(rank + 1) * R].copy()
        for r in range(P):
            if r != rank:
                ref += _f64(peers[r])
        got = orc.gemm_rs(X, W, peers, P, rank, lib=lib)
        np.testing.assert_array_equal(got, ref)


def pin_zero_W(lib):
    """W = 0: the local contribution vanishes and the output is the sum of the
    peers' contributions, in both peer dtypes."""
    g = rng(902, 0, 0)
    M, N, K, P, rank = 24, 16, 8, 3, 1
    R = M // P
    X = _rand_bf16(g, (M, K))
    W = np.zeros((N, K), dtype=np.uint16)
    for fp32 in (False, True):
        peers = []
        for r in range(P):
            if r == rank:
                peers.append(None)
            elif fp32:
                peers.append(g.standard_normal((R, N), dtype=np.float32))
            else:
                peers.append(_rand_bf16(g, (R, N)))
        ref = sum((peers[r].astype(np.float64) if fp32 else _f64(peers[r]))
                  for r in range(P) if r != rank)
        got = orc.gemm_rs(X, W, peers, P, rank, lib=lib)
        np.testing.assert_array_equal(got, ref)


def pin_row_parallel_identity(lib):
    """The defining property of row-parallel GEMM + ReduceScatter: if every
    rank r holds a K-slice (X_r, W_r) and each peer hands over exactly its
    partial product's rows, then stacking all ranks' outputs gives the
    unsharded product X_full @ W_full, where X_full and W_full concatenate
    the slices along K.  Integer inputs keep every value exact."""
    P, M, N, Kr = 3, 18, 10, 8
    R = M // P
    w = custom("pin", M, N, Kr, P, index=903)
    Xs, Ws = [], []
    for r in range(P):
        X, W, _ = exact_operands(w, r, nnz_per_row=4)
        Xs.append(X)
        Ws.append(W)
    X_full = np.concatenate([_f64(x) for x in Xs], axis=1)  # [M][P*Kr]
    W_full = np.concatenate([_f64(x) for x in Ws], axis=1)  # [N][P*Kr]
    want = X_full @ W_full.T
    C = [_f64(Xs[r]) @ _f64(Ws[r]).T for r in range(P)]
    rows = []
    for d in range(P):
        peers = [None if r == d else bf16_bits(C[r][d * R:(d + 1) * R].astype(np.float32))
                 for r in range(P)]
        rows.append(orc.gemm_rs(Xs[d], Ws[d], peers, P, d, lib=lib))
    np.testing.assert_array_equal(np.concatenate(rows, axis=0), want)


def pin_handworked(lib):
    """A hand-worked example (tests/golden/handworked_p2_rank1.json)."""
    with open(os.path.join(GOLDEN, "handworked_p2_rank1.json")) as f:
        fx = json.load(f)
    X = bf16_bits(np.array(fx["X"], dtype=np.float32))
    Wkn = bf16_bits(np.array(fx["W_kn"], dtype=np.float32))
    P, rank = fx["P"], fx["rank"]
    peers = [None] * P
    for k, v in fx["peers"].items():
        peers[int(k)] = bf16_bits(np.array(v, dtype=np.float32))
    want = np.array(fx["out"], dtype=np.float64)
    got = orc.gemm_rs(X, Wkn, peers, P, rank, w_layout=orc.W_KN, lib=lib)
    np.testing.assert_array_equal(got, want)
    got = orc.gemm_rs(X, w_as_kn(Wkn), peers, P, rank, w_layout=orc.W_NK, lib=lib)
    np.testing.assert_array_equal(got, want)


def pin_reduce_rounding(lib):
    """fp32 -> bf16 output rounding is round-to-nearest-even: compared with
    torch's CPU bfloat16 conversion on random values and on exact ties
    (1 + 2^-8 rounds down to 1, 1 + 3*2^-8 rounds up to 1 + 2^-6)."""
    g = rng(904, 0, 0)
    own = np.concatenate([
        g.standard_normal(4096, dtype=np.float32) * 3,
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 65504.5,
                  3.0e38, -3.0e38], dtype=np.float32)]).reshape(1, -1)
    zero = np.zeros_like(own)
    got = orc.reduce_f32(own, [None, zero], 2, 0, orc.BF16, lib=lib)
    want = torch.from_numpy(own).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    ties = bf16_to_f32(got[0, 4096:4098])
    np.testing.assert_array_equal(ties, np.array([1.0, 1 + 2 ** -6], dtype=np.float32))


def pin_reduce_order(lib):
    """The reduction adds in fp32 starting from the local value, then peers in
    ascending rank order.  Values where fp32 addition is not associative make
    any other order or precision visible:
      own = 2^24, V_0 = 1, V_2 = -2^24 (P = 3, rank = 1):
      ((2^24 + 1) - 2^24) = 0 in fp32 (2^24 + 1 rounds to 2^24, ties to even),
      whereas V_2 before V_0 gives 1 and exact arithmetic gives 1."""
    own = np.array([[2.0 ** 24, 1.0, 3.0]], dtype=np.float32)
    v0 = np.array([[1.0, 2.0 ** -30, -1.0]], dtype=np.float32)
    v2 = np.array([[-(2.0 ** 24), 0.0, 0.5]], dtype=np.float32)
    got = orc.reduce_f32(own, [v0, None, v2], 3, 1, orc.F32, lib=lib)
    np.testing.assert_array_equal(got, np.array([[0.0, 1.0, 2.5]], dtype=np.float32))
    # bf16 peers are widened exactly before the fp32 add
    got = orc.reduce_f32(own, [bf16_bits(v0), None, bf16_bits(v2)], 3, 1, orc.BF16, lib=lib)
    np.testing.assert_array_equal(bf16_to_f32(got), np.array([[0.0, 1.0, 2.5]], dtype=np.float32))


def pin_reduce_matches_fp64_when_exact(lib):
    """On integer data every fp32 partial sum is exact, so the fp32 reduction
    equals the fp64 operation's result (oracle_gemm_rs on the same inputs)."""
    w = custom("pin2", 48, 40, 24, 4, rank=2, index=905)
    X, W, peers = exact_operands(w, 2, nnz_per_row=6)
    ref = orc.gemm_rs(X, W, peers, 4, 2, lib=lib)
    own = (_f64(X) @ _f64(W).T)[2 * 12:3 * 12].astype(np.float32)
    got = orc.reduce_f32(own, peers, 4, 2, orc.BF16, lib=lib)
    np.testing.assert_array_equal(bf16_to_f32(got).astype(np.float64), ref)


def pin_residual_is_added_last(lib):
    """With a residual, the fp32 reduction adds it as one more term after the
    peers: the same as a reduction over one more rank whose contribution is the
    residual, at a rank index above all others.  The values are chosen so that
    adding the residual first (or in fp64) gives other bits:
      own = 2^24, V_0 = 1, residual = -2^24  ->  ((2^24 + 1) - 2^24) = 0."""
    own = np.array([[2.0 ** 24, 1.0, 3.0, -7.25]], dtype=np.float32)
    v0 = np.array([[1.0, 2.0 ** -30, -1.0, 0.25]], dtype=np.float32)
    res = np.array([[-(2.0 ** 24), 0.0, 0.5, 7.0]], dtype=np.float32)
    got = orc.reduce_f32(own, [v0, None], 2, 1, orc.F32, lib=lib, residual=res)
    np.testing.assert_array_equal(got, np.array([[0.0, 1.0, 2.5, 0.0]], dtype=np.float32))
    as_rank = orc.reduce_f32(own, [v0, None, res], 3, 1, orc.F32, lib=lib)
    np.testing.assert_array_equal(got, as_rank)
    # bf16 operands and output on random data: the same identity
    g = rng(906, 0, 0)
    own = g.standard_normal((8, 40), dtype=np.float32)
    peers = [_rand_bf16(g, (8, 40)) if r != 2 else None for r in range(4)]
    res = _rand_bf16(g, (8, 40), 4.0)
    got = orc.reduce_f32(own, peers, 4, 2, orc.BF16, lib=lib, residual=res)
    np.testing.assert_array_equal(got, orc.reduce_f32(own, peers + [res], 5, 2, orc.BF16, lib=lib))
    zero = np.zeros((8, 40), dtype=np.uint16)
    np.testing.assert_array_equal(orc.reduce_f32(own, peers, 4, 2, orc.BF16, lib=lib, residual=zero),
                                  orc.reduce_f32(own, peers, 4, 2, orc.BF16, lib=lib))


def pin_rmsnorm_handworked(lib):
    """RMSNorm by hand (tests/golden/rmsnorm_handworked.json): h = [1, 2, 3, 4],
    mean of squares 30/4 = 7.5; with eps = 0.5 the divisor is sqrt(8), so
    y = gamma * h / (2 sqrt 2)."""
    with open(os.path.join(GOLDEN, "rmsnorm_handworked.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        h = np.array(case["h"], dtype=np.float32)
        gamma = np.array(case["gamma"], dtype=np.float32)
        got = orc.rmsnorm(h, gamma, case["eps"], lib=lib)
        np.testing.assert_allclose(got, np.array(case["y"]), rtol=1e-15, atol=0)
        got = orc.rmsnorm(bf16_bits(h), bf16_bits(gamma), case["eps"], lib=lib)
        np.testing.assert_allclose(got, np.array(case["y"]), rtol=1e-15, atol=0)


def pin_rmsnorm_invariants(lib):
    """Closed forms: a constant row c gives gamma * c / sqrt(c^2 + eps); with
    eps = 0 the result does not change when a row is scaled by a > 0 and flips
    sign for a < 0; every output row has mean square mean(gamma^2 h^2)/ms."""
    g = rng(907, 0, 0)
    N = 96
    gamma = g.standard_normal(N, dtype=np.float32)
    for c, eps in ((3.0, 1e-5), (-0.125, 0.25), (1e-3, 1e-6)):
        h = np.full((1, N), c, dtype=np.float32)
        c = float(h[0, 0])  # the value stored
        got = orc.rmsnorm(h, gamma, eps, lib=lib)
        want = gamma.astype(np.float64) * c / np.sqrt(c * c + eps)
        np.testing.assert_allclose(got[0], want, rtol=1e-14, atol=0)
    h = g.standard_normal((5, N), dtype=np.float32)
    base = orc.rmsnorm(h, gamma, 0.0, lib=lib)
    for a in (2.0, 0.5, -4.0):
        got = orc.rmsnorm((h * np.float32(a)).astype(np.float32), gamma, 0.0, lib=lib)
        np.testing.assert_allclose(got, np.sign(a) * base, rtol=1e-13, atol=1e-15)
    ones = np.ones(N, dtype=np.float32)
    y = orc.rmsnorm(h, ones, 0.0, lib=lib)
    np.testing.assert_allclose((y ** 2).mean(axis=1), np.ones(5), rtol=1e-13)


ALL_PINS = [
    pin_single_rank_is_matmul,
    pin_identity_X,
    pin_zero_W,
    pin_row_parallel_identity,
    pin_handworked,
    pin_reduce_rounding,
    pin_reduce_order,
    pin_reduce_matches_fp64_when_exact,
    pin_residual_is_added_last,
    pin_rmsnorm_handworked,
    pin_rmsnorm_invariants,
]
