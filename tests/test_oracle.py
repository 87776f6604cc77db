"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle_pins
from oracle import oracle as orc
from workloads import BY_NAME, custom, operands, peer_partials


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_tiny_workload_runs_and_is_finite(oracle_lib):
    """The tiny workload end to end: fp32 peers, shape and scale sanity
    (the partial product entries are ~N(0,1) by the input recipe, peers
    N(0,1), so the output variance is about P = 4)."""
    w = BY_NAME["tiny"]
    X, W = operands(w)
    peers = peer_partials(w)
    out = orc.gemm_rs(X, W, peers, w.P, w.rank, lib=oracle_lib)
    assert out.shape == (w.rows, w.N)
    assert np.isfinite(out).all()
    assert 2.0 < out.var() < 8.0


def test_row_ranges_compose(oracle_lib):
    """Computing a partition in row chunks gives the same rows as one call."""
    w = custom("chunks", 64, 48, 32, 4, rank=3, index=906)
    X, W = operands(w)
    peers = peer_partials(w)
    full = orc.gemm_rs(X, W, peers, 4, 3, lib=oracle_lib)
    a = orc.gemm_rs(X, W, peers, 4, 3, row_begin=0, row_end=5, lib=oracle_lib)
    b = orc.gemm_rs(X, W, peers, 4, 3, row_begin=5, row_end=16, threads=3, lib=oracle_lib)
    np.testing.assert_array_equal(np.concatenate([a, b]), full)


def test_rejects_bad_arguments(oracle_lib):
    w = custom("bad", 12, 8, 8, 4, index=907)
    X, W = operands(w)
    with pytest.raises(ValueError):
        orc.gemm_rs(X[:10], W, [None] * 4, 4, 0, lib=oracle_lib)  # M % P != 0
    with pytest.raises(ValueError):
        orc.gemm_rs(X, W, [None] * 4, 4, 0, lib=oracle_lib)  # missing peers
