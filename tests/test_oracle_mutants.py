"""Plants plausible mistakes in copies of the oracle and requires the pins to
catch every one (no GPU).  The real oracle source is never modified."""
import os
import subprocess
import sys

import pytest

import oracle_pins
from oracle import oracle as orc

MUTANTS = {
    # forgot the partition's row offset
    "partition_offset": ("(int64_t)rank * R + row_begin,", "row_begin,"),
    # the last peer is dropped
    "dropped_peer": ("""        for (int r = 0; r < P; ++r) {
            if (r == rank)
                continue;
            for (int64_t j = 0; j < N; ++j)""",
                     """        for (int r = 0; r < P - 1; ++r) {
            if (r == rank)
                continue;
            for (int64_t j = 0; j < N; ++j)"""),
    # peers subtracted instead of added
    "peer_sign": ("o[j] += load_elem", "o[j] -= load_elem"),
    # peers read with their rows reversed
    "peer_rows": ("load_elem(peers[r], peer_dtype, i * N + j)",
                  "load_elem(peers[r], peer_dtype, (row_end - 1 - i + row_begin) * N + j)"),
    # W read transposed in the [N][K] layout
    "transposed_w": ("s += x[k] * w[k];", "s += x[k] * g->Wd[k * N + j];"),
    # last k dropped from the dot product
    "short_k": ("for (int64_t k = 0; k < K; ++k)\n                    s += x[k] * w[k];",
                "for (int64_t k = 0; k + 1 < K; ++k)\n                    s += x[k] * w[k];"),
    # [K][N] layout: wrong W row stride
    "kn_stride": ("const double *w = g->Wd + k * N;", "const double *w = g->Wd + k * (N - 1);"),
    # fp32 reduction in descending rank order
    "reduce_order": ("""        float acc = own[e];
        for (int r = 0; r < P; ++r) {""", """        float acc = own[e];
        for (int r = P - 1; r >= 0; --r) {"""),
    # reduction accumulates in double instead of fp32
    "reduce_precision": ("float acc = own[e];", "double acc = own[e];"),
    # round half up instead of half to even
    "rounding": ("(u + 0x7fffu + lsb) >> 16", "(u + 0x8000u) >> 16"),
    # the local contribution is left out of the reduction
    "reduce_no_local": ("float acc = own[e];", "float acc = 0.0f * own[e];"),
    # the residual is added before the peers
    "residual_first": ("""        float acc = own[e];
        for (int r = 0; r < P; ++r) {""", """        float acc = own[e];
        if (residual)
            acc = acc + (float)load_elem(residual, res_dtype, e);
        for (int r = 0; r < P; ++r) {"""),
    # the residual is not added
    "residual_dropped": ("            acc = acc + (float)load_elem(residual, res_dtype, e);",
                         "            acc = acc + 0.0f;"),
    # RMSNorm: sum of squares instead of the mean
    "rms_sum": ("sqrt(ss / (double)N + eps)", "sqrt(ss + eps)"),
    # RMSNorm: eps left out
    "rms_eps": ("sqrt(ss / (double)N + eps)", "sqrt(ss / (double)N)"),
    # RMSNorm: no square root
    "rms_sqrt": ("1.0 / sqrt(ss / (double)N + eps)", "1.0 / (ss / (double)N + eps)"),
    # RMSNorm: gamma not applied
    "rms_gamma": ("load_elem(gamma, g_dtype, j) * load_elem(h, h_dtype, i * N + j) * scale",
                  "load_elem(h, h_dtype, i * N + j) * scale"),
}


RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle_pins
from oracle import oracle as orc
lib = orc.load({so!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError):
        failed.append(pin.__name__)
print("caught by:", failed)
sys.exit(3 if failed else 0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    """A mutant counts as caught when a pin fails or the mutant crashes; the
    pins run in a child process so a crashing mutant cannot take pytest down."""
    old, new = MUTANTS[name]
    src = open(orc.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"liboracle_{name}.so")
    orc.build(src=str(path), out=so)
    tests = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(root=os.path.dirname(tests), tests=tests, so=so)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, f"no pin caught mutant {name}: {res.stdout}"


def test_runner_passes_on_the_real_oracle(tmp_path):
    """Control: the same child-process runner accepts the unmodified oracle,
    so a 'caught' verdict above is due to the planted mistake alone."""
    so = str(tmp_path / "liboracle_control.so")
    orc.build(out=so)
    tests = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(root=os.path.dirname(tests), tests=tests, so=so)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
