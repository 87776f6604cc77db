"""Test helper: the built HIP library (built here only if nothing is built)."""
import os

import tile_overlapped_gemm_amd as tog
from tile_overlapped_gemm_amd import _build


def ensure_built():
    if not os.path.exists(tog.LIB):
        _build.build()
    return tog.load()
