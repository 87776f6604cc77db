"""Compile the HIP library libentwine.so for gfx950 (in-tree).

Every source under csrc/ is compiled to an object by its own hipcc process
(in parallel), then the objects are linked into
tile_overlapped_gemm_amd/libentwine.so.  Packed-fp32 instructions are
disabled for the device code; the host pass warns that it does not know the
feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libentwine.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stderr[-8000:]}")


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="entwine_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *FLAGS, *(extra or []), "-x", "hip", "-I", INCLUDE, "-I", CSRC, "-c",
                 "-o", obj, src] for src, obj in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
