"""Build libgemmepi.so in-tree with hipcc for gfx950.

Every translation unit is compiled to an object under ``_build/`` (in
parallel), then linked into ``activation_epilogue_gemm_amd/libgemmepi.so``.
Runs without a GPU: hipcc cross-compiles for the named offload target.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemmepi.so")
# measurement helpers used by the benchmark only, in a library of their own
MEASURE_SOURCES = ["measure.hip"]
MEASURE_LIB = os.path.join(PKG, "libgemmepi_measure.so")
# the LDS race-detector build of the same library (GEMMEPI_LDS_POISON=1), for
# tests/test_gpu_lds_poison.py only
POISON_LIB = os.path.join(PKG, "libgemmepi_poison.so")
POISON_FLAGS = ["-DGEMMEPI_LDS_POISON=1"]

SOURCES = [
    "gemmepi_api.cpp",
    "elementwise.hip",
    "decode.hip",
    "noalloc.hip",
    "gemm_f16_bn.hip",
    "gemm_f16_bt.hip",
    "gemm_bf16_bn.hip",
    "gemm_bf16_bt.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags(extra=()):
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # keep fp32 arithmetic scalar: no packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *extra,
    ]


def _compile(src: str, extra=(), objdir: str = "") -> str:
    obj = os.path.join(objdir or BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, jobs: int = 0, extra=(), poison: bool = True) -> str:
    """Compile every source and link the shared library (plus the measurement
    library and, with ``poison``, the LDS race-detector build); returns the
    library's path."""
    pdir = os.path.join(BUILD, "poison")
    os.makedirs(pdir, exist_ok=True)
    t0 = time.time()
    jobs = jobs or max(1, (os.cpu_count() or 4))
    units = [(s, tuple(extra), "") for s in SOURCES + MEASURE_SOURCES]
    if poison:
        units += [(s, tuple(extra) + tuple(POISON_FLAGS), pdir) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(*u), units))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + len(MEASURE_SOURCES)], MEASURE_LIB)
    if poison:
        _link(objs[n + len(MEASURE_SOURCES):], POISON_LIB)
    if verbose:
        print(f"[gemmepi] built {LIB}, {os.path.basename(MEASURE_LIB)}"
              f"{' and ' + os.path.basename(POISON_LIB) if poison else ''} "
              f"in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
