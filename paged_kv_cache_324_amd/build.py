"""Build the C-ABI paged-attention libraries for gfx950 with hipcc.

Two libraries come from the same sources:

* ``libpa.so``: the library;
* ``libpa_check.so``: the same entry points compiled with ``PA_CHECK_INDICES``, whose
  kernels record out-of-range block ids, slots and lengths on the device instead of
  skipping them silently (``pa_take_index_errors``).

Every call recompiles all sources in parallel into ``_build/`` and ``_build_check/`` and
links both libraries next to this file (each replaced atomically).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
CHECK_LIB = os.path.join(HERE, "libpa_check.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

# (library, object directory, preprocessor definitions)
VARIANTS = ((LIB, BUILD, ()),
            (CHECK_LIB, os.path.join(HERE, "_build_check"), ("PA_CHECK_INDICES",)))

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpa.so")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def compile_source(src: str, out_dir: str, defines=()) -> str:
    """Compile one source into ``out_dir`` with extra preprocessor definitions; the object."""
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *(f"-D{d}" for d in defines), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def link_library(objs, lib: str) -> str:
    """Link objects into a shared library at ``lib`` (replaced atomically)."""
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build_library(verbose: bool = False) -> str:
    """Build both libraries; returns the path of libpa.so."""
    srcs = sources()
    jobs = [(lib, out_dir, defines, src) for lib, out_dir, defines in VARIANTS for src in srcs]
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: compile_source(j[3], j[1], j[2]), jobs))
    for lib, out_dir, _ in VARIANTS:
        link_library([o for o, j in zip(objs, jobs) if j[0] == lib], lib)
        if verbose:
            print(f"built {lib}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
