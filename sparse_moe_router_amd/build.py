"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m sparse_moe_router_amd.build

Every source is compiled each time (objects under ``_build/``), then linked
into ``sparse_moe_router_amd/libmoe.so`` and, with the entry points' range
checks compiled in, ``sparse_moe_router_amd/libmoe_debug.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
OUT_DEBUG = os.path.join(PKG, "libmoe_debug.so")
DEBUG_SOURCES = ("moe_abi.cpp", "checks.hip")  # the only sources that MOE_RANGE_CHECKS changes
BUILD = os.path.join(PKG, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return p


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".debug.o" if debug else ".o"))
    cmd = [hipcc(), *FLAGS, *(["-DMOE_RANGE_CHECKS"] if debug else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Both libraries: the release one and the debug one, whose entry points
    range-check caller-provided routing arrays (the sources that differ are
    compiled twice, with MOE_RANGE_CHECKS; the kernels' objects are shared)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = [(src, False) for src in srcs] + [(src, True) for src in srcs if os.path.basename(src) in DEBUG_SOURCES]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    rel = objs[:len(srcs)]
    dbg_by_src = {os.path.basename(j[0]): o for j, o in zip(jobs[len(srcs):], objs[len(srcs):])}
    dbg = [dbg_by_src.get(os.path.basename(src), o) for src, o in zip(srcs, rel)]
    _link(rel, OUT)
    _link(dbg, OUT_DEBUG)
    if verbose:
        print(f"built {OUT} and {OUT_DEBUG}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
