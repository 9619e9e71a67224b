"""Build libmoc.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python sparse_chunk_routed_amd/build.py [--jobs N] [--verbose]

MOC_BUILD_DEFINES (extra -D flags) and MOC_BUILD_OUT (another output path for libmoc) build a
variant of the library from the same sources next to the in-tree one, to compare kernels on one
GPU (MOC_LIB_PATH then selects it at load time).

Run as a script (or loaded by file path): importing the package would load the library that
this rebuilds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoc.so")
# benchmark helper (register-only MFMA loops), a library of its own that only bench.py loads
PROBE_LIB = os.path.join(PKG, "libmoc_bench_probe.so")
PROBE_SOURCE = "probe.hip"
ARCH = "gfx950"

SOURCES = ["moc_api.hip", "pool.hip", "route.hip", "outer.hip", "varlen.hip", "attn_fwd.hip",
           "mx.hip", "attn_bwd.hip", "layout_check.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of every kernel (the compiler would otherwise pair
    # scalar fp32 math into them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoc)")


EXTRA_DEFINES = [d for d in os.environ.get("MOC_BUILD_DEFINES", "").split() if d]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + EXTRA_DEFINES + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                     os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link libmoc.so (and the benchmark's probe library). Always
    recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [PROBE_SOURCE]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    out = os.environ.get("MOC_BUILD_OUT") or LIB
    _link(objs[:-1], out)
    if out == LIB:
        _link(objs[-1:], PROBE_LIB)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
