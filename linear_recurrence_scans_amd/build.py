"""Build libmiscan.so (the HIP kernels + C ABI) for gfx950, in-tree.

Each .hip source compiles to an object in parallel; the objects link into
``linear_recurrence_scans_amd/libmiscan.so``.  No fast-math: arithmetic stays
IEEE fp32.  Packed-fp32 instructions are disabled on the device side.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmiscan.so")
SOURCES = ["api.hip", "linear_scan.hip", "log_scan.hip", "affine_scan.hip"]
# The benchmark's probe kernels (streaming ceiling, cache flush): a library of
# their own, not part of libmiscan.so.
BENCH_LIB = os.path.join(PKG, "libmiscan_bench.so")
BENCH_SOURCES = ["bench_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wshadow", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag: drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, out: str = LIB, defines=(), build_dir: str = BUILD, bench: bool = True) -> str:
    """Compile and link libmiscan.so (and, with `bench`, libmiscan_bench.so).
    `defines` (NAME=VALUE) override the compile-time tile shapes; `out` and
    `build_dir` keep such variants apart from the default."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + (BENCH_SOURCES if bench else [])
    workers = min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), srcs))
    _link(objs[:len(SOURCES)], out)
    if verbose:
        print("built", out)
    if bench:
        _link(objs[len(SOURCES):], BENCH_LIB)
        if verbose:
            print("built", BENCH_LIB)
    return out


if __name__ == "__main__":
    build(verbose=True)
