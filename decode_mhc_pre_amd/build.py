"""Build libmhc.so in-tree with hipcc for gfx950 (CDNA4)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmhc.so")
SOURCES = [os.path.join(CSRC, "mhc.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, f) for f in ("mhc_device.hpp", "mhc_kernels.hpp", "mhc_persist.hpp")] + \
    [os.path.join(INCLUDE, "mhc.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 VALU forms are switched off for all device code.  The
# persistent pre kernel's 40-step sweep must unroll completely (its register
# queues are indexed by step), which exceeds LLVM's default size limit for
# pragma-requested unrolling.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-pragma-unroll-threshold=1000000",
         "-Wno-pass-failed", "-I" + INCLUDE]


# The benchmark's memory-ceiling probes (bench_ceilings.hip beside bench.py): not
# part of the library, built with the same compiler and flags.
CEIL_SRC = os.path.join(ROOT, "bench_ceilings.hip")
CEIL_LIB = os.path.join(ROOT, "bench_ceilings.so")


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in DEPENDS)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmhc.so")
    os.replace(tmp, LIB)
    return LIB


def build_ceilings(verbose: bool = False) -> str:
    tmp = CEIL_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, CEIL_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building bench_ceilings.so")
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceilings(verbose=True))
