"""Build the HIP library libmoe_layout.so for gfx950 in the package folder.

    python -m combine_moe_layout_06_amd.build

Each .hip file is compiled with hipcc for gfx950 only, then linked into one
shared library. Flags:
  -O3 -std=c++17 -fPIC         optimised, position independent
  -ffp-contract=off            no implicit fused multiply-adds (FMAs are
                               written out where the method wants them)
  -fhip-fp32-correctly-rounded-divide-sqrt
                               IEEE fp32 division (FP8 scales use it)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               keep the compiler from emitting packed fp32
                               arithmetic
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
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_layout.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["moe_api.hip", "route.hip", "layout.hip", "dispatch.hip", "combine.hip",
           "hierarchical.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r.stderr


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for log in ex.map(_run, jobs):
            if verbose and log:
                sys.stderr.write(log)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ABI_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "moe_abi_check.cpp")
ABI_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "moe_abi_check")


def build_abi_check() -> str:
    """Compile the stand-alone host program that checks the C ABI through
    include/moe.h alone; it finds the library through its run path."""
    _run([hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
          "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include"),
          ABI_CHECK_SRC, "-L" + PKG, "-lmoe_layout",
          "-Wl,-rpath,$ORIGIN/../../combine_moe_layout_06_amd", "-o", ABI_CHECK_BIN])
    return ABI_CHECK_BIN


CEIL_SRC = os.path.join(CSRC, "ceilings.hip")
CEIL_LIB = os.path.join(PKG, "libmoe_ceilings.so")


def build_ceilings() -> str:
    """Compile the benchmark's access-pattern ceiling kernels (plain copy,
    read, write, row gather and row scatter) into their own library; the
    path never calls them."""
    tmp = CEIL_LIB + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, "-shared", CEIL_SRC, "-o", tmp])
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB


SWEEP_SRC = os.path.join(ROOT, "tests", "hip", "convert_sweep.hip")
SWEEP_LIB = os.path.join(ROOT, "tests", "hip", "libconvert_sweep.so")


def build_convert_sweep() -> str:
    """Compile the test library that compares the hardware converts used by
    the kernels (their device functions, included from csrc/) with integer
    rounding references on every fp32 pattern."""
    tmp = SWEEP_LIB + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, "-I" + CSRC, "-shared", SWEEP_SRC, "-o", tmp])
    os.replace(tmp, SWEEP_LIB)
    return SWEEP_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_abi_check())
    print(build_convert_sweep())
    print(build_ceilings())
