"""Build the HIP C-ABI library ``libmoe_route.so`` in-tree for gfx950.

    python expert_grouping_dispatch_amd/build_lib.py

Compiles every ``csrc/*.hip`` with hipcc (device code for gfx950 only) and
links them into ``expert_grouping_dispatch_amd/libmoe_route.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_route.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # combine is defined with separately rounded products and sums
    "-ffp-contract=off",
    # MXFP4 scaling reads bf16 subnormals as fp32 subnormals
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "route_smoke.c")
C_EXAMPLE_BIN = os.path.join(ROOT, "tests", "c_abi", "route_smoke.bin")


def build_c_example(verbose: bool = True) -> str:
    """A plain-C program (no torch) linked against the library: it shows the
    C ABI is usable on its own; a GPU test runs it."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(rocm, "include"),
           C_EXAMPLE_SRC, "-o", C_EXAMPLE_BIN, "-L", PKG, "-lmoe_route",
           "-Wl,-rpath,$ORIGIN/../../expert_grouping_dispatch_amd",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C example build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_EXAMPLE_BIN}", flush=True)
    return C_EXAMPLE_BIN


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", flush=True)
    build_c_example(verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
