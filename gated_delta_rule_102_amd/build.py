"""Build libkda.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m gated_delta_rule_102_amd.build``.  The library lands next to
this file; object files go to ``_build/``.  Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
SOURCES = ["kda_prefill.hip", "kda_fused.hip", "kda_prefill_fp32.hip", "kda_decode.hip",
           "kda_backward.hip", "kda_context.hip", "kda_noalloc.hip"]
HOST_SOURCES = ["kda_api.cpp"]


def _compile(src: str, host_only: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if host_only:
        cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
               "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-Wall", "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in HOST_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
