"""Builds libraggedshard.so (HIP for gfx950 + host C++) in-tree with hipcc.

    python -m sharded_state_raggedshard_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libraggedshard.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["plan.cpp", "abi.cpp", "copy_kernels.hip", "adam8_kernels.hip", "fp8_kernels.hip",
           "muon.cpp", "muon_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # binary32 semantics the step relies on: no FMA contraction, correctly
    # rounded '/' and sqrt
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 arithmetic stays off (v_pk_* fp32 forms)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines()
            if "warning" in l and "packed-fp32-ops" not in l and "feature" not in l]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
