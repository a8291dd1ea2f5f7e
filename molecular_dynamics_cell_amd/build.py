"""Build libmpnn.so (the C-ABI library of include/mpnn.h) for gfx950 with hipcc.

Each HIP translation unit is compiled separately (in parallel) and linked into one shared
library next to this file.  Packed-FP32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmpnn.so")
SOURCES = ["api.hip", "scan.hip", "neighbors.hip", "edges.hip", "mlp.hip", "integrate.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fno-gpu-rdc",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        # hipcc's host pass reports the device-only feature flag; keep the rest visible
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if any(ln.strip() for ln in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # a stand-alone C++ user of the C ABI (no Python), linked against the library
    drv = os.path.join(HERE, "abi_driver")
    cmd = [HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950", "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "abi_driver.cpp"), "-L" + HERE, "-lmpnn", "-Wl,-rpath,$ORIGIN", "-o", drv + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_driver build failed:\n{r.stderr}")
    os.replace(drv + ".tmp", drv)
    if verbose:
        print("built", LIB, "and", drv)
    return LIB


if __name__ == "__main__":
    build()
