"""Builds libpi.so (the HIP kernels and the C ABI of include/pi.h) for gfx950.

Run as `python -m sparse_activation_ffn_amd.build`; hipcc cross-compiles, no
GPU is needed.  The library is written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpi.so")
SOURCES = [os.path.join(CSRC, "pi_api.hip")]
# host-core code of the hybrid step: built by the host compiler, linked in
HOST_SOURCES = [os.path.join(CSRC, "pi_host.cpp")]
DEPS = SOURCES + HOST_SOURCES + \
    [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")] + \
    [os.path.join(INCLUDE, "pi.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
# AVX2 / F16C / FMA code is selected per function at run time, so the baseline ISA stays generic
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: only plain fp32 VALU ops are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libpi.so.  With force=False an up-to-date library is kept."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in DEPS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp"
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(PKG, os.path.basename(src) + ".tmp.o")
        cmd = [CXX, *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-x", "none", *objs, "-pthread", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose="-v" in sys.argv))
