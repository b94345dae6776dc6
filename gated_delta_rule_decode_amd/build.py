"""Ahead-of-time build of libkda_mi355x.so for gfx950 (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda_mi355x.so")
SOURCES = [os.path.join(PKG, "csrc", "kda_kernels.hip"), os.path.join(PKG, "csrc", "kda_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "kda.h"), os.path.join(PKG, "csrc", "kda_internal.h")]

# Packed fp32 VALU ops are disabled for the device code (only plain fp32
# VALU instructions are emitted); the host pass prints a harmless warning.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Wall", *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libkda_mi355x.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
