"""Build libsimsd.so (the HIP kernels and the C ABI of include/simsd.h) in-tree.

Every .hip file under csrc/ is compiled for gfx950 with hipcc into one shared
library next to this file.  Packed fp32 instructions are disabled for the
whole library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libsimsd.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)


def hipcc_path() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libsimsd.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))
    tmp = LIB_PATH + ".tmp"
    cmd = [
        hipcc_path(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *extra_flags, *srcs, "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
