"""Builds libmoel.so (HIP kernels + C ABI) for gfx950, in-tree next to this file.

    python -m moe_layer_persistent_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoel.so")
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    val_obj = os.path.join(objdir, "moel_validate.o")
    # host-only validation: plain C++
    cmd_val = ["g++", "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-c",
               os.path.join(CSRC, "moel_validate.cpp"), "-o", val_obj]
    ker_obj = os.path.join(objdir, "moel_kernels.o")
    cmd_ker = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # a single-lane atomic keeps its result where it is used instead of being
               # broadcast to the wave right away (which would wait for every load in flight)
               "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
               "-Wno-unused-result", "-Wno-unused-value", "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, "moel_kernels.hip"), "-o", ker_obj]
    cmd_link = [HIPCC, "-shared", "-fPIC", ker_obj, val_obj, "-o", LIB + ".tmp"]
    for c in (cmd_val, cmd_ker, cmd_link):
        if verbose:
            print(" ".join(c), flush=True)
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("build failed: " + " ".join(c))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
