"""Builds libsana_linattn.so (gfx950) in-tree with hipcc.

    python relu_linear_attention_attn_amd/csrc/build.py [--asm]

The library lands next to the Python binding, in the package directory.
``--asm`` also writes the gfx950 assembly of the kernels to ``_build/`` for
inspection.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsana_linattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"
SOURCES = ["api.cpp", "linattn_kernels.hip", "qkv_kernels.hip", "noalloc.hip"]

# Packed fp32 VALU ops are disabled for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, asm: bool = False) -> str:
    """Compile every source for gfx950 into LIB_PATH; returns the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I", INCLUDE, "-I", HERE, *DEVICE_FLAGS,
           *[os.path.join(HERE, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    os.replace(tmp, LIB_PATH)
    if asm:
        out = os.path.join(ROOT, "_build")
        os.makedirs(out, exist_ok=True)
        subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
                        "--cuda-device-only", "-S", "-I", INCLUDE, "-I", HERE, *DEVICE_FLAGS,
                        os.path.join(HERE, "linattn_kernels.hip"),
                        "-o", os.path.join(out, "linattn_kernels.s")], check=True,
                       capture_output=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
