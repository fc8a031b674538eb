"""Build libvqkv.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m vector_quantized_bit_amd.build        # or: python vector_quantized_bit_amd/build.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libvqkv.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no kernel relies on NaN semantics (masked scores are -inf); this lets
    # max() fold into DPP forms without quieting its operands
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """libvqkv_hostsan.so: the library with its host code (argument
    validation, split planning, workspace layout, dispatch) built with
    AddressSanitizer and UndefinedBehaviorSanitizer; device code as usual.
    Test infrastructure for the C ABI's host side."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(os.path.dirname(HERE), "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
