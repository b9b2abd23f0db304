"""Build libigc.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libigc.so")
SOURCES = [os.path.join(CSRC, "igc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Every fp32 multiply and add in the epilogues is its own rounded
    # operation: the requantize step is defined with two roundings.
    "-ffp-contract=off",
    # No packed-fp32 instructions anywhere.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into libigc.so next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def assembly(out_dir: str, extra_flags=()) -> str:
    """Write the gfx950 assembly of the kernels to out_dir; returns the .s path."""
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "igc.o")
    cmd = [HIPCC, *[f for f in HIP_FLAGS if f != "-shared"], *extra_flags, "-c", "--save-temps",
           SOURCES[0], "-o", obj]
    subprocess.check_call(cmd, cwd=out_dir, stderr=subprocess.DEVNULL)
    for name in os.listdir(out_dir):
        if name.endswith("gfx950.s"):
            return os.path.join(out_dir, name)
    raise FileNotFoundError("no gfx950 assembly produced")


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
