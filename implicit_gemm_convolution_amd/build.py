"""Build libigc.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

The C ABI (csrc/igc.hip) and the kernel instantiations (csrc/igc_launch.hip,
compiled once per kernel kind with -DIGC_LAUNCH_UNIT=<n>) are separate
objects compiled in parallel, then linked into one shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libigc.so")
ABI_SOURCE = os.path.join(CSRC, "igc.hip")
LAUNCH_SOURCE = os.path.join(CSRC, "igc_launch.hip")
LAUNCH_UNITS = 38  # the (kind, variant) pairs of IGC_LAUNCH_KINDS in igc_host.hpp
SOURCES = [ABI_SOURCE, LAUNCH_SOURCE]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Every fp32 multiply and add in the epilogues is its own rounded
    # operation: the requantize step is defined with two roundings.
    "-ffp-contract=off",
    # No packed-fp32 instructions anywhere.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _units():
    """(source, extra defines, object name) of every object of the library."""
    yield ABI_SOURCE, [], "igc.o"
    for n in range(LAUNCH_UNITS):
        yield LAUNCH_SOURCE, [f"-DIGC_LAUNCH_UNIT={n}"], f"igc_launch_{n}.o"


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16, LAUNCH_UNITS + 1))


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source and link libigc.so next to this file; returns its path."""
    tmpdir = tempfile.mkdtemp(prefix="igc_build_")
    try:
        cmds = []
        for src, defs, obj in _units():
            cmds.append([HIPCC, *HIP_FLAGS, *extra_flags, *defs, "-c", src, "-o", os.path.join(tmpdir, obj)])

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)

        with ThreadPoolExecutor(_jobs()) as ex:
            list(ex.map(run, cmds))
        tmp = LIB_PATH + ".tmp"
        objs = [os.path.join(tmpdir, obj) for _, _, obj in _units()]
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        run(link)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


def assembly(out_dir: str, extra_flags=()) -> str:
    """Write the gfx950 assembly of every kernel to out_dir (one file); returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIP_FLAGS]

    def one(n):
        d = os.path.join(out_dir, f"unit{n}")
        os.makedirs(d, exist_ok=True)
        cmd = [HIPCC, *flags, *extra_flags, f"-DIGC_LAUNCH_UNIT={n}", "-c", "--save-temps",
               LAUNCH_SOURCE, "-o", os.path.join(d, "u.o")]
        subprocess.check_call(cmd, cwd=d, stderr=subprocess.DEVNULL)
        for name in os.listdir(d):
            if name.endswith("gfx950.s"):
                return os.path.join(d, name)
        raise FileNotFoundError("no gfx950 assembly produced")

    with ThreadPoolExecutor(_jobs()) as ex:
        parts = list(ex.map(one, range(LAUNCH_UNITS)))
    out = os.path.join(out_dir, "igc-kernels-gfx950.s")
    with open(out, "w") as f:
        for part in parts:
            with open(part) as g:
                f.write(g.read())
            f.write("\n")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
