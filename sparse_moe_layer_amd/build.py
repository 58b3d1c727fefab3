"""Build libmoe.so (all HIP sources of csrc/) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off (hipcc still vectorises plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


PEAKS_LIB = os.path.join(HERE, "peaks", "libmoe_peaks.so")


def _hipcc(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd), tmp


def build(verbose: bool = False) -> str:
    """libmoe.so (the layer, csrc/*.hip) and libmoe_peaks.so (the benchmark's peak-rate
    probes, peaks/*.hip), compiled side by side."""
    jobs = [(_hipcc(sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip"))), LIB, verbose), LIB),
            (_hipcc(sorted(glob.glob(os.path.join(HERE, "peaks", "*.hip"))), PEAKS_LIB, verbose),
             PEAKS_LIB)]
    for (proc, tmp), out in jobs:
        if proc.wait() != 0:
            raise subprocess.CalledProcessError(proc.returncode, "hipcc " + out)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
