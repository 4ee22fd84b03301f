"""Build probe/libet_probe.so, the plain-stream yardstick bench.py times the
library's kernels against (probe/stream_ceiling.hip).  It is not part of the
library: libet.so neither contains nor loads it.

Usage: ``python probe/build.py`` (``__graft_entry__.build()`` runs it too).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_ceiling.hip")
LIB = os.path.join(HERE, "libet_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# The library's device flags: -O3, no fast-math, denormals kept, packed-f32
# instruction selection off.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
