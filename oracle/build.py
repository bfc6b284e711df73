"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only.  Flags: -O2 -ffp-contract=off and no -march flags,
so every float operation is one IEEE operation (no fused multiply-add); no
fast-math.  OpenMP parallelises the per-Gaussian and per-tile loops.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# GS_ORACLE_LIB names another build of these sources (the planted-mistake
# tests load deliberately broken copies this way); it is never rebuilt here.
LIB_OVERRIDE = os.environ.get("GS_ORACLE_LIB")
LIB = LIB_OVERRIDE or os.path.join(HERE, "liboracle.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wno-unused-function"]
SOURCES = ["gs_oracle.c"]
HEADERS = ["gs_oracle.h", "project_real.h"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc"] + CFLAGS + ["-o", LIB + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def needs_build() -> bool:
    if LIB_OVERRIDE:
        return False
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(os.path.join(HERE, f)) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
