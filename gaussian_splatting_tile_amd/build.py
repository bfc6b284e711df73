"""Compile the HIP library (csrc/*.hip) for gfx950 into libgs_hip.so, in tree.

    python -m gaussian_splatting_tile_amd.build

Each source is compiled to an object in parallel, then linked.  Packed-fp32
instruction selection is disabled; the projection source turns off
floating-point contraction itself with a pragma.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgs_hip.so")
SOURCES = ["gs_api.hip", "gs_project.hip", "gs_sort.hip", "gs_render.hip", "gs_mask.hip", "gs_adam.hip"]
# the peak-rate microbenchmarks the roofline fractions are also taken against
# (not part of the rasterizer's ABI)
PEAKS_LIB = os.path.join(PKG, "libgs_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
HEADERS = [os.path.join(CSRC, "gs_internal.h"), os.path.join(CSRC, "gs_adam.h"), os.path.join(INCLUDE, "gs.h")]
ARCH = os.environ.get("GS_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the GPU target feature; everything else is shown
    for line in (r.stderr or "").splitlines():
        if "packed-fp32-ops" in line or "not a recognized feature" in line:
            continue
        if line.strip():
            print(line, file=sys.stderr)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(PEAKS_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print("built", LIB, "and", PEAKS_LIB)
    return LIB


def needs_build() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(PEAKS_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(PEAKS_LIB))
    return any(os.path.getmtime(p) > t
               for p in [os.path.join(CSRC, s) for s in SOURCES + PEAKS_SOURCES] + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
