"""Measured peak rates of the GPU (csrc/peaks.hip, built into libgs_peaks.so):
the denominators the roofline fractions are also taken against, besides the
chip's published figures.  Not part of the rasterizer's ABI."""

from __future__ import annotations

import ctypes as C
import os

from . import build as _build

FMA32, FMA64, EXP32, MIX, LDS, COPY, ADD32, MUL32, SEL32, ADD64 = range(10)
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.PEAKS_LIB):
            raise RuntimeError(f"peaks library not built: {_build.PEAKS_LIB}")
        L = C.CDLL(_build.PEAKS_LIB)
        L.gsp_measure.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]
        L.gsp_measure.restype = C.c_double
        L.gsp_scratch_bytes.argtypes = [C.c_int]
        L.gsp_scratch_bytes.restype = C.c_size_t
        _lib = L
    return _lib


def measure(torch, device, copy_gib: float = 1.0) -> dict:
    """Each rate once (after a warm-up run of the same kernel), on the
    current stream.  Rates: lane operations per second (fp32 and fp64 FMA,
    v_exp_f32), rounds of one exp + four fp32 FMAs per second, LDS and copy
    bytes per second."""
    L = lib()
    st = C.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    arith = max(int(L.gsp_scratch_bytes(k)) for k in (FMA32, FMA64, EXP32, MIX, LDS, ADD32, MUL32, SEL32, ADD64))
    buf = torch.empty(arith, dtype=torch.uint8, device=device)
    out = {}
    for name, kind, iters in (("fma32", FMA32, 200), ("fma64", FMA64, 200), ("exp32", EXP32, 60),
                              ("mix", MIX, 100), ("lds", LDS, 200), ("add32", ADD32, 200),
                              ("mul32", MUL32, 200), ("sel32", SEL32, 100), ("add64", ADD64, 200)):
        r = L.gsp_measure(kind, iters, C.c_void_p(buf.data_ptr()), arith, st)
        if r <= 0:
            raise RuntimeError(f"peak measurement {name} failed ({r})")
        out[name] = r
    del buf
    nbytes = int(2 * copy_gib * (1 << 30))
    cbuf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    r = L.gsp_measure(COPY, 4, C.c_void_p(cbuf.data_ptr()), nbytes, st)
    del cbuf
    if r <= 0:
        raise RuntimeError(f"copy measurement failed ({r})")
    out["copy"] = r
    return out


if __name__ == "__main__":
    import json

    import torch
    dev = torch.device("cuda:0")
    r = measure(torch, dev)
    print(json.dumps({"fp32_fma_lane_per_s": r["fma32"], "fp64_fma_lane_per_s": r["fma64"],
                      "exp_f32_lane_per_s": r["exp32"], "exp_plus_4fma_rounds_per_s": r["mix"],
                      "lds_read_bytes_per_s": r["lds"], "copy_bytes_per_s": r["copy"],
                      "add_f32_lane_per_s": r["add32"], "mul_f32_lane_per_s": r["mul32"],
                      "select_f32_lane_per_s": r["sel32"], "add_f64_lane_per_s": r["add64"]}), flush=True)
