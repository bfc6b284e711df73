"""Write tests/golden/*.json from the CPU oracle alone.

The pages print no worked numeric example for any stage of the rasterizer,
so the stored values here are the oracle's own, frozen: a regression pin
that makes any later change to the oracle's arithmetic visible.  Run
    python tests/golden/make_golden.py
and commit the result together with the change that justifies it.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gaussian_splatting_tile_amd import scenes  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_forward_record():
    sc = scenes.config(1)
    proj, bins, out = oracle.forward(sc)
    u32 = lambda k: proj[k].astype(np.float32)
    return {
        "workload": "1000 Gaussians, SH degree 0, 128x128, seed 1",
        "K": int(bins["K"]),
        "P_eval": int(out["p_eval"]),
        "visible": int((proj["radius"] > 0).sum()),
        "sha256_keys": digest(bins["keys"]),
        "sha256_vals": digest(bins["vals"]),
        "sha256_ranges": digest(bins["ranges"]),
        "sha256_uvz_f32": digest(np.stack([u32("u"), u32("v"), u32("z")])),
        "sha256_conic_f32": digest(proj["conic"].astype(np.float32)),
        "sha256_radius": digest(proj["radius"]),
        "image_sum": float(out["image"].sum()),
        "final_T_sum": float(out["final_T"].sum()),
        "n_contrib_sum": int(out["n_contrib"].sum()),
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_1k_forward.json")
    with open(path, "w") as f:
        json.dump(tiny_forward_record(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)
