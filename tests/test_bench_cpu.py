"""Host logic of bench.py, on the CPU: the one-GPU guard, the pair counters
behind the blend kernels' rooflines (checked on the oracle's outputs against
brute-force counts), and the tie between the reported traffic and the
kernel sources the counters were taken on."""

import hashlib
import os
import subprocess
import sys
import types

import numpy as np
import torch

import bench
import oracle
from gaussian_splatting_tile_amd import scenes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _view_from_oracle(sc, view=0):
    cam = sc.cameras[view]
    op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sc.sh_decoded(), cam)
    ob = oracle.bin_sort(op, cam)
    oo = oracle.render(op, ob, cam)
    n = sc.n
    sp = np.zeros((n, 12), np.float32)
    sp[:, 0], sp[:, 1], sp[:, 2] = op["u"], op["v"], op["z"]
    sp[:, 4:7] = op["conic"].T
    sp[:, 7] = op["opacity"]
    b = types.SimpleNamespace(
        cam=cam, ranges=torch.from_numpy(ob["ranges"].astype(np.int64).reshape(-1, 2)),
        final_T=torch.from_numpy(oo["final_T"].astype(np.float32)),
        n_contrib=torch.from_numpy(oo["n_contrib"].astype(np.int64)),
        splats=torch.from_numpy(sp), vals=torch.from_numpy(ob["vals"].astype(np.int64)))
    return b, op, ob, oo


def test_blend_pair_counts_against_brute_force():
    sc = scenes.tiny(seed=6, n=600)
    b, op, ob, oo = _view_from_oracle(sc)
    cnt = bench.blend_pairs(torch, b)
    p_eval, p_need, p_tile = cnt["eval"], cnt["needed"], cnt["tile"]
    cam = sc.cameras[0]
    TX = cam.tiles_x
    ranges = ob["ranges"].reshape(-1, 2).astype(np.int64)
    vals = ob["vals"].astype(np.int64)
    brute_eval = brute_need = brute_comp = brute_bwd = 0
    a, bb, c = (op["conic"][i].astype(np.float64) for i in range(3))
    for y in range(cam.height):
        for x in range(cam.width):
            t = (y // 16) * TX + x // 16
            s, e = ranges[t]
            m = int(oo["n_contrib"][y, x]) if oo["final_T"][y, x] < 1e-4 else e - s
            brute_eval += m
            # composited: alpha >= 1/255 among the entries before n_contrib
            nci = int(oo["n_contrib"][y, x])
            brute_bwd += nci
            for g in vals[s:s + nci]:
                dxp, dyp = op["u"][g] - (x + 0.5), op["v"][g] - (y + 0.5)
                pw = -0.5 * (a[g] * dxp * dxp + c[g] * dyp * dyp) - bb[g] * dxp * dyp
                brute_comp += op["opacity"][g] * np.exp(pw) >= 1.0 / 255.0
            # the pixel's strip: rows 4r .. 4r + 3 of its tile, all 16 columns,
            # the quadratic form at every pixel centre of it
            y0 = (y // 16) * 16 + ((y % 16) // 4) * 4
            xs = (x // 16) * 16 + np.arange(16) + 0.5
            ys = y0 + np.arange(4) + 0.5
            for g in vals[s:s + m]:
                dx = xs[None, :] - op["u"][g]
                dy = ys[:, None] - op["v"][g]
                qmin = (a[g] * dx * dx + 2 * bb[g] * dx * dy + c[g] * dy * dy).min()
                if op["opacity"][g] * np.exp(-0.5 * qmin) >= 1.0 / 255.0:
                    brute_need += 1
    assert p_eval == brute_eval
    # the counter's strip test is over the box spanned by the pixel centres
    # (with a 1e-3 margin), so it keeps every entry some centre can use
    assert brute_need <= p_need <= p_tile <= p_eval
    assert p_need <= 1.05 * brute_need + 50
    assert p_need > 0
    assert cnt["bwd_examined"] == brute_bwd
    assert abs(cnt["composited"] - brute_comp) <= 2 and brute_comp > 1000
    assert cnt["composited"] <= cnt["bwd_examined"] <= p_eval


def test_traffic_figure_follows_the_kernel_sources(tmp_path, monkeypatch):
    h = hashlib.sha256()
    for f in bench.TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    good = tmp_path / "good.md"
    good.write_text(f"# x\n\ntraffic_bytes_per_launch: 12345\nsource_sha256 (sources): {h.hexdigest()}\n")
    stale = tmp_path / "stale.md"
    stale.write_text("traffic_bytes_per_launch: 12345\nsource_sha256 (sources): " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(good))
    assert bench.measured_traffic() == 12345
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
