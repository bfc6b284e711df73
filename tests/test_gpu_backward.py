"""GPU backward parity: gs_render_bwd through the C ABI against the oracle's
fp64 reverse pass (same forward decisions), within 1e-3 relative error.

Pixels where the oracle's forward holds a near-threshold decision (alpha near
1/255, T near 1e-4, alpha near the 0.99 cap) get a zero upstream gradient:
there either branch is a correct forward, and the two sides may have taken
different ones.  Gaussians whose colour sits within 1e-5 of the clamp at 0
are left out of the SH and mean comparison for the same reason.
"""

import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_tile_amd import binding as B
from gaussian_splatting_tile_amd import scenes
from tests.gpu_util import run_view, say

pytestmark = pytest.mark.gpu

NAMES = ("means", "log_scales", "quats", "opacity_logits", "sh")


def _upstream(cam, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((3, cam.height, cam.width)) * 0.1).astype(np.float32)


def _oracle_grads(sc, view, G, tile_mask=None, sh=None):
    cam = sc.cameras[view]
    sh = sc.sh_decoded() if sh is None else sh
    op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sh, cam)
    ob = oracle.bin_sort(op, cam)
    oo = oracle.render(op, ob, cam, tile_mask=tile_mask)
    amb = (oo["events"] > 0) | (oo["capflag"] > 0)
    Gz = G.astype(np.float64).copy()
    Gz[:, amb] = 0.0
    if tile_mask is not None:
        tx = (np.arange(cam.width) // 16)[None, :]
        ty = (np.arange(cam.height) // 16)[:, None]
        sel = tile_mask.reshape(-1)[ty * cam.tiles_x + tx].astype(bool)
        Gz[:, ~sel] = 0.0
    g2 = oracle.render_bwd(op, ob, cam, Gz, tile_mask=tile_mask)
    grads = oracle.project_bwd(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sh, cam, op, g2)
    near_clamp = np.abs(op["rgb_raw"]).min(axis=0) < 1e-5
    return grads, Gz.astype(np.float32), near_clamp, int(amb.sum())


def _gpu_grads(sc, views_and_G, sh=None):
    K_sh = (sc.sh_degree + 1) ** 2
    n = sc.n
    grads = dict(means=torch.zeros((3, n), device="cuda"), log_scales=torch.zeros((3, n), device="cuda"),
                 quats=torch.zeros((4, n), device="cuda"), opacity_logits=torch.zeros(n, device="cuda"),
                 sh=torch.zeros((K_sh, 3, n), device="cuda"))
    for view, G in views_and_G:
        buf, K = run_view(sc, view, with_keys=False, sh=sh)
        ws = buf.backward_workspace()
        g, act, gs = buf._keep
        dL = torch.from_numpy(np.ascontiguousarray(G)).cuda()
        buf.backward(gs, dL, grads, ws)
        torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}


def _compare(gpu, ref, near_clamp, name, rel=1e-3, floor=1e-3):
    """Per tensor: relative L2 error <= rel, and elementwise
    |g - r| <= rel * max(|r|, floor * max|r|).  The floor stands for the
    fp32 accumulation error of an element that is a near-cancelling sum of
    per-pixel terms; the worst element at the looser floor 1e-2 is reported
    too."""
    report = {}
    for k in NAMES:
        g, r = gpu[k], ref[k]
        if k in ("sh", "means"):
            keep = ~near_clamp
            g = g[..., keep]
            r = r[..., keep]
        scale = np.abs(r).max(initial=0.0)
        if scale == 0.0:
            assert np.abs(g).max(initial=0.0) == 0.0, (name, k)
            continue
        l2 = np.linalg.norm(g - r) / np.linalg.norm(r)
        err = np.abs(g - r)
        rep = dict(rel_l2=float(l2))
        for f in (floor, 1e-2):
            den = np.maximum(np.abs(r), f * scale)
            rel_e = err / den
            i = int(np.argmax(rel_e))
            rep[f"floor{f:g}"] = dict(worst=float(rel_e.flat[i]), frac_over=float(np.mean(rel_e > rel)),
                                      at=(float(g.flat[i]), float(r.flat[i])), max=float(scale))
        report[k] = rep
    say(f"[gpu] {name}: {report}")
    for k, rep in report.items():
        assert rep["rel_l2"] <= rel, (name, k, rep)
        assert rep[f"floor{floor:g}"]["frac_over"] == 0.0, (name, k, rep)
    return report


def test_backward_tiny_1k_sh0():
    sc = scenes.config(1)
    say("[gpu] backward tiny_1k")
    G = _upstream(sc.cameras[0], 101)
    ref, Gz, nc, amb = _oracle_grads(sc, 0, G)
    gpu = _gpu_grads(sc, [(0, Gz)])
    _compare(gpu, ref, nc, "bwd tiny_1k")


def test_backward_box_100k_sh3():
    sc = scenes.config(2)
    say("[gpu] backward box_100k")
    G = _upstream(sc.cameras[0], 102)
    ref, Gz, nc, amb = _oracle_grads(sc, 0, G)
    gpu = _gpu_grads(sc, [(0, Gz)])
    _compare(gpu, ref, nc, "bwd box_100k")


def test_backward_accumulates_over_views():
    sc = scenes.scene_like(seed=8, n=60_000, width=640, height=360, f=466.7, n_views=2)
    say("[gpu] backward two views accumulate")
    G0 = _upstream(sc.cameras[0], 103)
    G1 = _upstream(sc.cameras[1], 104)
    r0, Gz0, nc0, _ = _oracle_grads(sc, 0, G0)
    r1, Gz1, nc1, _ = _oracle_grads(sc, 1, G1)
    ref = {k: r0[k] + r1[k] for k in NAMES}
    gpu = _gpu_grads(sc, [(0, Gz0), (1, Gz1)])
    _compare(gpu, ref, nc0 | nc1, "bwd 2 views")


def test_backward_scene_5m_1080p_tile_sample():
    """The 5M-Gaussian 1080p workload on a seeded 1/8 sample of tiles
    (upstream gradient zero outside the sample)."""
    sc = scenes.config(4)
    cam = sc.cameras[0]
    say(f"[gpu] backward scene_5m 1080p, tile sample")
    rng = np.random.default_rng(404)
    tile_mask = (rng.random(cam.n_tiles) < 0.125).astype(np.uint8)
    G = sc.upstream(0)
    ref, Gz, nc, amb = _oracle_grads(sc, 0, G, tile_mask=tile_mask)
    gpu = _gpu_grads(sc, [(0, Gz)])
    _compare(gpu, ref, nc, "bwd scene_5m sample")


def test_batched_backward_matches_per_view_calls():
    """gs_render_bwd_screen_views over the views + one gs_project_bwd gives
    the per-view gs_render_bwd sum (up to the order of fp32 additions), and
    the oracle's gradients; the batched screen pass equals the single-view
    one bit for bit."""
    sc = scenes.scene_like(seed=9, n=40_000, width=480, height=272, f=350.0, n_views=3)
    say("[gpu] batched projection backward, 3 views")
    Gs = [_upstream(sc.cameras[v], 200 + v) for v in range(3)]
    refs = [_oracle_grads(sc, v, Gs[v]) for v in range(3)]
    ref = {k: sum(r[0][k] for r in refs) for k in NAMES}
    nc = refs[0][2] | refs[1][2] | refs[2][2]
    per_view = _gpu_grads(sc, [(v, refs[v][1]) for v in range(3)])
    n = sc.n
    grads = dict(means=torch.zeros((3, n), device="cuda"), log_scales=torch.zeros((3, n), device="cuda"),
                 quats=torch.zeros((4, n), device="cuda"), opacity_logits=torch.zeros(n, device="cuda"),
                 sh=torch.zeros((16, 3, n), device="cuda"))
    bufs, g2s, wss, dLs = [], [], [], []
    for v in range(3):
        buf, K = run_view(sc, v, with_keys=False)
        wss.append(torch.empty(B.render_bwd_screen_workspace_bytes(buf.k_capacity), dtype=torch.uint8,
                               device="cuda"))
        g2s.append(torch.full((n, 9), float("nan"), device="cuda"))
        dLs.append(torch.from_numpy(np.ascontiguousarray(refs[v][1])).cuda())
        bufs.append(buf)
    # one view through gs_render_bwd_screen, the three through the batched call
    g2_single = torch.full((n, 9), float("nan"), device="cuda")
    bufs[1].backward_screen(dLs[1], g2_single, wss[1])
    torch.cuda.synchronize()
    B.render_bwd_screen_views(bufs, dLs, g2s, wss)
    torch.cuda.synchronize()
    for b, g in zip(bufs, g2s):
        visible = b.splats[:, 3].view(torch.int32) != 0
        assert bool(torch.isfinite(g[visible]).all())             # visible Gaussians' rows written
        assert bool(torch.isnan(g[~visible]).all())               # culled ones' rows untouched
    vis1 = bufs[1].splats[:, 3].view(torch.int32) != 0
    assert torch.equal(g2_single[vis1], g2s[1][vis1])
    for b in bufs:
        assert torch.all(b.schedule[b.ranges.shape[0]:] == 0)
    gs = bufs[0]._keep[2]
    B.project_bwd(gs, [b.camc for b in bufs], [b.splats for b in bufs], g2s, grads)
    torch.cuda.synchronize()
    batched = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    for k in NAMES:
        scale = np.abs(per_view[k]).max()
        assert np.abs(batched[k] - per_view[k]).max() <= 1e-5 * scale, k
    _compare(batched, ref, nc, "bwd batched 3 views")


def test_batched_backward_large_views_equals_per_view_calls():
    """Views of 2880x2048 (23040 tiles, more than 4 per resident wave of the
    blend backward), where the batched launch runs the views one after
    another instead of interleaving their tiles: every view's per-Gaussian
    sums equal its single-view call's bit for bit."""
    sc = scenes.scene_like(seed=19, n=20_000, width=2880, height=2048, f=2000.0, n_views=3)
    say("[gpu] batched blend backward, 3 views of 2880x2048")
    n = sc.n
    bufs, g2s, wss, dLs, singles = [], [], [], [], []
    for v in range(3):
        buf, K = run_view(sc, v, with_keys=False)
        ws = torch.empty(B.render_bwd_screen_workspace_bytes(buf.k_capacity), dtype=torch.uint8, device="cuda")
        dL = torch.from_numpy(np.ascontiguousarray(_upstream(sc.cameras[v], 300 + v).astype(np.float32))).cuda()
        g1 = torch.full((n, 9), float("nan"), device="cuda")
        buf.backward_screen(dL, g1, ws)
        torch.cuda.synchronize()
        bufs.append(buf)
        wss.append(ws)
        dLs.append(dL)
        singles.append(g1)
        g2s.append(torch.full((n, 9), float("nan"), device="cuda"))
    B.render_bwd_screen_views(bufs, dLs, g2s, wss)
    torch.cuda.synchronize()
    for b, g, g1 in zip(bufs, g2s, singles):
        visible = b.splats[:, 3].view(torch.int32) != 0
        assert int(visible.sum()) > 0
        assert torch.equal(g[visible], g1[visible])
        assert bool(torch.isnan(g[~visible]).all())
        assert torch.all(b.schedule[b.ranges.shape[0]:] == 0)
