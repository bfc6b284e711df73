"""Helpers shared by the GPU parity tests: upload a scene, run one view through
the C ABI, compare with the oracle under the near-threshold protocol."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gaussian_splatting_tile_amd import binding as B


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_gaussians(sc, sh=None, device="cuda"):
    """Scene parameters as contiguous device tensors (SH stays in its storage
    dtype; sh may be an 8-bit (codes, bounds) pair)."""
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if sh is None:
        sh = sc.sh_fp16 if sc.sh_fp16 is not None else sc.sh
    g = dict(means=f(sc.means), scales=f(sc.scales), quats=f(sc.quats), opacities=f(sc.opacities))
    if isinstance(sh, tuple):
        g["sh"], g["sh_bounds"] = f(sh[0]), f(sh[1])
    else:
        g["sh"] = f(sh)
    if getattr(sc, "velocity", None) is not None:
        g["velocity"], g["t_offset"] = f(sc.velocity), f(sc.t_offset)
    return g


def splats_np(buf: B.ViewBuffers):
    s = buf.splats[: buf.n].cpu().numpy() if buf.n > 0 else np.zeros((0, 12), np.float32)
    return dict(u=s[:, 0], v=s[:, 1], z=s[:, 2], radius=s[:, 3].view(np.int32),
                conic=s[:, 4:7].T, opacity=s[:, 7], rgb=s[:, 8:11].T, tiles=s[:, 11].view(np.uint32))


def run_view(sc, view=0, k_capacity=None, with_keys=True, bg=(0.0, 0.0, 0.0), active=None, sh=None):
    """Project, bin and render one view on the GPU; returns (buffers, K)."""
    cam = sc.cameras[view]
    g = device_gaussians(sc, sh=sh)
    act = None if active is None else torch.from_numpy(np.ascontiguousarray(active, np.uint8)).cuda()
    gs = B.gaussians_struct(g, sc.sh_degree, act)
    if k_capacity is None:
        # first pass with a generous bound, then the exact K
        probe = B.ViewBuffers(sc.n, cam, max(16 * sc.n, 1024), with_keys=False)
        probe.forward(gs, bg)
        torch.cuda.synchronize()
        k_capacity = int(probe.k_total.item())
        del probe
    buf = B.ViewBuffers(sc.n, cam, k_capacity, with_keys=with_keys)
    buf.forward(gs, bg)
    torch.cuda.synchronize()
    buf._keep = (g, act, gs)
    return buf, int(buf.k_total.item())


def compare_records(gpu, orc, name=""):
    """u, v, depth, radius, tiles, conic bit-exact; colour within 4e-6."""
    vis = orc["radius"] > 0
    assert np.array_equal(gpu["radius"], orc["radius"]), f"{name}: radius differs"
    assert np.array_equal(gpu["tiles"].astype(np.int64), orc["tiles"].astype(np.int64)), f"{name}: tiles"
    for k in ("u", "v", "z"):
        a = gpu[k][vis].astype(np.float32)
        b = orc[k][vis].astype(np.float32)
        bad = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0]
        assert bad.size == 0, f"{name}: {k} differs at {bad[:5]}: {a[bad[:5]]} vs {b[bad[:5]]}"
    ca = gpu["conic"][:, vis].astype(np.float32)
    cb = orc["conic"][:, vis].astype(np.float32)
    assert np.array_equal(ca.view(np.uint32), cb.view(np.uint32)), f"{name}: conic differs"
    assert np.array_equal(gpu["opacity"][vis], orc["opacity"][vis].astype(np.float32))
    err = np.abs(gpu["rgb"][:, vis].astype(np.float64) - orc["rgb"][:, vis]).max(initial=0.0)
    assert err <= 4e-6, f"{name}: rgb error {err}"
    # culled records are all zero
    assert np.all(gpu["u"][~vis] == 0) and np.all(gpu["conic"][:, ~vis] == 0)


def compare_bins(buf, K, ob, name=""):
    assert K == ob["K"], f"{name}: K {K} vs {ob['K']}"
    vals = buf.vals[:K].cpu().numpy().view(np.uint32)
    ranges = buf.ranges.cpu().numpy().view(np.uint32)
    assert np.array_equal(vals, ob["vals"]), f"{name}: vals differ"
    assert np.array_equal(ranges, ob["ranges"]), f"{name}: ranges differ"
    if buf.keys is not None:
        keys = buf.keys[:K].cpu().numpy().view(np.uint64)
        assert np.array_equal(keys, ob["keys"]), f"{name}: keys differ"


def _flip_sets(k: int):
    """Branch combinations to try for a pixel with k near-threshold events:
    all of them when k <= 6, otherwise every single and double reversal among
    the first 32 (the render_pixel mask is 32 bits wide)."""
    if k <= 0:
        return []
    if k <= 6:
        return list(range(1, 1 << k))
    m = min(k, 32)
    out = [1 << a for a in range(m)]
    out += [(1 << a) | (1 << b) for a in range(m) for b in range(a + 1, m)]
    return out


def compare_image(buf, cam, oproj, obins, oout, tile_mask=None, bg=(0.0, 0.0, 0.0), tol=1e-4):
    """Max |diff| per channel <= tol, final_T within tol, n_contrib equal; a
    pixel that fails is accepted only if the oracle flagged near-threshold
    decisions and one of their alternative branches matches.  Returns stats."""
    img = buf.image.cpu().numpy().astype(np.float64)
    T = buf.final_T.cpu().numpy().astype(np.float64)
    nc = buf.n_contrib.cpu().numpy()
    H, W = cam.height, cam.width
    sel = np.ones((H, W), bool)
    if tile_mask is not None:
        tx = (np.arange(W) // 16)[None, :]
        ty = (np.arange(H) // 16)[:, None]
        sel = tile_mask.reshape(-1)[ty * cam.tiles_x + tx].astype(bool)
    d_img = np.abs(img - oout["image"]).max(axis=0)
    d_T = np.abs(T - oout["final_T"])
    bad = sel & ((d_img > tol) | (d_T > tol) | (nc != oout["n_contrib"]))
    ys, xs = np.nonzero(bad)
    resolved = unresolved = 0
    details = []
    for y, x in zip(ys, xs):
        k = int(oout["events"][y, x])
        ok = False
        for flips in _flip_sets(k):
            rgb, tt, nn, _ = oracle.render_pixel(oproj, obins, cam, int(x), int(y), flips=flips, bg=bg)
            if (np.abs(rgb - img[:, y, x]).max() <= tol and abs(tt - T[y, x]) <= tol and nn == nc[y, x]):
                ok = True
                break
        if ok:
            resolved += 1
        else:
            unresolved += 1
            if len(details) < 5:
                details.append((int(x), int(y), k, img[:, y, x], oout["image"][:, y, x], T[y, x],
                                oout["final_T"][y, x], int(nc[y, x]), int(oout["n_contrib"][y, x])))
    maxerr = float(np.where(sel & ~bad, d_img, 0).max(initial=0.0))
    return dict(pixels=int(sel.sum()), mismatched=int(bad.sum()), resolved=resolved,
                unresolved=unresolved, details=details, max_err_clean=maxerr,
                flagged=int((sel & (oout["events"] > 0)).sum()))
