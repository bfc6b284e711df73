"""Python marshalling for the CPU oracle (oracle/gs_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.  Every function
here only converts numpy arrays and calls the C oracle; the arithmetic lives
in gs_oracle.c and project_real.h.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import numpy as np

from . import build as _build

_lib = None


class OrcCam(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32),
                ("fx", C.c_double), ("fy", C.c_double), ("cx", C.c_double), ("cy", C.c_double),
                ("viewmat", C.c_double * 12), ("znear", C.c_double), ("guard", C.c_double),
                ("lod_px", C.c_double)]


class OrcProjOut(C.Structure):
    _fields_ = [("u", C.c_void_p), ("v", C.c_void_p), ("z", C.c_void_p), ("radius", C.c_void_p),
                ("rect", C.c_void_p), ("conic", C.c_void_p), ("opacity", C.c_void_p),
                ("rgb", C.c_void_p), ("tiles", C.c_void_p), ("clamped", C.c_void_p),
                ("rgb_raw", C.c_void_p)]


class OrcBands(C.Structure):
    _fields_ = [("alpha", C.c_double), ("trans", C.c_double), ("cap", C.c_double),
                ("clamp", C.c_double)]


# Relative widths of the near-threshold bands.  They bound how far an fp32
# evaluation of the same alpha / transmittance can sit from the fp64 value:
# alpha carries ~1e-6 relative error (power from fp32 conic terms, exp), the
# transmittance after several near-opaque layers ~1e-4.
DEFAULT_BANDS = dict(alpha=3e-5, trans=2e-3, cap=3e-5, clamp=1e-6)


def lib():
    global _lib
    if _lib is None:
        if _build.needs_build():
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _lib.orc_bin.restype = C.c_int64
        _lib.orc_bin_reach.restype = C.c_int64
        _lib.orc_tile_reach.restype = C.c_double
        _lib.orc_tile_reach.argtypes = [C.c_double] * 6 + [C.c_int, C.c_int]
        _lib.orc_render.restype = C.c_int64
        _lib.orc_render_pixel.restype = C.c_int
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else C.c_void_p(a.ctypes.data)


def cam_struct(cam) -> OrcCam:
    c = OrcCam()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    vm = np.asarray(cam.viewmat, dtype=np.float64).reshape(-1)
    for i in range(12):
        c.viewmat[i] = float(vm[i])
    c.znear, c.guard = float(cam.znear), float(cam.guard)
    c.lod_px = float(cam.lod_min_radius_px)
    return c


def bands_struct(**kw) -> OrcBands:
    d = dict(DEFAULT_BANDS)
    d.update(kw)
    b = OrcBands()
    b.alpha, b.trans, b.cap, b.clamp = d["alpha"], d["trans"], d["cap"], d["clamp"]
    return b


def project(means, scales, quats, opacities, sh_degree, sh, cam, active=None,
            precision: str = "f32") -> Dict[str, np.ndarray]:
    """Per-Gaussian projection records.  precision "f32": float inputs, fp32
    op-order contract; "f64": double inputs, smooth fp64."""
    dt = np.float32 if precision == "f32" else np.float64
    means = np.ascontiguousarray(means, dtype=dt)
    scales = np.ascontiguousarray(scales, dtype=dt)
    quats = np.ascontiguousarray(quats, dtype=dt)
    opacities = np.ascontiguousarray(opacities, dtype=dt)
    sh = np.ascontiguousarray(sh, dtype=dt)
    n = means.shape[1]
    out = dict(u=np.zeros(n), v=np.zeros(n), z=np.zeros(n), radius=np.zeros(n, np.int32),
               rect=np.zeros((4, n), np.int32), conic=np.zeros((3, n)), opacity=np.zeros(n),
               rgb=np.zeros((3, n)), tiles=np.zeros(n, np.int32), clamped=np.zeros(n, np.uint8),
               rgb_raw=np.zeros((3, n)))
    po = OrcProjOut(*[_p(out[k]) for k in ("u", "v", "z", "radius", "rect", "conic", "opacity",
                                           "rgb", "tiles", "clamped", "rgb_raw")])
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    c = cam_struct(cam)
    fn = lib().orc_project_f32 if precision == "f32" else lib().orc_project_f64
    fn(C.c_int64(n), _p(means), _p(scales), _p(quats), _p(opacities), C.c_int(sh_degree), _p(sh),
       _p(act), C.byref(c), C.byref(po))
    return out


def bin_sort(proj: Dict[str, np.ndarray], cam, reach: bool = False) -> Dict[str, np.ndarray]:
    """Per-tile lists sorted by (tile, depth, index); keys built as
    tile << 32 | fp32 bits of the depth (valid for fp32-contract records).
    reach=True keeps only the tiles each Gaussian reaches (orc_bin_reach)."""
    rect = np.ascontiguousarray(proj["rect"], dtype=np.int32)
    z = np.ascontiguousarray(proj["z"], dtype=np.float64)
    n = rect.shape[1]
    k = int(proj["tiles"].astype(np.int64).sum())
    tx, ty = (cam.width + 15) // 16, (cam.height + 15) // 16
    vals = np.zeros(max(k, 1), np.uint32)
    tile_of = np.zeros(max(k, 1), np.uint32)
    ranges = np.zeros(2 * tx * ty, np.uint32)
    if reach:
        f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
        u, v, conic, opac = f64(proj["u"]), f64(proj["v"]), f64(proj["conic"]), f64(proj["opacity"])
        k = lib().orc_bin_reach(C.c_int64(n), _p(rect), _p(z), _p(u), _p(v), _p(conic), _p(opac), C.c_int(tx),
                                C.c_int(ty), _p(vals), _p(tile_of), _p(ranges))
    else:
        kk = lib().orc_bin(C.c_int64(n), _p(rect), _p(z), C.c_int(tx), C.c_int(ty), _p(vals),
                           _p(tile_of), _p(ranges))
        assert kk == k
    vals, tile_of = vals[:k], tile_of[:k]
    depth_bits = proj["z"].astype(np.float32).view(np.uint32).astype(np.uint64)
    keys = (tile_of.astype(np.uint64) << np.uint64(32)) | depth_bits[vals]
    return dict(K=k, vals=vals, tile_of=tile_of, ranges=ranges.reshape(-1, 2), keys=keys)


def tile_reach(proj, g: int, tile: int, cam) -> float:
    """orc_tile_reach for Gaussian g and tile id `tile` of the camera's grid."""
    tx_n = (cam.width + 15) // 16
    c = proj["conic"]
    return float(lib().orc_tile_reach(float(proj["u"][g]), float(proj["v"][g]), float(c[0][g]), float(c[1][g]),
                                      float(c[2][g]), float(proj["opacity"][g]), tile % tx_n, tile // tx_n))


def render(proj, bins, cam, bg=(0.0, 0.0, 0.0), tile_mask=None, bands=None, weight=False):
    """Forward compositing (orc_render).  With weight=True the result also
    holds weight[n]: per Gaussian, the sum over the rendered pixels of its
    blending weight alpha_i T_i."""
    W, H = cam.width, cam.height
    n = proj["u"].shape[0]
    image = np.full((3, H, W), np.nan)
    final_T = np.full((H, W), np.nan)
    n_contrib = np.full((H, W), -1, np.int32)
    events = np.zeros((H, W), np.int32)
    capflag = np.zeros((H, W), np.uint8)
    w = np.zeros(n, np.float64) if weight else None
    bgv = np.asarray(bg, dtype=np.float64)
    tm = None if tile_mask is None else np.ascontiguousarray(tile_mask, dtype=np.uint8)
    b = bands_struct(**(bands or {}))
    c = cam_struct(cam)
    arr = {k: np.ascontiguousarray(proj[k], dtype=np.float64) for k in ("u", "v", "conic", "opacity", "rgb")}
    vals = np.ascontiguousarray(bins["vals"], dtype=np.uint32)
    ranges = np.ascontiguousarray(bins["ranges"], dtype=np.uint32)
    p_eval = lib().orc_render(C.byref(c), _p(arr["u"]), _p(arr["v"]), _p(arr["conic"]),
                              _p(arr["opacity"]), _p(arr["rgb"]), C.c_int64(n), _p(vals),
                              _p(ranges), _p(bgv), _p(tm), C.byref(b), _p(image), _p(final_T),
                              _p(n_contrib), _p(events), _p(capflag), _p(w))
    out = dict(image=image, final_T=final_T, n_contrib=n_contrib, events=events,
               capflag=capflag, p_eval=int(p_eval))
    if weight:
        out["weight"] = w
    return out


def render_pixel(proj, bins, cam, px, py, flips=0, bg=(0.0, 0.0, 0.0), bands=None):
    n = proj["u"].shape[0]
    out_rgb = np.zeros(3)
    out_T = C.c_double(0.0)
    out_n = C.c_int32(0)
    b = bands_struct(**(bands or {}))
    c = cam_struct(cam)
    bgv = np.asarray(bg, dtype=np.float64)
    arr = {k: np.ascontiguousarray(proj[k], dtype=np.float64) for k in ("u", "v", "conic", "opacity", "rgb")}
    vals = np.ascontiguousarray(bins["vals"], dtype=np.uint32)
    ranges = np.ascontiguousarray(bins["ranges"], dtype=np.uint32)
    ev = lib().orc_render_pixel(C.byref(c), _p(arr["u"]), _p(arr["v"]), _p(arr["conic"]),
                                _p(arr["opacity"]), _p(arr["rgb"]), C.c_int64(n), _p(vals),
                                _p(ranges), _p(bgv), C.byref(b), C.c_int(px), C.c_int(py),
                                C.c_uint32(flips), _p(out_rgb), C.byref(out_T), C.byref(out_n))
    return out_rgb, out_T.value, out_n.value, ev


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls."""
    lib().orc_set_num_threads(C.c_int(int(n)))


def render_pixels(proj, bins, cam, xs, ys, bg=(0.0, 0.0, 0.0), bands=None):
    """render_pixel over many pixels, the arrays marshalled once (for images
    too large to composite whole).  Returns rgb [3][m], T [m], n_contrib [m],
    events [m]."""
    n = proj["u"].shape[0]
    b = bands_struct(**(bands or {}))
    c = cam_struct(cam)
    bgv = np.asarray(bg, dtype=np.float64)
    arr = {k: np.ascontiguousarray(proj[k], dtype=np.float64) for k in ("u", "v", "conic", "opacity", "rgb")}
    vals = np.ascontiguousarray(bins["vals"], dtype=np.uint32)
    ranges = np.ascontiguousarray(bins["ranges"], dtype=np.uint32)
    m = len(xs)
    rgb = np.zeros((3, m))
    T = np.zeros(m)
    nc = np.zeros(m, np.int64)
    ev = np.zeros(m, np.int64)
    one = np.zeros(3)
    t = C.c_double(0.0)
    k = C.c_int32(0)
    for i in range(m):
        ev[i] = lib().orc_render_pixel(C.byref(c), _p(arr["u"]), _p(arr["v"]), _p(arr["conic"]),
                                       _p(arr["opacity"]), _p(arr["rgb"]), C.c_int64(n), _p(vals),
                                       _p(ranges), _p(bgv), C.byref(b), C.c_int(int(xs[i])), C.c_int(int(ys[i])),
                                       C.c_uint32(0), _p(one), C.byref(t), C.byref(k))
        rgb[:, i] = one
        T[i] = t.value
        nc[i] = k.value
    return rgb, T, nc, ev


def render_bwd(proj, bins, cam, dL_dimage, bg=(0.0, 0.0, 0.0), tile_mask=None):
    n = proj["u"].shape[0]
    grad2d = np.zeros((9, n))
    bgv = np.asarray(bg, dtype=np.float64)
    tm = None if tile_mask is None else np.ascontiguousarray(tile_mask, dtype=np.uint8)
    b = bands_struct()
    c = cam_struct(cam)
    arr = {k: np.ascontiguousarray(proj[k], dtype=np.float64) for k in ("u", "v", "conic", "opacity", "rgb")}
    vals = np.ascontiguousarray(bins["vals"], dtype=np.uint32)
    ranges = np.ascontiguousarray(bins["ranges"], dtype=np.uint32)
    g = np.ascontiguousarray(dL_dimage, dtype=np.float64)
    lib().orc_render_bwd(C.byref(c), _p(arr["u"]), _p(arr["v"]), _p(arr["conic"]),
                         _p(arr["opacity"]), _p(arr["rgb"]), C.c_int64(n), _p(vals), _p(ranges),
                         _p(bgv), _p(tm), C.byref(b), _p(g), _p(grad2d))
    return grad2d


def project_bwd(means, scales, quats, opacities, sh_degree, sh, cam, proj, grad2d):
    """Raw-parameter gradients (fp64) from the 2D record gradients."""
    f = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    means, scales, quats, opacities, sh = map(f, (means, scales, quats, opacities, sh))
    n = means.shape[1]
    k = (sh_degree + 1) ** 2
    out = dict(means=np.zeros((3, n)), log_scales=np.zeros((3, n)), quats=np.zeros((4, n)),
               opacity_logits=np.zeros(n), sh=np.zeros((k, 3, n)))
    c = cam_struct(cam)
    radius = np.ascontiguousarray(proj["radius"], dtype=np.int32)
    clamped = np.ascontiguousarray(proj["clamped"], dtype=np.uint8)
    g2 = f(grad2d)
    lib().orc_project_bwd(C.c_int64(n), _p(means), _p(scales), _p(quats), _p(opacities),
                          C.c_int(sh_degree), _p(sh), C.byref(c), _p(radius), _p(clamped), _p(g2),
                          _p(out["means"]), _p(out["log_scales"]), _p(out["quats"]),
                          _p(out["opacity_logits"]), _p(out["sh"]))
    return out


def topk_mask(scores, k):
    s = np.ascontiguousarray(scores, dtype=np.float32)
    m = np.zeros(s.shape[0], np.uint8)
    lib().orc_topk_mask(C.c_int64(s.shape[0]), _p(s), C.c_int64(k), _p(m))
    return m


def sh_quantize8(sh):
    """8-bit block quantization of SH [K][3][n] (orc_sh_quantize8): codes
    u8 [K][3][n] and bounds f32 [K*3][ceil(n/256)][2]."""
    x = np.ascontiguousarray(sh, dtype=np.float32)
    K, C3, n = x.shape
    nb = (n + 255) // 256
    q = np.zeros(x.shape, np.uint8)
    bounds = np.zeros((K * C3, nb, 2), np.float32)
    lib().orc_sh_quantize8(C.c_int64(n), C.c_int(K * C3), _p(x), _p(q), _p(bounds))
    return q, bounds


def sh_dequantize8(q, bounds):
    """Decode of sh_quantize8's codes to f32 [K][3][n]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    b = np.ascontiguousarray(bounds, dtype=np.float32)
    K, C3, n = q.shape
    x = np.zeros(q.shape, np.float32)
    lib().orc_sh_dequantize8(C.c_int64(n), C.c_int(K * C3), _p(q), _p(b), _p(x))
    return x


def sh_basis(d):
    d = np.ascontiguousarray(d, dtype=np.float64)
    Y = np.zeros(16)
    dY = np.zeros((16, 3))
    lib().orc_sh_basis(_p(d), _p(Y), _p(dY))
    return Y, dY


def forward(scene, view: int = 0, precision: str = "f32", tile_mask=None, bg=(0.0, 0.0, 0.0),
            active=None, sh=None):
    """Whole forward of one view: project, bin, composite."""
    cam = scene.cameras[view]
    sh = scene.sh_decoded() if sh is None else sh
    proj = project(scene.means, scene.scales, scene.quats, scene.opacities, scene.sh_degree,
                   sh, cam, active=active, precision=precision)
    bins = bin_sort(proj, cam)
    out = render(proj, bins, cam, bg=bg, tile_mask=tile_mask)
    return proj, bins, out
