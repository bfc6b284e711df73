"""ctypes binding of libgs_hip.so (C ABI in include/gs.h).

Argument marshalling only: torch tensors supply device memory and the
stream, every step of the rasterizer runs in the HIP library.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import torch

from . import build as _build

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_UNSUPPORTED, GS_ERR_WORKSPACE, GS_ERR_HIP = range(5)
GS_SH_F32, GS_SH_F16, GS_SH_Q8 = 0, 1, 2
GS_ADAM_F32, GS_ADAM_Q8LOG = 0, 1
GS_ADAM_DENSE, GS_ADAM_LAZY = 0, 1
SPLAT_FLOATS = 12          # gs_splat is 48 bytes


class GsCamera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("viewmat", C.c_float * 12),
                ("znear", C.c_float), ("guard", C.c_float), ("lod_min_radius_px", C.c_float),
                ("time", C.c_float)]


class GsFwdView(C.Structure):
    _fields_ = [("camera", GsCamera), ("splats", C.c_void_p), ("vals", C.c_void_p),
                ("tile_ranges", C.c_void_p), ("schedule", C.c_void_p), ("image", C.c_void_p),
                ("final_T", C.c_void_p), ("n_contrib", C.c_void_p), ("weight", C.c_void_p),
                ("reached_lists", C.c_int32)]


class GsSortView(C.Structure):
    _fields_ = [("camera", GsCamera), ("splats", C.c_void_p), ("n", C.c_int64), ("k_capacity", C.c_int64),
                ("vals", C.c_void_p), ("tile_ranges", C.c_void_p), ("schedule", C.c_void_p),
                ("bwd_index", C.c_void_p), ("keys", C.c_void_p), ("k_total", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("depth_keys", C.c_void_p), ("tile_rects", C.c_void_p), ("reach_tiles", C.c_int32)]


class GsBinKeys(C.Structure):
    _fields_ = [("depth_keys", C.c_void_p), ("tile_rects", C.c_void_p)]


class GsBwdView(C.Structure):
    _fields_ = [("camera", GsCamera), ("n", C.c_int64), ("splats", C.c_void_p), ("vals", C.c_void_p),
                ("tile_ranges", C.c_void_p), ("schedule", C.c_void_p), ("bwd_index", C.c_void_p),
                ("k_capacity", C.c_int64), ("final_T", C.c_void_p), ("n_contrib", C.c_void_p),
                ("dL_dimage", C.c_void_p), ("g2", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("reached_lists", C.c_int32)]


class GsGaussians(C.Structure):
    _fields_ = [("n", C.c_int64), ("sh_degree", C.c_int32), ("sh_dtype", C.c_int32),
                ("means", C.c_void_p), ("scales", C.c_void_p), ("quats", C.c_void_p),
                ("opacities", C.c_void_p), ("sh", C.c_void_p), ("active", C.c_void_p),
                ("sh_bounds", C.c_void_p), ("velocity", C.c_void_p), ("t_offset", C.c_void_p)]


class GsGrads(C.Structure):
    _fields_ = [("means", C.c_void_p), ("log_scales", C.c_void_p), ("quats", C.c_void_p),
                ("opacity_logits", C.c_void_p), ("sh", C.c_void_p), ("velocity", C.c_void_p),
                ("t_offset", C.c_void_p)]


class GsShAdam(C.Structure):
    _fields_ = [("n", C.c_int64), ("rows", C.c_int32), ("value_dtype", C.c_int32),
                ("state_dtype", C.c_int32), ("step", C.c_int32), ("lr", C.c_float),
                ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float), ("update", C.c_int32),
                ("grad", C.c_void_p), ("value", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p),
                ("m_bounds", C.c_void_p), ("v_bounds", C.c_void_p)]


class GsError(RuntimeError):
    pass


_lib = None
SYMBOLS = ("gs_project", "gs_bin_sort_workspace_bytes", "gs_schedule_words", "gs_bwd_index_words", "gs_bin_sort",
           "gs_bin_sort_views",
           "gs_render_fwd_views", "gs_render_bwd_screen_views", "gs_project_views", "gs_project_views_binned",
           "gs_render_fwd",
           "gs_render_bwd_workspace_bytes", "gs_render_bwd", "gs_render_bwd_screen_workspace_bytes",
           "gs_render_bwd_screen", "gs_project_bwd", "gs_project_bwd_binned", "gs_active_mask_workspace_bytes",
           "gs_active_mask", "gs_active_mask_static", "gs_active_mask_static_scratch_bytes",
           "gs_sh_q8_bounds_floats", "gs_sh_quantize8", "gs_sh_adam_step", "gs_status_string",
           "gs_version")


def lib_path() -> str:
    return _build.LIB


def lib():
    """Load the HIP library (built in tree by build.py); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise GsError(f"HIP library not built: {path} (run python -m gaussian_splatting_tile_amd.build)")
    L = C.CDLL(path)
    for name in SYMBOLS:
        getattr(L, name)
    vp, i64, sz = C.c_void_p, C.c_int64, C.c_size_t
    L.gs_project.argtypes = [C.POINTER(GsGaussians), C.POINTER(GsCamera), vp, vp]
    L.gs_bin_sort_workspace_bytes.argtypes = [i64, i64, C.c_int32]
    L.gs_bin_sort_workspace_bytes.restype = sz
    L.gs_schedule_words.argtypes = [C.c_int32, C.c_int32]
    L.gs_schedule_words.restype = sz
    L.gs_bwd_index_words.argtypes = [i64, i64]
    L.gs_bwd_index_words.restype = sz
    L.gs_bin_sort.argtypes = [vp, i64, C.POINTER(GsCamera), i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gs_bin_sort_views.argtypes = [C.c_int32, C.POINTER(GsSortView), vp]
    L.gs_render_fwd.argtypes = [vp, vp, vp, vp, C.POINTER(GsCamera), vp, vp, vp, vp, vp]
    L.gs_render_fwd_views.argtypes = [C.c_int32, C.POINTER(GsFwdView), vp, vp]
    L.gs_project_views.argtypes = [C.POINTER(GsGaussians), C.c_int32, C.POINTER(GsCamera), C.POINTER(vp), vp]
    L.gs_project_views_binned.argtypes = [C.POINTER(GsGaussians), C.c_int32, C.POINTER(GsCamera), C.POINTER(vp),
                                          C.POINTER(GsBinKeys), vp]
    L.gs_render_bwd_screen_views.argtypes = [C.c_int32, C.POINTER(GsBwdView), vp, vp]
    L.gs_render_bwd_workspace_bytes.argtypes = [i64, i64]
    L.gs_render_bwd_workspace_bytes.restype = sz
    L.gs_render_bwd.argtypes = [C.POINTER(GsGaussians), C.POINTER(GsCamera), vp, vp, vp, vp, vp, i64, vp, vp,
                                vp, vp, C.POINTER(GsGrads), vp, sz, vp]
    L.gs_render_bwd_screen_workspace_bytes.argtypes = [i64]
    L.gs_render_bwd_screen_workspace_bytes.restype = sz
    L.gs_render_bwd_screen.argtypes = [C.POINTER(GsCamera), i64, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp,
                                       vp, sz, vp]
    L.gs_project_bwd.argtypes = [C.POINTER(GsGaussians), C.c_int32, C.POINTER(GsCamera), C.POINTER(vp),
                                 C.POINTER(vp), C.POINTER(GsGrads), vp]
    L.gs_project_bwd_binned.argtypes = [C.POINTER(GsGaussians), C.c_int32, C.POINTER(GsCamera), C.POINTER(vp),
                                        C.POINTER(vp), C.POINTER(vp), C.POINTER(GsGrads), vp]
    L.gs_active_mask_workspace_bytes.argtypes = [i64]
    L.gs_active_mask_workspace_bytes.restype = sz
    L.gs_active_mask.argtypes = [vp, i64, i64, vp, vp, sz, vp]
    L.gs_active_mask_static.argtypes = [vp, i64, i64, vp, vp]
    L.gs_active_mask_static_scratch_bytes.argtypes = []
    L.gs_active_mask_static_scratch_bytes.restype = sz
    L.gs_sh_q8_bounds_floats.argtypes = [i64, C.c_int32]
    L.gs_sh_q8_bounds_floats.restype = sz
    L.gs_sh_quantize8.argtypes = [vp, i64, C.c_int32, vp, vp, vp]
    L.gs_sh_adam_step.argtypes = [C.POINTER(GsShAdam), vp]
    L.gs_status_string.restype = C.c_char_p
    L.gs_status_string.argtypes = [C.c_int]
    L.gs_version.restype = C.c_int32
    for name in ("gs_project", "gs_project_views", "gs_project_views_binned", "gs_bin_sort", "gs_bin_sort_views", "gs_render_fwd",
                 "gs_render_fwd_views",
                 "gs_render_bwd",
                 "gs_render_bwd_screen", "gs_render_bwd_screen_views",
                 "gs_project_bwd", "gs_project_bwd_binned", "gs_active_mask", "gs_active_mask_static",
                 "gs_sh_quantize8"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def _check(status: int, what: str):
    if status != GS_OK:
        msg = lib().gs_status_string(status).decode()
        raise GsError(f"{what} failed: {msg} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def camera_struct(cam) -> GsCamera:
    """From an object with width, height, fx, fy, cx, cy, viewmat[3][4],
    znear, guard, lod_min_radius_px (see scenes.Camera)."""
    c = GsCamera()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    vm = [float(x) for x in __import__("numpy").asarray(cam.viewmat, dtype="float32").reshape(-1)]
    for i in range(12):
        c.viewmat[i] = vm[i]
    c.znear, c.guard = float(cam.znear), float(cam.guard)
    c.lod_min_radius_px = float(getattr(cam, "lod_min_radius_px", 0.0))
    c.time = float(getattr(cam, "time", 0.0))
    return c


def grads_struct(grads: Dict[str, torch.Tensor]) -> GsGrads:
    """fp32 gradient arrays by name; "velocity" and "t_offset" only with
    moving Gaussians."""
    return GsGrads(_ptr(grads["means"]), _ptr(grads["log_scales"]), _ptr(grads["quats"]),
                   _ptr(grads["opacity_logits"]), _ptr(grads["sh"]), _ptr(grads.get("velocity")),
                   _ptr(grads.get("t_offset")))


def gaussians_struct(g: Dict[str, torch.Tensor], sh_degree: int, active: Optional[torch.Tensor] = None
                     ) -> GsGaussians:
    s = GsGaussians()
    s.n = int(g["means"].shape[1])
    s.sh_degree = int(sh_degree)
    s.sh_dtype = {torch.float16: GS_SH_F16, torch.uint8: GS_SH_Q8}.get(g["sh"].dtype, GS_SH_F32)
    for k in ("means", "scales", "quats", "opacities"):
        t = g[k]
        assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous(), k
    assert g["sh"].is_cuda and g["sh"].is_contiguous()
    s.means, s.scales, s.quats = g["means"].data_ptr(), g["scales"].data_ptr(), g["quats"].data_ptr()
    s.opacities, s.sh = g["opacities"].data_ptr(), g["sh"].data_ptr()
    if active is not None:
        assert active.is_cuda and active.dtype == torch.uint8 and active.is_contiguous()
        s.active = active.data_ptr()
    if s.sh_dtype == GS_SH_Q8:
        b = g["sh_bounds"]
        assert b.is_cuda and b.dtype == torch.float32 and b.is_contiguous()
        s.sh_bounds = b.data_ptr()
    if g.get("velocity") is not None:
        v, t = g["velocity"], g["t_offset"]
        assert v.is_cuda and v.dtype == torch.float32 and v.is_contiguous() and tuple(v.shape) == (3, s.n)
        assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and t.numel() == s.n
        s.velocity, s.t_offset = v.data_ptr(), t.data_ptr()
    return s


def sh_q8_bounds_floats(n: int, rows: int) -> int:
    return int(lib().gs_sh_q8_bounds_floats(n, rows))


def sh_quantize8(sh: torch.Tensor, codes: torch.Tensor, bounds: torch.Tensor, stream=None):
    """gs_sh_quantize8: sh float32 [K][3][n] -> codes uint8 [K][3][n], bounds
    float32 [K*3][ceil(n/256)][2]."""
    K, c3, n = sh.shape
    assert sh.dtype == torch.float32 and sh.is_contiguous() and codes.dtype == torch.uint8
    assert bounds.numel() >= sh_q8_bounds_floats(n, K * c3)
    _check(lib().gs_sh_quantize8(_ptr(sh), int(n), int(K * c3), _ptr(codes), _ptr(bounds), _stream(stream)),
           "gs_sh_quantize8")


def sh_adam_struct(grad: torch.Tensor, value: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                   m_bounds: Optional[torch.Tensor] = None, v_bounds: Optional[torch.Tensor] = None,
                   step: int = 1, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                   eps: float = 1e-15, lazy: bool = True) -> GsShAdam:
    """Descriptor of gs_sh_adam_step over [rows][n] (or [K][3][n]) arrays:
    grad float32; value float32 or float16; m, v float32 (full-precision
    state) or uint8 codes with float32 bounds [rows][ceil(n/256)][2];
    lazy: units with a zero gradient keep their state (else every unit
    moves)."""
    n = grad.shape[-1]
    rows = grad.numel() // n if n else grad.shape[0]
    for t in (grad, value, m, v):
        assert t.is_contiguous() and t.shape == grad.shape, "arrays must be contiguous and of one shape"
    assert grad.dtype == torch.float32 and value.dtype in (torch.float32, torch.float16)
    a = GsShAdam()
    a.n, a.rows, a.step = int(n), int(rows), int(step)
    a.value_dtype = GS_SH_F16 if value.dtype == torch.float16 else GS_SH_F32
    a.lr, a.beta1, a.beta2, a.eps = float(lr), float(beta1), float(beta2), float(eps)
    a.update = GS_ADAM_LAZY if lazy else GS_ADAM_DENSE
    a.grad, a.value, a.m, a.v = _ptr(grad), _ptr(value), _ptr(m), _ptr(v)
    if m.dtype == torch.uint8:
        assert v.dtype == torch.uint8 and m_bounds is not None and v_bounds is not None
        nbf = sh_q8_bounds_floats(n, rows)
        assert m_bounds.dtype == torch.float32 and m_bounds.numel() >= nbf and m_bounds.is_contiguous()
        assert v_bounds.dtype == torch.float32 and v_bounds.numel() >= nbf and v_bounds.is_contiguous()
        a.state_dtype = GS_ADAM_Q8LOG
        a.m_bounds, a.v_bounds = _ptr(m_bounds), _ptr(v_bounds)
    else:
        assert m.dtype == torch.float32 and v.dtype == torch.float32
        a.state_dtype = GS_ADAM_F32
    return a


def sh_adam_step(grad, value, m, v, m_bounds=None, v_bounds=None, step=1, lr=1e-3, beta1=0.9,
                 beta2=0.999, eps=1e-15, stream=None, lazy=True):
    """gs_sh_adam_step: one fused Adam update of value, m, v (and the bounds)
    in place; lazy (SparseAdam's rule) or dense (every unit)."""
    a = sh_adam_struct(grad, value, m, v, m_bounds, v_bounds, step, lr, beta1, beta2, eps, lazy)
    _check(lib().gs_sh_adam_step(C.byref(a), _stream(stream)), "gs_sh_adam_step")


# ---- the four calls ---------------------------------------------------------
def project(gs: GsGaussians, cam: GsCamera, splats: torch.Tensor, stream=None):
    _check(lib().gs_project(C.byref(gs), C.byref(cam), _ptr(splats), _stream(stream)), "gs_project")


def bin_sort_workspace_bytes(n: int, k_capacity: int, n_tiles: int) -> int:
    return int(lib().gs_bin_sort_workspace_bytes(n, k_capacity, n_tiles))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def schedule_words(width: int, height: int) -> int:
    return int(lib().gs_schedule_words(width, height))


def bwd_index_words(n: int, k_capacity: int) -> int:
    return int(lib().gs_bwd_index_words(n, k_capacity))


def bin_sort(splats, n, cam: GsCamera, k_capacity, vals, tile_ranges, schedule, bwd_index, keys, k_total,
             workspace, stream=None):
    _check(lib().gs_bin_sort(_ptr(splats), int(n), C.byref(cam), int(k_capacity), _ptr(vals),
                             _ptr(tile_ranges), _ptr(schedule), _ptr(bwd_index), _ptr(keys), _ptr(k_total),
                             _ptr(workspace), _nbytes(workspace), _stream(stream)), "gs_bin_sort")


def bin_sort_views(bufs, with_bwd: bool = True, stream=None, prebinned=False, reach=False):
    """gs_bin_sort_views over ViewBuffers objects (their splats must be
    current): one launch per sort step for up to 8 views.  prebinned: take
    the depth keys and tile rects that project_views(..., binned=True) wrote
    into the buffers with those splats (one flag for all views, or one per
    view).  reach: list each Gaussian only in the tiles it reaches (one flag
    for all views, or one per view)."""
    nv = len(bufs)
    pre = list(prebinned) if isinstance(prebinned, (list, tuple)) else [prebinned] * nv
    rch = list(reach) if isinstance(reach, (list, tuple)) else [reach] * nv
    arr = (GsSortView * max(nv, 1))()
    for i, b in enumerate(bufs):
        b.reached = bool(rch[i])
        arr[i] = GsSortView(b.camc, _ptr(b.splats), int(b.n), int(b.k_capacity), _ptr(b.vals), _ptr(b.ranges),
                            _ptr(b.schedule), _ptr(b.bwd_index) if with_bwd else None, _ptr(b.keys),
                            _ptr(b.k_total),
                            _ptr(b.ws), _nbytes(b.ws),
                            _ptr(b.depth_keys) if pre[i] else None,
                            _ptr(b.tile_rects) if pre[i] and not rch[i] else None, 1 if rch[i] else 0)
    _check(lib().gs_bin_sort_views(nv, arr, _stream(stream)), "gs_bin_sort_views")


def render_fwd(splats, vals, tile_ranges, schedule, cam: GsCamera, bg: Sequence[float], image, final_T,
               n_contrib, stream=None):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    _check(lib().gs_render_fwd(_ptr(splats), _ptr(vals), _ptr(tile_ranges), _ptr(schedule), C.byref(cam),
                               C.cast(bgv, C.c_void_p), _ptr(image), _ptr(final_T), _ptr(n_contrib),
                               _stream(stream)), "gs_render_fwd")


def project_views(gs: GsGaussians, cams, splats_list, stream=None, bin_keys=None):
    """gs_project_views: records for every camera of the list in one pass.
    bin_keys: None, or one (depth_keys uint32/int32 [n], tile_rects
    uint32/int32 [2n] or None) pair (or None) per camera, for
    gs_project_views_binned (rects may be left out for views sorted with
    reach=True)."""
    nv = len(cams)
    cam_arr = (GsCamera * max(nv, 1))(*cams)
    sp_arr = (C.c_void_p * max(nv, 1))(*[_ptr(t) for t in splats_list])
    if bin_keys is None:
        _check(lib().gs_project_views(C.byref(gs), nv, cam_arr, sp_arr, _stream(stream)), "gs_project_views")
        return
    bk = (GsBinKeys * max(nv, 1))()
    for i, pair in enumerate(bin_keys):
        if pair is not None:
            bk[i] = GsBinKeys(_ptr(pair[0]), None if pair[1] is None else _ptr(pair[1]))
    _check(lib().gs_project_views_binned(C.byref(gs), nv, cam_arr, sp_arr, bk, _stream(stream)),
           "gs_project_views_binned")


def render_fwd_views(bufs, bg: Sequence[float] = (0.0, 0.0, 0.0), stream=None, weights=None):
    """gs_render_fwd_views over ViewBuffers objects (their splats, bins and
    schedules must be current).  weights: None, one float32 [n] tensor shared
    by all views, or a list with one tensor (or None) per view; the
    per-Gaussian blending weights are added to it."""
    nv = len(bufs)
    if weights is None or isinstance(weights, torch.Tensor):
        weights = [weights] * nv
    arr = (GsFwdView * max(nv, 1))()
    for i, b in enumerate(bufs):
        arr[i] = GsFwdView(b.camc, _ptr(b.splats), _ptr(b.vals), _ptr(b.ranges), _ptr(b.schedule),
                           _ptr(b.image), _ptr(b.final_T), _ptr(b.n_contrib), _ptr(weights[i]),
                           1 if getattr(b, "reached", False) else 0)
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    _check(lib().gs_render_fwd_views(nv, arr, C.cast(bgv, C.c_void_p), _stream(stream)), "gs_render_fwd_views")


def render_bwd_workspace_bytes(n: int, k_capacity: int) -> int:
    return int(lib().gs_render_bwd_workspace_bytes(n, k_capacity))


def render_bwd(gs: GsGaussians, cam: GsCamera, splats, vals, tile_ranges, schedule, bwd_index, k_capacity, bg,
               final_T, n_contrib, dL_dimage, grads: Dict[str, torch.Tensor], workspace, stream=None):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    gr = grads_struct(grads)
    _check(lib().gs_render_bwd(C.byref(gs), C.byref(cam), _ptr(splats), _ptr(vals), _ptr(tile_ranges),
                               _ptr(schedule), _ptr(bwd_index), int(k_capacity), C.cast(bgv, C.c_void_p), _ptr(final_T), _ptr(n_contrib), _ptr(dL_dimage),
                               C.byref(gr), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "gs_render_bwd")


def render_bwd_screen_workspace_bytes(k_capacity: int) -> int:
    return int(lib().gs_render_bwd_screen_workspace_bytes(k_capacity))


def render_bwd_screen(cam: GsCamera, n, splats, vals, tile_ranges, schedule, bwd_index, k_capacity, bg, final_T,
                      n_contrib, dL_dimage, g2, workspace, stream=None):
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    _check(lib().gs_render_bwd_screen(C.byref(cam), int(n), _ptr(splats), _ptr(vals), _ptr(tile_ranges),
                                      _ptr(schedule), _ptr(bwd_index), int(k_capacity), C.cast(bgv, C.c_void_p),
                                      _ptr(final_T), _ptr(n_contrib), _ptr(dL_dimage), _ptr(g2), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream)), "gs_render_bwd_screen")


def render_bwd_screen_views(bufs, dLs, g2s, workspaces, bg: Sequence[float] = (0.0, 0.0, 0.0), stream=None):
    """gs_render_bwd_screen_views over ViewBuffers objects with their upstream
    gradients, g2 outputs [n][9] and workspaces."""
    nv = len(bufs)
    arr = (GsBwdView * max(nv, 1))()
    for i, (b, dL, g2, ws) in enumerate(zip(bufs, dLs, g2s, workspaces)):
        arr[i] = GsBwdView(b.camc, b.n, _ptr(b.splats), _ptr(b.vals), _ptr(b.ranges), _ptr(b.schedule),
                           _ptr(b.bwd_index), b.k_capacity, _ptr(b.final_T), _ptr(b.n_contrib), _ptr(dL),
                           _ptr(g2), _ptr(ws), _nbytes(ws), 1 if getattr(b, "reached", False) else 0)
    bgv = (C.c_float * 3)(*[float(x) for x in bg])
    _check(lib().gs_render_bwd_screen_views(nv, arr, C.cast(bgv, C.c_void_p), _stream(stream)),
           "gs_render_bwd_screen_views")


def project_bwd(gs: GsGaussians, cams, splats_list, g2_list, grads: Dict[str, torch.Tensor], stream=None,
                depth_keys=None):
    """Chain rule of a batch of views: cams is a list of GsCamera, splats_list
    and g2_list the matching device tensors.  depth_keys (a list of the views'
    depth-key tensors from project_views(bin_keys=...), None entries allowed)
    selects gs_project_bwd_binned, which takes visibility from the keys."""
    nv = len(cams)
    cam_arr = (GsCamera * max(nv, 1))(*cams)
    sp_arr = (C.c_void_p * max(nv, 1))(*[_ptr(t) for t in splats_list])
    g2_arr = (C.c_void_p * max(nv, 1))(*[_ptr(t) for t in g2_list])
    gr = grads_struct(grads)
    if depth_keys is None:
        _check(lib().gs_project_bwd(C.byref(gs), nv, cam_arr, sp_arr, g2_arr, C.byref(gr), _stream(stream)),
               "gs_project_bwd")
        return
    if len(depth_keys) != nv:
        raise ValueError("project_bwd: one depth-key tensor (or None) per view")
    dk_arr = (C.c_void_p * max(nv, 1))(*[None if t is None else _ptr(t) for t in depth_keys])
    _check(lib().gs_project_bwd_binned(C.byref(gs), nv, cam_arr, sp_arr, g2_arr, dk_arr, C.byref(gr),
                                       _stream(stream)), "gs_project_bwd_binned")


def active_mask_workspace_bytes(n: int) -> int:
    return int(lib().gs_active_mask_workspace_bytes(n))


def active_mask(scores, n, keep, mask, workspace, stream=None):
    _check(lib().gs_active_mask(_ptr(scores), int(n), int(keep), _ptr(mask), _ptr(workspace),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream(stream)), "gs_active_mask")


def active_mask_static(scores, n, keep, mask, stream=None):
    """gs_active_mask with the library's fixed scratch array: no workspace,
    nothing allocated (n up to 2^30)."""
    _check(lib().gs_active_mask_static(_ptr(scores), int(n), int(keep), _ptr(mask), _stream(stream)),
           "gs_active_mask_static")


# ---- buffers for one view ---------------------------------------------------
class ViewBuffers:
    """Device buffers for rendering one camera with a fixed key capacity."""

    def __init__(self, n: int, cam, k_capacity: int, device="cuda", with_keys: bool = False,
                 with_backward: bool = True):
        self.n = n
        self.cam = cam
        self.camc = camera_struct(cam)
        self.n_tiles = ((cam.width + 15) // 16) * ((cam.height + 15) // 16)
        self.k_capacity = int(k_capacity)
        kc = max(self.k_capacity, 1)
        self.splats = torch.empty((max(n, 1), SPLAT_FLOATS), dtype=torch.float32, device=device)
        self.vals = torch.empty(kc, dtype=torch.int32, device=device)
        self.keys = torch.empty(kc, dtype=torch.int64, device=device) if with_keys else None
        self.ranges = torch.empty((self.n_tiles, 2), dtype=torch.int32, device=device)
        self.k_total = torch.zeros(1, dtype=torch.int64, device=device)
        wsb = bin_sort_workspace_bytes(n, self.k_capacity, self.n_tiles)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=device)
        H, W = cam.height, cam.width
        self.image = torch.empty((3, H, W), dtype=torch.float32, device=device)
        self.final_T = torch.empty((H, W), dtype=torch.float32, device=device)
        self.n_contrib = torch.empty((H, W), dtype=torch.int32, device=device)
        self.schedule = torch.empty(schedule_words(W, H), dtype=torch.int32, device=device)
        self.bwd_index = (torch.empty(bwd_index_words(n, self.k_capacity), dtype=torch.int32, device=device)
                          if with_backward else None)
        # the sort's per-Gaussian inputs when the projection writes them
        # set by bin_sort_views: the lists hold only reached tiles (a hint
        # passed on to the blend kernels)
        self.reached = False
        self.depth_keys = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.tile_rects = torch.empty(2 * max(n, 1), dtype=torch.int32, device=device)

    @property
    def bin_keys(self):
        return (self.depth_keys, self.tile_rects)

    def forward(self, gs: GsGaussians, bg=(0.0, 0.0, 0.0), stream=None):
        self.reached = False
        project(gs, self.camc, self.splats, stream)
        bin_sort(self.splats, self.n, self.camc, self.k_capacity, self.vals, self.ranges, self.schedule,
                 self.bwd_index, self.keys, self.k_total, self.ws, stream)
        render_fwd(self.splats, self.vals, self.ranges, self.schedule, self.camc, bg, self.image, self.final_T,
                   self.n_contrib, stream)

    def backward_workspace(self, device="cuda"):
        return torch.empty(render_bwd_workspace_bytes(self.n, self.k_capacity), dtype=torch.uint8, device=device)

    def backward_screen(self, dL_dimage, g2, workspace, bg=(0.0, 0.0, 0.0), stream=None):
        """Screen-space backward of this view into g2 [n][9] (for project_bwd)."""
        render_bwd_screen(self.camc, self.n, self.splats, self.vals, self.ranges, self.schedule, self.bwd_index,
                          self.k_capacity, bg, self.final_T, self.n_contrib, dL_dimage, g2, workspace, stream)

    def backward(self, gs: GsGaussians, dL_dimage, grads, workspace, bg=(0.0, 0.0, 0.0), stream=None):
        render_bwd(gs, self.camc, self.splats, self.vals, self.ranges, self.schedule, self.bwd_index,
                   self.k_capacity, bg, self.final_T, self.n_contrib, dL_dimage, grads, workspace, stream)
