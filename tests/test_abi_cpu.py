"""Host-side checks of the C ABI that need no GPU: the library builds, loads,
and exports every function include/gs.h declares; the header's struct
layouts match the binding's; argument errors that are decided on the host
come back without touching a device."""
import ctypes as C
import os
import re

import pytest

from gaussian_splatting_tile_amd import binding as B
from gaussian_splatting_tile_amd import build as gbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "gs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gs_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    if gbuild.needs_build():
        gbuild.build()
    L = B.lib()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"{n} missing from {B.lib_path()}"
    assert set(names) == set(B.SYMBOLS)


def test_struct_layouts_match_header():
    """Every field offset and struct size of the ctypes mirrors equals what a
    C compiler makes of include/gs.h."""
    import shutil
    import subprocess
    import tempfile
    pairs = [("gs_camera", B.GsCamera), ("gs_gaussians", B.GsGaussians), ("gs_grads", B.GsGrads),
             ("gs_fwd_view", B.GsFwdView), ("gs_sort_view", B.GsSortView), ("gs_bwd_view", B.GsBwdView),
             ("gs_sh_adam", B.GsShAdam), ("gs_bin_keys", B.GsBinKeys)]
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "gs.h"', "int main(void) {"]
    expect = []
    for cname, cls in pairs:
        lines.append(f'printf("%zu\\n", sizeof({cname}));')
        expect.append(C.sizeof(cls))
        for fname, _ in cls._fields_:
            lines.append(f'printf("%zu\\n", offsetof({cname}, {fname}));')
            expect.append(getattr(cls, fname).offset)
    lines += ['printf("%zu\\n", sizeof(gs_splat));', "return 0; }"]
    expect.append(B.SPLAT_FLOATS * 4)
    cc = shutil.which("gcc") or shutil.which("cc")
    assert cc, "no C compiler"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "layout.c")
        open(src, "w").write("\n".join(lines) + "\n")
        exe = os.path.join(d, "layout")
        subprocess.run([cc, "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert got == expect


def test_status_strings_and_version():
    L = B.lib()
    assert L.gs_version() >= 1
    assert L.gs_status_string(0).decode() == "ok"
    assert "workspace" in L.gs_status_string(3).decode()


def test_host_side_argument_errors_without_device():
    L = B.lib()
    cam = B.GsCamera()
    cam.width, cam.height, cam.fx, cam.fy = 0, 10, 1.0, 1.0
    gs = B.GsGaussians()
    gs.n = 0
    assert L.gs_project(C.byref(gs), C.byref(cam), None, None) == B.GS_ERR_INVALID_ARG
    cam.width = 10
    cam.guard = 1.3
    gs.sh_degree = 7
    assert L.gs_project(C.byref(gs), C.byref(cam), None, None) == B.GS_ERR_UNSUPPORTED
    assert L.gs_bin_sort(None, -1, C.byref(cam), 0, None, None, None, None, None, None, None, 0, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_active_mask(None, 10, 11, None, None, 0, None) == B.GS_ERR_INVALID_ARG
    # the allocation-free mask: same argument rules, and n above the fixed
    # scratch array's maximum (2^30) is refused before any device call
    assert L.gs_active_mask_static(None, 10, 11, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_active_mask_static(None, 10, 5, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_active_mask_static(None, -1, 0, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_active_mask_static(0x1000, (1 << 30) + 1, 7, 0x1000, None) == B.GS_ERR_WORKSPACE
    assert L.gs_active_mask_static(0x1000, 1 << 31, 7, 0x1000, None) == B.GS_ERR_INVALID_ARG
    # the array holds the workspace layout of 2^30 scores (one word per
    # 4096-score block plus histograms and state)
    sb = L.gs_active_mask_static_scratch_bytes()
    assert sb >= L.gs_active_mask_workspace_bytes(1 << 30) - 256 and sb < (2 << 20)
    # 8-bit SH storage
    assert L.gs_sh_quantize8(None, -1, 48, None, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_sh_quantize8(None, 10, 0, None, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_sh_quantize8(None, 10, 48, None, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_sh_quantize8(None, 0, 48, None, None, None) == B.GS_OK
    assert L.gs_sh_q8_bounds_floats(257, 48) == 48 * 2 * 2
    assert L.gs_sh_q8_bounds_floats(-1, 48) == 0
    gq = B.GsGaussians()
    gq.n, gq.sh_degree, gq.sh_dtype = 5, 3, B.GS_SH_Q8
    gq.means = gq.scales = gq.quats = gq.opacities = gq.sh = 0x1000
    camq = B.GsCamera()
    camq.width, camq.height, camq.fx, camq.fy, camq.guard = 16, 16, 10.0, 10.0, 1.3
    assert L.gs_project(C.byref(gq), C.byref(camq), 0x1000, None) == B.GS_ERR_INVALID_ARG   # no bounds
    gq.sh_dtype = 3
    assert L.gs_project(C.byref(gq), C.byref(camq), 0x1000, None) == B.GS_ERR_UNSUPPORTED
    # moving Gaussians: velocity and time offsets come together, the view's
    # time must be finite, and the backward needs both gradient arrays
    gm = B.GsGaussians()
    gm.n, gm.sh_degree, gm.sh_dtype = 5, 0, B.GS_SH_F32
    gm.means = gm.scales = gm.quats = gm.opacities = gm.sh = 0x1000
    gm.velocity = 0x1000
    assert L.gs_project(C.byref(gm), C.byref(camq), 0x1000, None) == B.GS_ERR_INVALID_ARG
    gm.t_offset = 0x1000
    camq.time = float("nan")
    assert L.gs_project(C.byref(gm), C.byref(camq), 0x1000, None) == B.GS_ERR_INVALID_ARG
    camq.time = 0.5
    grm = B.GsGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, None)
    sp = (C.c_void_p * 1)(0x1000)
    assert L.gs_project_bwd(C.byref(gm), 1, C.byref(camq), sp, sp, C.byref(grm), None) == B.GS_ERR_INVALID_ARG
    # the keyed projection backward: the key array is required, each key
    # pointer 4-byte aligned (checked before anything is launched)
    gk = B.GsGaussians()
    gk.n, gk.sh_degree, gk.sh_dtype = 5, 0, B.GS_SH_F32
    gk.means = gk.scales = gk.quats = gk.opacities = gk.sh = 0x1000
    grk = B.GsGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, None)
    keys = (C.c_void_p * 1)(0x1002)
    assert L.gs_project_bwd_binned(C.byref(gk), 1, C.byref(camq), sp, sp, None, C.byref(grk),
                                   None) == B.GS_ERR_INVALID_ARG
    assert L.gs_project_bwd_binned(C.byref(gk), 1, C.byref(camq), sp, sp, keys, C.byref(grk),
                                   None) == B.GS_ERR_INVALID_ARG
    assert L.gs_project_bwd_binned(C.byref(gk), 0, None, None, None, None, C.byref(grk), None) == B.GS_OK
    # batched sort: every view is checked before anything runs
    views = (B.GsSortView * 2)()
    assert L.gs_bin_sort_views(-1, views, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_bin_sort_views(2, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_bin_sort_views(0, None, None) == B.GS_OK
    for v in views:
        v.camera = cam
        v.n, v.k_capacity = 0, 0
        v.tile_ranges = v.schedule = v.k_total = v.workspace = 0x1000
        v.workspace_bytes = 1 << 20
    views[1].k_total = None
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_INVALID_ARG
    views[1].k_total = 0x1000
    views[1].n = 100
    views[1].splats = 0x1000
    views[1].workspace_bytes = 16
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_WORKSPACE
    # the projection's sort inputs: both or neither, aligned
    views[1].workspace_bytes = 1 << 30
    views[1].depth_keys = 0x1000
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_INVALID_ARG
    # a reach sort takes its rects from the records: view 1 passes its
    # checks, so the call fails only at view 2's small workspace (and
    # launches nothing)
    views3 = (B.GsSortView * 3)(views[0], views[1], views[1])
    views3[1].reach_tiles = 1
    views3[2].depth_keys = None
    views3[2].workspace_bytes = 16
    assert L.gs_bin_sort_views(3, views3, None) == B.GS_ERR_WORKSPACE
    views3[1].reach_tiles = 0
    assert L.gs_bin_sort_views(3, views3, None) == B.GS_ERR_INVALID_ARG
    views[1].depth_keys, views[1].tile_rects = None, 0x1008
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_INVALID_ARG
    views[1].depth_keys = 0x1000
    views[1].tile_rects = 0x1004
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_INVALID_ARG
    views[1].depth_keys, views[1].tile_rects = 0x1002, 0x1008
    assert L.gs_bin_sort_views(2, views, None) == B.GS_ERR_INVALID_ARG
    views[1].depth_keys = views[1].tile_rects = None
    gb = B.GsGaussians()
    gb.n, gb.sh_degree = 0, 0
    camb = B.GsCamera()
    camb.width, camb.height, camb.fx, camb.fy, camb.guard = 16, 16, 10.0, 10.0, 1.3
    spb = (C.c_void_p * 1)(0x1000)
    bk = (B.GsBinKeys * 1)()
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, bk, None) == B.GS_OK   # n = 0: nothing runs
    bk[0].depth_keys = 0x1000                  # depth keys alone are allowed
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, bk, None) == B.GS_OK
    bk[0].depth_keys, bk[0].tile_rects = None, 0x1008
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, bk, None) == B.GS_ERR_INVALID_ARG
    bk[0].depth_keys = 0x1000
    bk[0].tile_rects = 0x100C
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, bk, None) == B.GS_ERR_INVALID_ARG
    bk[0].tile_rects = 0x1008
    assert L.gs_project_views_binned(C.byref(gb), 1, C.byref(camb), spb, bk, None) == B.GS_OK
    bgv = (C.c_float * 3)(0.0, 0.0, 0.0)
    # a negative near plane would let depths of either sign through, which the
    # depth key does not order; it is refused like any other bad camera field
    camz = B.GsCamera()
    camz.width, camz.height, camz.fx, camz.fy, camz.guard = 16, 16, 10.0, 10.0, 1.3
    gz = B.GsGaussians()
    gz.n = 0
    assert L.gs_project(C.byref(gz), C.byref(camz), None, None) == B.GS_OK
    camz.znear = -0.1
    assert L.gs_project(C.byref(gz), C.byref(camz), None, None) == B.GS_ERR_INVALID_ARG
    camz.znear = float("nan")
    assert L.gs_project(C.byref(gz), C.byref(camz), None, None) == B.GS_ERR_INVALID_ARG
    camz.znear = 0.2
    # the forward refuses NULL records or list entries (a GPU fault otherwise)
    d = 0x1000
    assert L.gs_render_fwd(None, d, d, d, C.byref(camz), C.cast(bgv, C.c_void_p), d, d, d, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_render_fwd(d, None, d, d, C.byref(camz), C.cast(bgv, C.c_void_p), d, d, d, None) == B.GS_ERR_INVALID_ARG
    fv = (B.GsFwdView * 1)()
    fv[0].camera = camz
    fv[0].splats, fv[0].vals = d, None
    fv[0].tile_ranges = fv[0].schedule = fv[0].image = fv[0].final_T = fv[0].n_contrib = d
    assert L.gs_render_fwd_views(1, fv, C.cast(bgv, C.c_void_p), None) == B.GS_ERR_INVALID_ARG
    fv[0].splats, fv[0].vals = None, d
    assert L.gs_render_fwd_views(1, fv, C.cast(bgv, C.c_void_p), None) == B.GS_ERR_INVALID_ARG
    assert L.gs_render_bwd_screen(None, 10, None, None, None, None, None, 0, C.cast(bgv, C.c_void_p), None,
                                  None, None, None, None, 0, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_project_bwd(C.byref(gs), 1, None, None, None, None, None) == B.GS_ERR_UNSUPPORTED
    gs.sh_degree = 0
    assert L.gs_project_bwd(C.byref(gs), -1, None, None, None, None, None) == B.GS_ERR_INVALID_ARG
    assert L.gs_render_bwd_screen_workspace_bytes(1000) >= 1000 * 36
    assert L.gs_bin_sort_workspace_bytes(1000, 5000, 64) > 5000 * 12
    assert L.gs_render_bwd_workspace_bytes(1000, 4000) >= 5000 * 36
    assert L.gs_bwd_index_words(10, 100) == 100 + 2 * 10 + 2
    assert L.gs_schedule_words(128, 128) == 64 + 4
    assert L.gs_schedule_words(0, 128) == 0


def test_sh_adam_argument_errors_without_device():
    """gs_sh_adam_step checks its descriptor on the host; n == 0 launches
    nothing."""
    L = B.lib()
    assert L.gs_sh_adam_step(None, None) == B.GS_ERR_INVALID_ARG

    def desc(**kw):
        a = B.GsShAdam()
        a.n, a.rows, a.value_dtype, a.state_dtype, a.step = 1000, 45, B.GS_SH_F16, B.GS_ADAM_Q8LOG, 1
        a.lr, a.beta1, a.beta2, a.eps = 1e-3, 0.9, 0.999, 1e-15
        a.grad = a.value = a.m = a.v = a.m_bounds = a.v_bounds = 0x1000
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    bad = [dict(n=-1), dict(rows=0), dict(rows=65536), dict(value_dtype=B.GS_SH_Q8), dict(state_dtype=2),
           dict(step=0), dict(lr=-1.0), dict(lr=float("inf")), dict(beta1=1.0), dict(beta2=-0.5),
           dict(eps=0.0), dict(eps=float("nan")), dict(grad=None), dict(value=None), dict(m=None),
           dict(v=None), dict(m_bounds=None), dict(v_bounds=None), dict(update=2), dict(update=-1)]
    for kw in bad:
        assert L.gs_sh_adam_step(C.byref(desc(**kw)), None) == B.GS_ERR_INVALID_ARG, kw
    # the full-precision state needs no bounds; an empty update does nothing
    a = desc(n=0, state_dtype=B.GS_ADAM_F32, m_bounds=None, v_bounds=None, grad=None, value=None, m=None, v=None)
    assert L.gs_sh_adam_step(C.byref(a), None) == B.GS_OK


def test_misaligned_splats_and_workspaces_are_rejected():
    """Splat arrays and workspaces are read with 16-byte vector accesses: a
    pointer off a 16-byte boundary is an argument error, found before
    anything is launched."""
    L = B.lib()
    cam = B.GsCamera()
    cam.width, cam.height, cam.fx, cam.fy, cam.guard = 16, 16, 10.0, 10.0, 1.3
    g = B.GsGaussians()
    g.n, g.sh_degree, g.sh_dtype = 5, 0, B.GS_SH_F32
    g.means = g.scales = g.quats = g.opacities = g.sh = 0x1000
    assert L.gs_project(C.byref(g), C.byref(cam), 0x1008, None) == B.GS_ERR_INVALID_ARG
    sp = (C.c_void_p * 1)(0x1004)
    assert L.gs_project_views(C.byref(g), 1, C.byref(cam), sp, None) == B.GS_ERR_INVALID_ARG
    bgv = (C.c_float * 3)(0.0, 0.0, 0.0)
    assert L.gs_render_fwd(0x1008, 0x1000, 0x1000, 0x1000, C.byref(cam), C.cast(bgv, C.c_void_p), 0x1000,
                           0x1000, 0x1000, None) == B.GS_ERR_INVALID_ARG
    v = B.GsSortView()
    v.camera = cam
    v.n, v.k_capacity = 5, 100
    v.splats, v.vals, v.tile_ranges, v.schedule, v.k_total = 0x1000, 0x1000, 0x1000, 0x1000, 0x1000
    v.workspace, v.workspace_bytes = 0x1004, 1 << 30
    assert L.gs_bin_sort_views(1, C.byref(v), None) == B.GS_ERR_INVALID_ARG
    assert L.gs_active_mask(0x1000, 10, 5, 0x1000, 0x1004, 1 << 20, None) == B.GS_ERR_INVALID_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library the binding raises; nothing falls back to
    another implementation."""
    import pytest
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "lib_path", lambda: str(tmp_path / "absent.so"))
    with pytest.raises(B.GsError, match="not built"):
        B.lib()


def test_peaks_library_loads_and_refuses_bad_arguments_without_device():
    """The measured-peak microbenchmarks (libgs_peaks.so) load and check their
    arguments before touching a device."""
    from gaussian_splatting_tile_amd import peaks
    L = peaks.lib()
    assert L.gsp_measure(99, 1, C.c_void_p(0x1000), 1 << 20, None) == -3.0
    assert L.gsp_measure(peaks.FMA32, 0, C.c_void_p(0x1000), 1 << 20, None) == -3.0
    assert L.gsp_measure(peaks.FMA32, 1, None, 1 << 20, None) == -3.0
