"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Records (u, v, depth, radius, rect size, conic) and the bins (keys, values,
ranges, K) must be bit-exact; images within 1e-4 per channel after the
near-threshold protocol.  Every case prints its name before it touches the
GPU.
"""

import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_tile_amd import binding as B
from gaussian_splatting_tile_amd import scenes
from tests.gpu_util import (compare_bins, compare_image, compare_records, device_gaussians, run_view,
                            say, splats_np)

pytestmark = pytest.mark.gpu


def _oracle_fwd(sc, view, tile_mask=None, bg=(0.0, 0.0, 0.0), active=None, sh=None):
    cam = sc.cameras[view]
    sh = sc.sh_decoded() if sh is None else sh
    op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sh, cam, active=active)
    ob = oracle.bin_sort(op, cam)
    oo = oracle.render(op, ob, cam, bg=bg, tile_mask=tile_mask)
    return op, ob, oo


def _check_view(sc, view, name, tile_mask=None, bg=(0.0, 0.0, 0.0)):
    say(f"[gpu] {name}: N={sc.n} {sc.cameras[view].width}x{sc.cameras[view].height} view {view}")
    buf, K = run_view(sc, view, bg=bg)
    op, ob, oo = _oracle_fwd(sc, view, tile_mask=tile_mask, bg=bg)
    compare_records(splats_np(buf), op, name)
    compare_bins(buf, K, ob, name)
    st = compare_image(buf, sc.cameras[view], op, ob, oo, tile_mask=tile_mask, bg=bg)
    say(f"[gpu] {name}: K={K} P_eval={oo['p_eval']} {st}")
    assert st["unresolved"] == 0, st["details"]
    return buf, st


def test_library_loads_and_reports_version():
    assert B.lib().gs_version() >= 1
    assert torch.cuda.is_available()


def test_tiny_1k_sh0_128():
    _check_view(scenes.config(1), 0, "tiny_1k")


def test_box_100k_sh3_720p():
    _check_view(scenes.config(2), 0, "box_100k")


def test_box_with_background_colour():
    sc = scenes.config(2, n_override=20000)
    _check_view(sc, 0, "box_20k_bg", bg=(0.2, 0.5, 1.0))


@pytest.mark.parametrize("view", [0, 5])
def test_scene_1m_sh3_1080p(view):
    sc = scenes.config(3)
    _check_view(sc, view, f"scene_1m_view{view}")


def test_needle_gaussians_exponent_precision():
    """Very thin, long Gaussians (aspect ratio ~1e4) in every orientation: far
    along the major axis the exponent's terms reach ~1e5 and cancel, which
    an fp32 evaluation of the quadratic form cannot reproduce to 1e-4."""
    rng = np.random.default_rng(77)
    n = 1500
    sc = scenes.tiny(seed=77, n=n, width=512, height=384)
    sc.cameras[0].fx = sc.cameras[0].fy = 450.0
    sc.means[2] = rng.uniform(3.0, 6.0, n).astype(np.float32)
    sc.means[0:2] = rng.uniform(-2.0, 2.0, (2, n)).astype(np.float32)
    ls = np.stack([rng.uniform(-1.5, 0.0, n), np.full(n, -9.0), np.full(n, -9.0)]).astype(np.float32)
    sc.log_scales = ls
    sc.scales = np.exp(ls).astype(np.float32)
    sc.opacities = rng.uniform(0.3, 0.99, n).astype(np.float32)
    _check_view(sc, 0, "needles_1500")


def test_ragged_image_sizes():
    # widths/heights that are not multiples of 16, and a single partial tile
    for (w, h) in [(100, 37), (15, 9), (16, 16), (17, 33)]:
        sc = scenes.tiny(seed=3, n=300, width=w, height=h)
        _check_view(sc, 0, f"tiny_{w}x{h}")


def test_zero_gaussians_and_all_culled():
    sc = scenes.tiny(seed=4, n=50)
    say("[gpu] empty scene")
    empty = scenes.Scene("empty", sc.means[:, :0].copy(), sc.log_scales[:, :0].copy(), sc.scales[:, :0].copy(),
                         sc.quats[:, :0].copy(), sc.opacity_logits[:0].copy(), sc.opacities[:0].copy(), 0,
                         sc.sh[:, :, :0].copy(), sc.cameras)
    buf, K = run_view(empty, 0, k_capacity=0)
    assert K == 0
    assert torch.all(buf.image == 0) and torch.all(buf.final_T == 1) and torch.all(buf.n_contrib == 0)
    assert torch.all(buf.ranges == 0)
    say("[gpu] all behind the camera")
    behind = scenes.tiny(seed=4, n=50)
    behind.means[2] = -behind.means[2]
    buf, K = run_view(behind, 0, k_capacity=16)
    assert K == 0 and torch.all(buf.image == 0) and torch.all(buf.ranges == 0)
    assert torch.all(buf.splats == 0)


def test_capacity_overflow_reports_k_and_stays_in_bounds():
    sc = scenes.config(1, n_override=400)
    say("[gpu] capacity overflow")
    _, K = run_view(sc, 0)
    cap = K // 3
    cam = sc.cameras[0]
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, sc.sh_degree)
    buf = B.ViewBuffers(sc.n, cam, cap)
    # guard zone: the vals buffer is larger than the capacity passed in
    big = torch.full((K + 64,), -7, dtype=torch.int32, device="cuda")
    buf.vals = big
    buf.forward(gs)
    torch.cuda.synchronize()
    assert int(buf.k_total.item()) == K
    assert torch.all(big[cap:] == -7)


def test_forward_is_deterministic():
    sc = scenes.config(2, n_override=50000)
    say("[gpu] determinism")
    b1, _ = run_view(sc, 0)
    b2, _ = run_view(sc, 0)
    assert torch.equal(b1.image, b2.image) and torch.equal(b1.final_T, b2.final_T)
    assert torch.equal(b1.n_contrib, b2.n_contrib) and torch.equal(b1.vals, b2.vals)
    # the schedule's queue counters reset themselves: blending again from the
    # same schedule (three times, with a backward in between) gives the same image
    img = b1.image.clone()
    g, act, gs = b1._keep
    grads = dict(means=torch.zeros((3, sc.n), device="cuda"), log_scales=torch.zeros((3, sc.n), device="cuda"),
                 quats=torch.zeros((4, sc.n), device="cuda"), opacity_logits=torch.zeros(sc.n, device="cuda"),
                 sh=torch.zeros((16, 3, sc.n), device="cuda"))
    ws = b1.backward_workspace()
    for it in range(3):
        b1.image.zero_()
        B.render_fwd(b1.splats, b1.vals, b1.ranges, b1.schedule, b1.camc, (0.0, 0.0, 0.0), b1.image,
                     b1.final_T, b1.n_contrib)
        if it == 1:
            b1.backward(gs, torch.ones_like(b1.image), grads, ws)
        torch.cuda.synchronize()
        assert torch.equal(b1.image, img), it
    # the backward is free of atomics: a second call gives bit-identical gradients
    grads2 = {k: torch.zeros_like(v) for k, v in grads.items()}
    b1.backward(gs, torch.ones_like(b1.image), grads2, ws)
    torch.cuda.synchronize()
    for k in grads:
        assert torch.equal(grads[k], grads2[k]), k
    n_t = b1.ranges.shape[0]
    assert torch.all(b1.schedule[n_t:] == 0)
    order = b1.schedule[:n_t].cpu().numpy()
    assert np.array_equal(np.sort(order), np.arange(n_t))
    lens = (b1.ranges[:, 1] - b1.ranges[:, 0]).cpu().numpy()[order]
    # longest first, to within one ~1.4x length bucket
    assert np.all(lens[1:] <= np.maximum(lens[:-1], 1) * 1.5 + 1)


def test_invalid_arguments_are_rejected():
    sc = scenes.config(1, n_override=10)
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, 0)
    cam = B.camera_struct(sc.cameras[0])
    out = torch.empty((10, 12), device="cuda")
    bad = B.camera_struct(sc.cameras[0])
    bad.width = 0
    with pytest.raises(B.GsError, match="invalid argument"):
        B.project(gs, bad, out)
    gs4 = B.gaussians_struct(g, 0)
    gs4.sh_degree = 4
    with pytest.raises(B.GsError, match="unsupported"):
        B.project(gs4, cam, out)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.GsError, match="workspace"):
        B.bin_sort(out, 10, cam, 100, torch.empty(100, dtype=torch.int32, device="cuda"),
                   torch.empty(128, dtype=torch.int32, device="cuda"),
                   torch.empty(B.schedule_words(128, 128), dtype=torch.int32, device="cuda"), None, None,
                   torch.empty(1, dtype=torch.int64, device="cuda"), small)


def test_batched_forward_equals_per_view_calls():
    """gs_render_fwd_views over views of different sizes gives the per-view
    gs_render_fwd outputs bit for bit and leaves the queue counters reset."""
    say("[gpu] batched forward, 3 views of different sizes")
    bufs = []
    for i, (w, h) in enumerate([(640, 360), (333, 201), (512, 512)]):
        sc = scenes.scene_like(seed=30 + i, n=30_000, width=w, height=h, f=0.7 * w, n_views=1)
        buf, K = run_view(sc, 0)
        bufs.append(buf)
    ref = [(b.image.clone(), b.final_T.clone(), b.n_contrib.clone()) for b in bufs]
    for b in bufs:
        b.image.fill_(-1.0)
        b.final_T.fill_(-1.0)
        b.n_contrib.fill_(7)
    for rep in range(2):
        B.render_fwd_views(bufs, (0.0, 0.0, 0.0))
        torch.cuda.synchronize()
        for b, (img, T, nc) in zip(bufs, ref):
            assert torch.equal(b.image, img) and torch.equal(b.final_T, T) and torch.equal(b.n_contrib, nc)
        for b in bufs:
            n_t = b.ranges.shape[0]
            assert torch.all(b.schedule[n_t:] == 0)


def test_batched_projection_equals_per_view_calls():
    """gs_project_views writes, for every camera, the records gs_project writes."""
    sc = scenes.scene_like(seed=41, n=50_000, width=640, height=360, f=450.0, n_views=5)
    say("[gpu] batched projection, 5 views")
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, sc.sh_degree)
    cams = [B.camera_struct(c) for c in sc.cameras]
    outs = [torch.full((sc.n, 12), -1.0, device="cuda") for _ in cams]
    B.project_views(gs, cams, outs)
    torch.cuda.synchronize()
    for cam, out in zip(cams, outs):
        ref = torch.empty((sc.n, 12), device="cuda")
        B.project(gs, cam, ref)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def _bins_of(buf, K):
    """The defined parts of a view's binning outputs, as host arrays."""
    n, cap = buf.n, buf.k_capacity
    bi = buf.bwd_index.cpu().numpy().view(np.uint32)
    n_vis = int(bi[cap + 2 * n + 1])
    out = {"K": int(buf.k_total.item()), "vals": buf.vals[:K].cpu().numpy().copy(),
           "ranges": buf.ranges.cpu().numpy().copy(), "slots": bi[:K].copy(),
           "order": bi[cap:cap + n_vis].copy(), "off": bi[cap + n:cap + n + n_vis + 1].copy(), "n_vis": n_vis}
    if buf.keys is not None:
        out["keys"] = buf.keys[:K].cpu().numpy().copy()
    sched = buf.schedule.cpu().numpy().view(np.uint32)
    n_t = buf.ranges.shape[0]
    assert np.array_equal(np.sort(sched[:n_t]), np.arange(n_t)) and np.all(sched[n_t:] == 0)
    return out


def test_batched_sort_equals_per_view_calls():
    """gs_bin_sort_views over five views of different sizes and resolutions
    (one of a single tile, one without Gaussians) writes what five
    gs_bin_sort calls write, and the oracle's bins."""
    specs = [(640, 360, 30_000), (333, 201, 20_000), (15, 9, 500), (512, 512, 25_000), (64, 64, 0)]
    bufs, ref, Ks = [], [], []
    for i, (w, h, n) in enumerate(specs):
        say(f"[gpu] batched sort: view {i} {w}x{h} N={n} (per-view call)")
        if n == 0:
            t = scenes.tiny(seed=4, n=50, width=w, height=h)
            sc = scenes.Scene("empty", t.means[:, :0].copy(), t.log_scales[:, :0].copy(), t.scales[:, :0].copy(),
                              t.quats[:, :0].copy(), t.opacity_logits[:0].copy(), t.opacities[:0].copy(), 0,
                              t.sh[:, :, :0].copy(), t.cameras)
            buf, K = run_view(sc, 0, k_capacity=0)
        else:
            sc = scenes.scene_like(seed=50 + i, n=n, width=w, height=h, f=0.7 * w, n_views=1)
            buf, K = run_view(sc, 0)
            op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sc.sh, sc.cameras[0])
            compare_bins(buf, K, oracle.bin_sort(op, sc.cameras[0]), f"view {i}")
        bufs.append(buf)
        Ks.append(K)
        ref.append(_bins_of(buf, K))
        if n == 0:
            assert K == 0 and ref[-1]["n_vis"] == 0 and list(ref[-1]["off"]) == [0]
    for rep in range(2):
        say(f"[gpu] batched sort: gs_bin_sort_views over {len(bufs)} views, call {rep}")
        for b in bufs:
            b.vals.fill_(-1)
            b.ranges.fill_(-1)
            b.bwd_index.fill_(-1)
            b.schedule.fill_(-1)
            b.k_total.fill_(-1)
            if b.keys is not None:
                b.keys.fill_(-1)
        B.bin_sort_views(bufs, True)
        torch.cuda.synchronize()
        for i, (b, K, r) in enumerate(zip(bufs, Ks, ref)):
            got = _bins_of(b, K)
            for key in r:
                assert np.array_equal(np.asarray(got[key]), np.asarray(r[key])), f"view {i}: {key} differs"



def test_binned_projection_feeds_the_sort():
    """gs_project_views_binned writes the records of gs_project_views plus
    each view's depth keys and tile rects, and gs_bin_sort_views fed with
    them (all views, or some) writes the bins of the plain calls, bit for
    bit: four views of one scene, one of them a single tile."""
    import dataclasses
    sc = scenes.scene_like(seed=45, n=40_000, width=640, height=360, f=450.0, n_views=4)
    sc.cameras[3] = dataclasses.replace(sc.cameras[3], width=15, height=9, cx=7.5, cy=4.5)
    say("[gpu] binned projection: per-view references, 4 views")
    refs, bufs = [], []
    for v in range(4):
        buf, K = run_view(sc, v)
        refs.append((buf.splats.clone(), _bins_of(buf, K), K))
        bufs.append(buf)
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, sc.sh_degree)
    for rep, pre in enumerate((True, [True, False, True, False])):
        say(f"[gpu] binned projection + sort, call {rep} (prebinned {pre})")
        for b in bufs:
            for t in (b.splats, b.vals, b.ranges, b.bwd_index, b.schedule, b.k_total, b.keys, b.depth_keys,
                      b.tile_rects):
                t.fill_(-1)
        B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs], bin_keys=[b.bin_keys for b in bufs])
        torch.cuda.synchronize()
        for i, (b, (rec, _, _)) in enumerate(zip(bufs, refs)):
            assert torch.equal(b.splats.view(torch.int32), rec.view(torch.int32)), f"view {i}: records"
            tiles = rec[:, 11].view(torch.int32).cpu().numpy().view(np.uint32)
            depth = rec[:, 2].contiguous().view(torch.int32).cpu().numpy().view(np.uint32)
            dk = b.depth_keys.cpu().numpy().view(np.uint32)
            gr = b.tile_rects.view(-1, 2).cpu().numpy().view(np.uint32)
            vis = tiles > 0
            assert np.array_equal(dk[vis], depth[vis]) and np.all(dk[~vis] == 0xFFFFFFFF), f"view {i}: keys"
            assert np.all(gr[~vis] == 0), f"view {i}: culled rects"
            w, h = gr[:, 1] & 0xFFFF, gr[:, 1] >> 16
            assert np.array_equal((w * h)[vis], tiles[vis]), f"view {i}: rect sizes"
            x0, y0 = gr[:, 0] & 0xFFFF, gr[:, 0] >> 16
            assert np.all(x0[vis] + w[vis] <= b.cam.tiles_x) and np.all(y0[vis] + h[vis] <= b.cam.tiles_y)
        B.bin_sort_views(bufs, True, prebinned=pre)
        torch.cuda.synchronize()
        for i, (b, (_, r, K)) in enumerate(zip(bufs, refs)):
            got = _bins_of(b, K)
            for key in r:
                assert np.array_equal(np.asarray(got[key]), np.asarray(r[key])), f"view {i}: {key} differs"


def _pairs(vals, ranges):
    """(tile, Gaussian) pairs of a binning, as a set."""
    out = set()
    for t, (a, b) in enumerate(np.asarray(ranges).reshape(-1, 2)):
        out.update((t, int(g)) for g in vals[a:b])
    return out


def test_reach_binning_matches_oracle_and_leaves_results_unchanged():
    """Lists restricted to the tiles each Gaussian reaches (gs_sort_view
    .reach_tiles): bins equal the oracle's reach binning (a pair may differ
    only within 1e-5 of the reach bound, where fp32 and fp64 can decide
    apart); the blend over them writes the images and final_T of the full
    lists bit for bit, each pixel's last composited entry is the same
    Gaussian, and the backward's per-Gaussian sums are the same.  Three
    views, the projection writing the sort keys for two of them."""
    sc = scenes.scene_like(seed=47, n=40_000, width=640, height=360, f=450.0, n_views=3, upstream=True)
    # some large Gaussians: rects of 17-32 tiles are tested by a whole wave in
    # the slot scan, rects past 32 tiles also in the duplication's second pass
    big = np.random.default_rng(48).choice(sc.n, 300, replace=False)
    sc.scales = sc.scales.copy()
    sc.scales[:, big] *= np.float32(12.0)
    sc.log_scales = np.log(sc.scales).astype(np.float32)
    thr = (1.0 / 255.0) * (1.0 - 1e-3)
    say("[gpu] reach binning: full-list references, 3 views")
    full, reach = [], []
    for v in range(3):
        buf, K = run_view(sc, v)
        full.append((buf, K))
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, sc.sh_degree)
    bufs = [B.ViewBuffers(sc.n, sc.cameras[v], full[v][1], with_keys=True) for v in range(3)]
    say("[gpu] reach binning: batched projection + sort with reach_tiles")
    # view 0's projection writes depth keys only (a reach sort needs no rects)
    B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                    bin_keys=[(b.depth_keys, None) if v == 0 else b.bin_keys for v, b in enumerate(bufs)])
    B.bin_sort_views(bufs, True, prebinned=[True, False, True], reach=True)
    torch.cuda.synchronize()
    for v, b in enumerate(bufs):
        cam = sc.cameras[v]
        op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sc.sh, cam)
        ob = oracle.bin_sort(op, cam, reach=True)
        K = int(b.k_total.item())
        assert K < full[v][1]
        assert int((op["tiles"] > 32).sum()) > 20 and int(((op["tiles"] > 16) & (op["tiles"] <= 32)).sum()) > 20
        vals = b.vals[:K].cpu().numpy().view(np.uint32)
        ranges = b.ranges.cpu().numpy().view(np.uint32)
        diff = _pairs(vals, ranges) ^ _pairs(ob["vals"], ob["ranges"])
        for t, gi in diff:
            assert abs(oracle.tile_reach(op, gi, t, cam) / thr - 1.0) < 1e-5, f"view {v}: pair ({t}, {gi})"
        if not diff:
            assert K == ob["K"] and np.array_equal(vals, ob["vals"])
            assert np.array_equal(ranges.reshape(-1), ob["ranges"].reshape(-1))
            assert np.array_equal(b.keys[:K].cpu().numpy().view(np.uint64), ob["keys"])
        # backward index: the depth-ordered Gaussians' first slots partition [0, K)
        bi = b.bwd_index.cpu().numpy().view(np.uint32)
        n, cap = b.n, b.k_capacity
        n_vis = int(bi[cap + 2 * n + 1])
        off = bi[cap + n:cap + n + n_vis + 1].astype(np.int64)
        assert off[0] == 0 and off[-1] == K and np.all(np.diff(off) >= 0)
        order = bi[cap:cap + n_vis]
        slot_g = np.repeat(order, np.diff(off))
        assert np.array_equal(np.sort(vals), np.sort(slot_g))
        assert np.array_equal(slot_g[bi[:K]], vals)              # each entry's slot belongs to its Gaussian
    say("[gpu] reach binning: blend forward over reach and full lists")
    B.render_fwd_views(bufs, (0.1, 0.2, 0.3))
    for fb, _ in full:
        fb.n_contrib.zero_()
    B.render_fwd_views([fb for fb, _ in full], (0.1, 0.2, 0.3))
    torch.cuda.synchronize()
    for v, (b, (fb, _)) in enumerate(zip(bufs, full)):
        assert torch.equal(b.image, fb.image) and torch.equal(b.final_T, fb.final_T), f"view {v}"
        nr, nf = b.n_contrib.long(), fb.n_contrib.long()
        assert torch.equal(nr == 0, nf == 0) and bool((nr <= nf).all())
        H, W = nr.shape
        tile = ((torch.arange(H, device="cuda") // 16)[:, None] * b.cam.tiles_x +
                (torch.arange(W, device="cuda") // 16)[None, :]).long()
        has = nf > 0
        gr = b.vals.long()[b.ranges.long()[:, 0][tile] + nr - 1][has]
        gf = fb.vals.long()[fb.ranges.long()[:, 0][tile] + nf - 1][has]
        assert torch.equal(gr, gf), f"view {v}: last composited entry"
    say("[gpu] reach binning: blend backward sums over reach and full lists")
    dLs = [torch.from_numpy(np.ascontiguousarray(sc.upstream(v))).cuda() for v in range(3)]
    g2r = [torch.full((sc.n, 9), float("nan"), device="cuda") for _ in range(3)]
    g2f = [torch.full((sc.n, 9), float("nan"), device="cuda") for _ in range(3)]
    wsr = [torch.empty(B.render_bwd_screen_workspace_bytes(b.k_capacity), dtype=torch.uint8, device="cuda")
           for b in bufs]
    wsf = [torch.empty(B.render_bwd_screen_workspace_bytes(fb.k_capacity), dtype=torch.uint8, device="cuda")
           for fb, _ in full]
    B.render_bwd_screen_views(bufs, dLs, g2r, wsr, (0.1, 0.2, 0.3))
    B.render_bwd_screen_views([fb for fb, _ in full], dLs, g2f, wsf, (0.1, 0.2, 0.3))
    torch.cuda.synchronize()
    for v in range(3):
        vis = bufs[v].splats[:, 11].view(torch.int32) != 0
        assert torch.equal(g2r[v][vis], g2f[v][vis]), f"view {v}: screen-space sums"


def test_binned_projection_under_a_mask_leaves_inactive_records_unwritten():
    """With an importance mask, gs_project_views_binned writes no record of a
    Gaussian outside the mask (the sort takes visibility from the depth keys)
    and every other record as the plain projection does; the prebinned reach
    sort, the blend and the backward over those records equal the plain
    path's bit for bit."""
    sc = scenes.scene_like(seed=53, n=30_000, width=480, height=272, f=350.0, n_views=2, upstream=True)
    active = (np.random.default_rng(54).random(sc.n) < 0.4).astype(np.uint8)
    g = device_gaussians(sc)
    act = torch.from_numpy(active).cuda()
    gs = B.gaussians_struct(g, sc.sh_degree, act)
    say("[gpu] masked binned projection: plain references, 2 views")
    ref = []
    for v in range(2):
        buf, K = run_view(sc, v, active=active)
        ref.append(buf)
    bufs = [B.ViewBuffers(sc.n, sc.cameras[v], ref[v].k_capacity, with_keys=True) for v in range(2)]
    for b in bufs:
        b.splats.fill_(-1.0)
    say("[gpu] masked binned projection: binned path")
    B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                    bin_keys=[(b.depth_keys, None) for b in bufs])
    plain = [torch.empty_like(b.splats) for b in bufs]
    B.project_views(gs, [b.camc for b in bufs], plain)
    torch.cuda.synchronize()
    inactive = torch.from_numpy(active == 0).cuda()
    for b, p in zip(bufs, plain):
        assert bool((b.splats[inactive] == -1.0).all())
        assert torch.equal(b.splats[~inactive].view(torch.int32), p[~inactive].view(torch.int32))
    # reach sorts of the plain records as the reference lists
    for r, p in zip(ref, plain):
        r.splats.copy_(p)
    B.bin_sort_views(ref, True, reach=True)
    B.bin_sort_views(bufs, True, prebinned=True, reach=True)
    B.render_fwd_views(ref, (0.0, 0.0, 0.0))
    B.render_fwd_views(bufs, (0.0, 0.0, 0.0))
    torch.cuda.synchronize()
    for r, b in zip(ref, bufs):
        K = int(r.k_total.item())
        assert int(b.k_total.item()) == K and torch.equal(r.vals[:K], b.vals[:K]) and torch.equal(r.ranges, b.ranges)
        assert torch.equal(r.image, b.image) and torch.equal(r.final_T, b.final_T)
        assert torch.equal(r.n_contrib, b.n_contrib)
    say("[gpu] masked binned projection: backward (records, then the depth keys for visibility)")
    dLs = [torch.from_numpy(np.ascontiguousarray(sc.upstream(v))).cuda() for v in range(2)]
    out = []
    for set_, keys in ((ref, None), (bufs, None), (bufs, [b.depth_keys for b in bufs]),
                       (bufs, [bufs[0].depth_keys, None])):
        out.append(_screen_and_projection_backward(sc, gs, set_, dLs, keys))
    for o in out[1:]:
        for k in out[0]:
            assert torch.equal(out[0][k], o[k]), k


def _screen_and_projection_backward(sc, gs, bufs, dLs, depth_keys):
    g2s = [torch.empty((sc.n, 9), device="cuda") for _ in bufs]
    wss = [torch.empty(B.render_bwd_screen_workspace_bytes(b.k_capacity), dtype=torch.uint8, device="cuda")
           for b in bufs]
    B.render_bwd_screen_views(bufs, dLs, g2s, wss)
    grads = dict(means=torch.zeros((3, sc.n), device="cuda"), log_scales=torch.zeros((3, sc.n), device="cuda"),
                 quats=torch.zeros((4, sc.n), device="cuda"), opacity_logits=torch.zeros(sc.n, device="cuda"),
                 sh=torch.zeros((sc.sh.shape[0], 3, sc.n), device="cuda"))
    B.project_bwd(gs, [b.camc for b in bufs], [b.splats for b in bufs], g2s, grads, depth_keys=depth_keys)
    torch.cuda.synchronize()
    return grads


def test_projection_backward_with_depth_key_visibility_equals_record_visibility():
    """gs_project_bwd_binned, which reads each view's visibility from the
    projection's depth keys, gives the gradients of gs_project_bwd (radius
    from the records) bit for bit: all views keyed, and one view keyed with
    the other read from its records."""
    sc = scenes.scene_like(seed=57, n=30_000, width=480, height=272, f=350.0, n_views=3, upstream=True)
    g = device_gaussians(sc)
    gs = B.gaussians_struct(g, sc.sh_degree)
    say("[gpu] projection backward with depth-key visibility, 3 views")
    probe = [run_view(sc, v)[0] for v in range(3)]
    bufs = [B.ViewBuffers(sc.n, sc.cameras[v], probe[v].k_capacity, with_keys=True) for v in range(3)]
    B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                    bin_keys=[(b.depth_keys, None) for b in bufs])
    B.bin_sort_views(bufs, True, prebinned=True, reach=True)
    B.render_fwd_views(bufs, (0.0, 0.0, 0.0))
    torch.cuda.synchronize()
    for b in bufs:
        seen = b.depth_keys[: sc.n] != -1
        assert torch.equal(seen, b.splats[:, 3].view(torch.int32) != 0)
    dLs = [torch.from_numpy(np.ascontiguousarray(sc.upstream(v))).cuda() for v in range(3)]
    out = [_screen_and_projection_backward(sc, gs, bufs, dLs, keys)
           for keys in (None, [b.depth_keys for b in bufs], [None, bufs[1].depth_keys, None])]
    for o in out[1:]:
        for k in out[0]:
            assert torch.equal(out[0][k], o[k]), k


def _ambiguous_gaussians(ob, oo, cam):
    """Gaussians listed in a tile that holds a pixel with a near-threshold
    decision (or an alpha near the cap): their weights may legitimately
    differ between two correct forwards."""
    amb = (oo["events"] > 0) | (oo["capflag"] > 0)
    ty, tx = np.nonzero(amb)
    tiles = np.unique((ty // 16) * cam.tiles_x + tx // 16)
    out = np.zeros(0, np.int64)
    for t in tiles:
        s, e = ob["ranges"][t]
        out = np.concatenate([out, ob["vals"][s:e].astype(np.int64)])
    return np.unique(out)


def _compare_weights(gpu, ref, skip, name):
    keep = np.ones(ref.shape[0], bool)
    keep[skip] = False
    err = np.abs(gpu - ref)
    tol = 1e-4 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    bad = int(np.count_nonzero((err > tol) & keep))
    say(f"[gpu] {name}: compared {int(keep.sum())} of {ref.shape[0]} Gaussians, "
        f"max rel err {float((err[keep] / np.maximum(np.abs(ref[keep]), 1e-30)).max()):.2e}, bad {bad}")
    assert bad == 0
    assert np.all(gpu[ref == 0.0] == 0.0)             # culled or never composited: nothing added


def test_blend_weights_match_oracle():
    """The per-Gaussian blending weights of gs_render_fwd_views (sum over the
    view's pixels of alpha_i T_i) against the oracle's: one 720p view, then
    three views of another scene adding into one shared array."""
    sc = scenes.config(2)
    say("[gpu] blend weights: box_100k view 0")
    buf, K = run_view(sc, 0)
    op, ob, oo = _oracle_fwd(sc, 0)
    ref = oracle.render(op, ob, sc.cameras[0], weight=True)["weight"]
    w = torch.zeros(sc.n, dtype=torch.float32, device="cuda")
    B.render_fwd_views([buf], (0.0, 0.0, 0.0), weights=w)
    torch.cuda.synchronize()
    _compare_weights(w.cpu().numpy().astype(np.float64), ref, _ambiguous_gaussians(ob, oo, sc.cameras[0]),
                     "weights box_100k")

    sc = scenes.scene_like(seed=61, n=30_000, width=480, height=272, f=350.0, n_views=3)
    say("[gpu] blend weights: 3 views into one array")
    bufs, ref, skip = [], np.zeros(sc.n), []
    for v in range(3):
        b, K = run_view(sc, v)
        bufs.append(b)
        op, ob, oo = _oracle_fwd(sc, v)
        ref += oracle.render(op, ob, sc.cameras[v], weight=True)["weight"]
        skip.append(_ambiguous_gaussians(ob, oo, sc.cameras[v]))
    w = torch.zeros(sc.n, dtype=torch.float32, device="cuda")
    B.render_fwd_views(bufs, (0.0, 0.0, 0.0), weights=w)
    torch.cuda.synchronize()
    _compare_weights(w.cpu().numpy().astype(np.float64), ref, np.concatenate(skip), "weights 3 views")
    # the images are those of the forward without weights
    img = [b.image.clone() for b in bufs]
    B.render_fwd_views(bufs, (0.0, 0.0, 0.0))
    torch.cuda.synchronize()
    for b, i0 in zip(bufs, img):
        assert torch.equal(b.image, i0)
