"""Benchmark of the tiled Gaussian-splatting rasterizer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload scene_1m|...]

Workload (default): 1M Gaussians, SH degree 3, fp32, the scene-like mixture
(64 anisotropic clusters + a background shell at radius 50), 1920x1080,
fx = fy = 1400, 8 orbit views; synthetic, seeded, resident in HBM before the
timed region.  One step = the whole hot path for all 8 views: the 8 views'
records in one batched projection, the 8 views' binning and depth sorts in
one batched call (one launch per sort step), the 8 forward blends in one
batched launch, then the 8
screen-space backwards against an upstream dL/dimage ~ N(0, 1e-2) in one
batched launch, and the projection's chain rule for all 8 views in one
batched pass.

Other workloads: scene_5m (5M Gaussians, same law, 1920x1080, 8 views) and
scene_10m_4k (10M Gaussians, SH stored fp16, 3840x2160, f = 2800; each step
first builds the importance mask keeping 30 % of the Gaussians by their
Exp(1) scores, and the projection applies it and the 0.5 px LOD gate).

Prints ONE JSON line: value = forward ms/frame (project + bin/sort + blend),
plus fwd+bwd ms/frame, per-call averages, the roofline of the dominant
kernel (the forward blend, one kernel per gs_render_fwd call, timed with
events on its stream), and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="scene_1m",
                    choices=["scene_1m", "scene_5m", "scene_10m_4k", "box_100k", "tiny_1k"])
    ap.add_argument("--views", type=int, default=8)
    ap.add_argument("--sort", choices=["batched", "per-view"], default="batched",
                    help="bin/sort all views in one gs_bin_sort_views call, or one gs_bin_sort per view")
    ap.add_argument("--streams", type=int, default=4,
                    help="HIP streams the views' sorts spread over (batched: one group of views per stream)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--sh-q8", action="store_true",
                    help="store SH as 8-bit codes with per-256-Gaussian bounds (quantized from the fp32 source)")
    ap.add_argument("--weights", action="store_true",
                    help="the forward blend also accumulates per-Gaussian blending weights (one array for all views)")
    ap.add_argument("--sh-adam", choices=["q8", "f32"], default=None,
                    help="each step ends with the fused SH Adam update of the SH coefficients past DC: "
                         "q8 = fp16 values with 8-bit log-domain moments, f32 = fp32 values and moments")
    ap.add_argument("--motion", action="store_true",
                    help="moving Gaussians: a motion vector and a time offset each, the views spread over the "
                         "time window (the projection and its backward displace the means)")
    ap.add_argument("--scores-from-weights", action="store_true",
                    help="workloads with an importance mask: score each Gaussian by its blending weights "
                         "summed over the views (an untimed pass before the steps) instead of the synthetic scores")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel for "
                         "calibrating the HBM byte counters of a profiler run)")
    return ap.parse_args()


# Algorithmic work of the forward blend per evaluated (pixel, Gaussian) pair,
# in fp32 VALU lane-op slots: 2 sub (offset), 5 mul/fma (quadratic form),
# v_exp_f32 (quarter rate: 4 slots), 1 mul (o * G), 1 min (cap), 1 compare
# (skip), 1 mul (alpha T), 3 fma (colour), 1 sub (T), 1 select (n_contrib),
# 1 compare (stop) = 21; taken as 20 (the select of the stop is fused).
# Pairs are counted only for list entries that can reach alpha >= 1/255 at
# some pixel centre of their tile: the others are provably skipped by every
# pixel, and the kernel drops them before the per-pixel loop.
BLEND_FWD_SLOTS_PER_PAIR = 20
# 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz: one non-packed fp32 VALU op per lane
# per clock (packed-fp32 instructions are not used by this library).
VALU_PEAK_T = 256 * 64 * 2.4e9 / 1e12
HBM_PEAK_GBPS = 8000.0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              f"see the sharding design notes", file=sys.stderr)
        sys.exit(2)

    import torch
    from gaussian_splatting_tile_amd import binding as B
    from gaussian_splatting_tile_amd import scenes

    assert torch.cuda.is_available(), "no GPU visible"
    B.lib()                         # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mib > 0:
        words = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(words, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written",
              file=sys.stderr, flush=True)
        del src, dst

    t0 = time.time()
    if args.workload == "scene_1m":
        sc = scenes.scene_like(seed=3, n=1_000_000, upstream=True, name="scene_1m_sh3_1080p")
    elif args.workload == "scene_5m":
        sc = scenes.config(4)
    elif args.workload == "scene_10m_4k":
        sc = scenes.config(5)
    elif args.workload == "box_100k":
        sc = scenes.box()
        sc.upstream_seed = 22
    else:
        sc = scenes.tiny()
        sc.upstream_seed = 11
    if args.motion:
        sc = scenes.with_motion(sc, seed=sc.n % 1000 + 7)
    views = min(args.views, len(sc.cameras))
    print(f"# scene {sc.name}: N={sc.n} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = dict(means=f(sc.means), scales=f(sc.scales), quats=f(sc.quats), opacities=f(sc.opacities),
             sh=f(sc.sh_fp16 if sc.sh_fp16 is not None else sc.sh))
    if sc.velocity is not None:
        g["velocity"], g["t_offset"] = f(sc.velocity), f(sc.t_offset)
    if args.sh_q8:
        # 8-bit block-quantized SH storage, encoded on the GPU from the fp32 source
        src = f(sc.sh)
        K_, c3_, n_ = src.shape
        g["sh"] = torch.empty((K_, c3_, n_), dtype=torch.uint8, device=dev)
        g["sh_bounds"] = torch.empty(B.sh_q8_bounds_floats(n_, K_ * c3_), dtype=torch.float32, device=dev)
        B.sh_quantize8(src, g["sh"], g["sh_bounds"])
        torch.cuda.synchronize()
        del src
    stream = torch.cuda.current_stream()
    # importance mask (a global pre-pass of every step when the workload has scores)
    use_mask = sc.importance is not None
    if use_mask:
        keep = scenes.keep_count(sc.n, sc.keep_fraction)
        scores = f(sc.importance)
        if args.scores_from_weights:
            # cross-view visibility scores: every view rendered once without
            # a mask, each Gaussian's blending weights summed over the views
            gs_all = B.gaussians_struct(g, sc.sh_degree)
            scores = torch.zeros(sc.n, dtype=torch.float32, device=dev)
            for v in range(min(args.views, len(sc.cameras))):
                probe = B.ViewBuffers(sc.n, sc.cameras[v], 16 * sc.n, with_backward=False)
                probe.forward(gs_all)
                torch.cuda.synchronize()
                k = int(probe.k_total.item())
                del probe
                vb = B.ViewBuffers(sc.n, sc.cameras[v], k, with_backward=False)
                vb.forward(gs_all)
                B.render_fwd_views([vb], (0.0, 0.0, 0.0), stream, weights=scores)
                torch.cuda.synchronize()
                del vb
            print(f"# scores from blending weights: {int((scores > 0).sum())} of {sc.n} Gaussians seen",
                  file=sys.stderr, flush=True)
        mask = torch.zeros(sc.n, dtype=torch.uint8, device=dev)
        mask_ws = torch.empty(B.active_mask_workspace_bytes(sc.n), dtype=torch.uint8, device=dev)
        B.active_mask(scores, sc.n, keep, mask, mask_ws, stream)
        gs = B.gaussians_struct(g, sc.sh_degree, mask)
    else:
        gs = B.gaussians_struct(g, sc.sh_degree)

    # per-view buffers with the exact key capacity (K is deterministic)
    bufs, Ks = [], []
    for v in range(views):
        cam = sc.cameras[v]
        probe = B.ViewBuffers(sc.n, cam, 16 * sc.n, with_backward=False)
        probe.forward(gs)
        torch.cuda.synchronize()
        k = int(probe.k_total.item())
        del probe
        b = B.ViewBuffers(sc.n, cam, k)
        b.dL = f(sc.upstream(v))
        b.bwd_ws = torch.empty(B.render_bwd_screen_workspace_bytes(k), dtype=torch.uint8, device=dev)
        b.g2 = torch.empty((sc.n, 9), dtype=torch.float32, device=dev)
        bufs.append(b)
        Ks.append(k)
    K_sh = (sc.sh_degree + 1) ** 2
    grads = dict(means=torch.zeros((3, sc.n), device=dev), log_scales=torch.zeros((3, sc.n), device=dev),
                 quats=torch.zeros((4, sc.n), device=dev), opacity_logits=torch.zeros(sc.n, device=dev),
                 sh=torch.zeros((K_sh, 3, sc.n), device=dev))
    if sc.velocity is not None:
        grads["velocity"] = torch.zeros((3, sc.n), device=dev)
        grads["t_offset"] = torch.zeros(sc.n, device=dev)
    bg = (0.0, 0.0, 0.0)
    do_bwd = not args.no_backward
    wts = torch.zeros(sc.n, dtype=torch.float32, device=dev) if args.weights else None

    # fused SH Adam over the SH rows past DC (15 coefficients x 3 channels
    # at degree 3), from a fresh state, consuming the step's SH gradients
    adam = None
    if args.sh_adam and do_bwd and K_sh > 1:
        rest = torch.from_numpy(np.ascontiguousarray(sc.sh[1:])).to(dev)
        if args.sh_adam == "q8":
            val = rest.half()
            m_st = torch.zeros(rest.shape, dtype=torch.uint8, device=dev)
            v_st = torch.zeros(rest.shape, dtype=torch.uint8, device=dev)
            nbf = B.sh_q8_bounds_floats(sc.n, (K_sh - 1) * 3)
            mb_st = torch.zeros(nbf, dtype=torch.float32, device=dev)
            vb_st = torch.zeros(nbf, dtype=torch.float32, device=dev)
        else:
            val = rest
            m_st = torch.zeros(rest.shape, dtype=torch.float32, device=dev)
            v_st = torch.zeros(rest.shape, dtype=torch.float32, device=dev)
            mb_st = vb_st = None
        adam = dict(val=val, m=m_st, v=v_st, mb=mb_st, vb=vb_st, t=0, units=(K_sh - 1) * 3 * sc.n,
                    bytes_per_unit=(12.0 + 32.0 / 256.0) if args.sh_adam == "q8" else 28.0)
        del rest

    names = ("active_mask", "project_batch", "bin_sort", "bin_sort_batch", "render_fwd_batch",
             "render_bwd_batch", "project_bwd_batch", "sh_adam")
    # the views' sorts are independent: they may run on a few streams
    # (default priority) and join before the batched blend
    side = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.streams) - 1)]
    lanes = [stream] + side
    ev = {k: [] for k in names}
    step_ev = []

    def step(record: bool):
        for gr in grads.values():
            gr.zero_()
        e_fwd0 = torch.cuda.Event(enable_timing=True)
        e_fwd1 = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        e_fwd0.record(stream)

        def timed(name, fn, st=stream):
            if not record:
                fn()
                return
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            ev[name].append((a, b))

        if use_mask:
            timed("active_mask", lambda: B.active_mask(scores, sc.n, keep, mask, mask_ws, stream))
        # the views' records in one pass over the Gaussians
        timed("project_batch", lambda: B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                                                       stream))
        go = torch.cuda.Event()
        go.record(stream)
        for st in side:
            st.wait_event(go)
        if args.sort == "batched":
            # the views split into one group per stream, each group sorted
            # by one gs_bin_sort_views call
            for i, st in enumerate(lanes):
                grp = bufs[i::len(lanes)]
                if grp:
                    timed("bin_sort_batch", lambda: B.bin_sort_views(grp, do_bwd, st), st)
        else:
            for i, b in enumerate(bufs):
                st = lanes[i % len(lanes)]
                timed("bin_sort", lambda: B.bin_sort(b.splats, b.n, b.camc, b.k_capacity, b.vals, b.ranges,
                                                     b.schedule, b.bwd_index if do_bwd else None, None,
                                                     b.k_total, b.ws, st), st)
        for st in side:
            joined = torch.cuda.Event()
            joined.record(st)
            stream.wait_event(joined)
        # the 8 views' blends share one work queue
        if wts is not None:
            wts.zero_()
        timed("render_fwd_batch", lambda: B.render_fwd_views(bufs, bg, stream, weights=wts))
        e_fwd1.record(stream)
        if do_bwd:
            # the screen-space backward of all views in one launch (plus the
            # per-view sums), then the chain rule of all views in one pass
            # over the Gaussians
            timed("render_bwd_batch", lambda: B.render_bwd_screen_views(
                bufs, [b.dL for b in bufs], [b.g2 for b in bufs], [b.bwd_ws for b in bufs], bg, stream))
            timed("project_bwd_batch", lambda: B.project_bwd(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                                                             [b.g2 for b in bufs], grads, stream))
            if adam is not None:
                adam["t"] += 1
                timed("sh_adam", lambda: B.sh_adam_step(grads["sh"][1:], adam["val"], adam["m"], adam["v"],
                                                        adam["mb"], adam["vb"], step=adam["t"], lr=1e-3,
                                                        stream=stream))
        e_end.record(stream)
        if record:
            step_ev.append((e_fwd0, e_fwd1, e_end))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"# warmup done; K per view {Ks}", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in step_ev) / (args.steps * views)
    tot_ms = sum(a.elapsed_time(c) for a, _, c in step_ev) / (args.steps * views)
    per_call = {k: (sum(a.elapsed_time(b) for a, b in v) / len(v) if v else None) for k, v in ev.items()}
    ms_per_step = wall * 1e3 / args.steps

    # algorithmic work of the blend per view, from the outputs: a pixel that
    # stopped examined n_contrib entries of its tile's list, otherwise all.
    p_eval, p_need, p_tile = [], [], []
    for b in bufs:
        pe, pn, pt = blend_pairs(torch, b)
        p_eval.append(pe)
        p_need.append(pn)
        p_tile.append(pt)
    # one forward-blend launch covers all the step's views
    t_blend_s = per_call["render_fwd_batch"] / 1e3
    achieved = sum(p_need) * BLEND_FWD_SLOTS_PER_PAIR / t_blend_s / 1e12

    cam0 = sc.cameras[0]
    res = {
        "metric": (f"ms/frame fwd (+fwd+bwd) at {sc.n / 1e6:g}M Gaussians SH{sc.sh_degree} "
                   f"{cam0.width}x{cam0.height}; % VALU / HBM peak"),
        "value": round(fwd_ms, 4),
        "unit": "ms/frame",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32 (SH stored u8 + block bounds)" if args.sh_q8 else
                  "f32" if sc.sh_fp16 is None else "f32 (SH stored f16)"),
        "data": "synthetic (seeded scene generator; no dataset)",
        "config": {"workload": sc.name, "gaussians": sc.n, "sh_degree": sc.sh_degree,
                   "width": sc.cameras[0].width, "height": sc.cameras[0].height, "views_per_step": views,
                   "importance_keep": (keep if use_mask else None),
                   "importance_scores": (None if not use_mask else
                                         "blending weights summed over the views" if args.scores_from_weights
                                         else "synthetic Exp(1)"),
                   "lod_min_radius_px": cam0.lod_min_radius_px,
                   "step": ("importance mask, then " if use_mask else "") +
                           "batched project, " +
                           ("batched bin/sort" if args.sort == "batched" else "per view bin/sort") +
                           ", batched blend fwd of all views" +
                           (" with per-Gaussian blending weights" if args.weights else "") +
                           (" (moving Gaussians, views spread over the time window)" if args.motion else "") +
                           (", then batched blend bwd of all views + one batched project bwd" if do_bwd else "") +
                           (f", then the fused SH Adam update ({args.sh_adam})" if adam is not None else "")},
        "fwd_ms_per_frame": round(fwd_ms, 4),
        "fwd_bwd_ms_per_frame": round(tot_ms, 4) if do_bwd else None,
        "per_call_ms": {k: (round(v, 4) if v is not None else None) for k, v in per_call.items()},
        "K_per_view": Ks,
        "P_eval_per_view": p_eval,
        "P_needed_per_view": p_need,
        "P_tile_per_view": p_tile,
        "roofline": {"kernel": "render_fwd_kernel (forward blend)", "bound": "alu",
                     "achieved": round(achieved, 3), "peak": round(VALU_PEAK_T, 2), "unit": "TFLOP/s",
                     "frac": round(achieved / VALU_PEAK_T, 4),
                     "traffic": measured_traffic() if args.workload == "scene_1m" else None,
                     "work_unit": f"{BLEND_FWD_SLOTS_PER_PAIR} fp32 VALU lane-op slots per evaluated "
                                  f"(pixel, Gaussian) pair whose entry can reach alpha >= 1/255 in the pixel's 16x4 strip of its tile "
                                  f"(P_needed), summed over the {views} views of one launch; "
                                  f"peak = 256 CU x 64 lanes x 2.4 GHz"},
    }
    if adam is not None:
        t_adam = per_call["sh_adam"] / 1e3
        gbps = adam["units"] * adam["bytes_per_unit"] / t_adam / 1e9
        # the measured counterpart of the spec peak: a plain 1 GiB device copy
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) / 1e3) / 1e9
        del src, dst
        res["sh_adam"] = {"kernel": "adam_q8_kernel" if args.sh_adam == "q8" else "adam_f32_kernel",
                          "state": "8-bit log-domain moments, fp16 values" if args.sh_adam == "q8"
                          else "fp32 moments and values",
                          "units": adam["units"], "ms": round(per_call["sh_adam"], 4),
                          "bytes_per_unit": adam["bytes_per_unit"], "bound": "hbm",
                          "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gbps / HBM_PEAK_GBPS, 4),
                          "measured_copy_GBps": round(copy_gbps, 1),
                          "frac_of_measured_copy": round(gbps / copy_gbps, 4),
                          "traffic": (measured_adam_traffic(args.sh_adam) if args.workload == "scene_5m"
                                      else None)}
    # the oracle is timed beside the default workload only (a 10M / 4K view
    # takes it minutes)
    if not args.no_cpu_baseline and args.workload == "scene_1m":
        res["cpu_baseline"] = cpu_baseline(sc)
    print(json.dumps(res), flush=True)


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "traffic_scene_1m_sh3_1080p.md")
ADAM_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "sh_adam_scene_5m.md")


def measured_adam_traffic(state):
    """HBM bytes per launch of the fused SH Adam kernel at 5M x 45 units
    from the rocprofv3 counter summary, or None once gs_adam.hip differs from
    the source the counters were taken on."""
    import hashlib
    try:
        lines = open(ADAM_PROFILE).read().splitlines()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in lines if l.startswith(("traffic_bytes_per_launch", "source_sha256")))
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gaussian_splatting_tile_amd", "csrc",
                       "gs_adam.hip")
    if fields.get("source_sha256 (gs_adam.hip)", "").strip() != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    v = fields.get(f"traffic_bytes_per_launch {state}")
    return int(v) if v else None
TRAFFIC_SOURCES = ("gaussian_splatting_tile_amd/csrc/gs_render.hip", "gaussian_splatting_tile_amd/csrc/gs_internal.h")


def measured_traffic():
    """HBM bytes per forward-blend launch from the committed counter summary,
    or None when the kernel source has changed since the counters were taken
    (the summary records the sources' sha256)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "source_sha256")))
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(root, f), "rb").read())
    recorded = next((v for k, v in fields.items() if k.startswith("source_sha256")), None)
    if recorded is None or recorded.strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def blend_pairs(torch, b):
    """(pairs examined under the compositing rule, pairs among them whose list
    entry can reach alpha >= 1/255 at some pixel centre of the pixel's 16x4
    strip of its tile (rows 4r .. 4r+3, the strip a wave's pixel r covers),
    the same count with the whole tile instead of the strip)."""
    cam = b.cam
    TX, TY = cam.tiles_x, cam.tiles_y
    rng = b.ranges.long()
    L = rng[:, 1] - rng[:, 0]
    K = int(L.sum().item())
    start = rng[:, 0]
    Lpix = L.reshape(TY, TX).repeat_interleave(16, 0).repeat_interleave(16, 1)[: cam.height, : cam.width]
    examined = torch.where(b.final_T < 1e-4, b.n_contrib.long(), Lpix)
    p_eval = int(examined.sum().item())
    tile = torch.repeat_interleave(torch.arange(TX * TY, device=rng.device), L)
    sp = b.splats[b.vals[:K].long()].double()
    u, v, a, bb, c, o = sp[:, 0], sp[:, 1], sp[:, 4], sp[:, 5], sp[:, 6], sp[:, 7]
    dxl = (tile % TX).double() * 16 + 0.5 - u
    dyl = (tile // TX).double() * 16 + 0.5 - v
    del sp, tile
    q = lambda dx, dy: a * dx * dx + 2 * bb * dx * dy + c * dy * dy

    def box_keep(dyb, h):
        # the minimum of the quadratic form over the box of pixel centres
        # [dxl, dxl + 15] x [dyb, dyb + h] (at the mean if inside, else on an edge)
        best = torch.full_like(u, float("inf"))
        for dx in (dxl, dxl + 15):
            best = torch.minimum(best, q(dx, torch.clamp(-bb * dx / c, dyb, dyb + h)))
        for dy in (dyb, dyb + h):
            best = torch.minimum(best, q(torch.clamp(-bb * dy / a, dxl, dxl + 15), dy))
        inside = (dxl <= 0) & (dxl + 15 >= 0) & (dyb <= 0) & (dyb + h >= 0)
        best = torch.where(inside, torch.zeros_like(best), best)
        return o * torch.exp(-0.5 * best) >= (1.0 / 255.0) * (1 - 1e-3)

    s_pix = start.reshape(TY, TX).repeat_interleave(16, 0).repeat_interleave(16, 1)[: cam.height, : cam.width]
    zero = torch.zeros(1, dtype=torch.long, device=u.device)

    def count(keep, sel=None):
        ck = torch.cat([zero, torch.cumsum(keep.long(), 0)])
        d = ck[s_pix + examined] - ck[s_pix]
        return int((d if sel is None else d * sel).sum().item())

    keep_tile = box_keep(dyl, 15)
    p_tile = count(keep_tile)
    strip = ((torch.arange(cam.height, device=u.device) % 16) // 4)[:, None].expand(cam.height, cam.width)
    p_need = 0
    for r in range(4):
        p_need += count(keep_tile & box_keep(dyl + 4 * r, 3), (strip == r).long())
    return p_eval, p_need, p_tile


def cpu_baseline(sc):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    project + bin + composite of one full view (forward), repeated while under
    ~15 s; reported in ms/frame."""
    import oracle
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    frames = 0
    while True:
        oracle.forward(sc, view=frames % len(sc.cameras))
        frames += 1
        if time.perf_counter() - t0 > 10.0 or frames >= 4:
            break
    dt = time.perf_counter() - t0
    return {"value": round(dt * 1e3 / frames, 1), "unit": "ms/frame", "cores": threads, "kind": "oracle",
            "sample": f"{frames} full forward view(s) of {sc.name} (project fp32-contract, brute-force "
                      f"binning + qsort, fp64 compositing), OpenMP"}


if __name__ == "__main__":
    main()
