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

Each step copies the views' key counts to pinned host memory after the sort,
without waiting for them (every kernel clamps K to the view's capacity, so a
step that overflowed is memory-safe and would be run again with larger
buffers); the host checks every step's K against the key capacities, which
are sized once with 25 % headroom over a probe pass, when the steps are done,
as a training loop that never stalls on the host would.  Steps are timed warm
(back to back) and cold (a 2 GiB device copy before each step scrubs the
256 MB last-level cache and the L2).

Prints ONE JSON line: value = median warm forward ms/frame (project +
bin/sort + K copy + blend), plus p90 and the cold figures, fwd+bwd
ms/frame, per-call medians, the rooflines of the two blend kernels (VALU lane
slots against the chip's published rate and against the rate measured on the
same GPU by csrc/peaks.hip), the HBM fractions of the projection, the sort
and the projection backward, and the CPU oracle timed on a bounded sample
(all cores and one core).
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
    ap.add_argument("--tile-lists", choices=["reach", "rect"], default="reach",
                    help="batched sort only: list each Gaussian in the tiles it reaches (alpha >= 1/255 possible "
                         "at a pixel centre; same images and gradients), or in every tile of its 3-sigma rect")
    ap.add_argument("--bin-keys", choices=["projection", "sort"], default="projection",
                    help="batched sort only: each view's depth keys and tile rects written by the projection "
                         "(gs_project_views_binned), or read back from the records by the sort")
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
    ap.add_argument("--cold-steps", type=int, default=None,
                    help="steps timed after a cache scrub each (default: --steps; 0 skips them)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel for "
                         "calibrating the HBM byte counters of a profiler run)")
    return ap.parse_args()


# Algorithmic work of the forward blend per (pixel, Gaussian) pair, in VALU
# lane-op slots (one slot = one non-packed lane operation of a full-rate
# instruction): 2 sub (offset), 5 mul/fma (quadratic form), 1 mul (o * G),
# 1 min (cap), 1 compare (skip), 1 mul (alpha T), 3 fma (colour), 1 sub (T),
# 1 select (n_contrib) = 16, plus v_exp_f32 at its measured cost of 2 slots
# (half rate on this chip: csrc/peaks.hip) = 18.  Pairs are counted only for
# list entries that can reach alpha >= 1/255 somewhere in the pixel's 16x4
# strip of its tile (P_needed): the others are provably skipped by every
# such pixel, and the kernel drops them before the per-pixel loop.
BLEND_FWD_SLOTS_PER_PAIR = 18
# The backward per composited pair: ~45 lane ops of reverse compositing
# (transmittance recovery, colour and alpha gradients, the power's partials
# and the covariance sums) plus v_exp_f32 and v_rcp_f32 at 2 slots each = 49.
BLEND_BWD_SLOTS_PER_PAIR = 49
# 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz: one non-packed fp32 (or fp64) FMA
# per lane per clock (packed-fp32 instructions are not used by this library).
VALU_PEAK_T = 256 * 64 * 2.4e9 / 1e12
HBM_PEAK_GBPS = 8000.0
CAPACITY_HEADROOM = 1.25


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

    # the GPU's own peak rates (csrc/peaks.hip): fp32/fp64 FMA, exp, LDS, copy
    peaks_measured = None
    if not args.no_peaks:
        from gaussian_splatting_tile_amd import peaks
        peaks_measured = peaks.measure(torch, dev)
        torch.cuda.synchronize()

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

    # the projection writes the sort's keys; lists hold the tiles each
    # Gaussian reaches (both with the batched sort)
    prebinned = args.sort == "batched" and args.bin_keys == "projection"
    reach = args.sort == "batched" and args.tile_lists == "reach"
    # per-view buffers: key capacity = 25 % over a probe pass (rounded up to
    # 1024); every step reads the true K back and checks it
    k_all = torch.zeros(views, dtype=torch.int64, device=dev)
    bufs, Ks, caps = [], [], []
    for v in range(views):
        cam = sc.cameras[v]
        probe = B.ViewBuffers(sc.n, cam, 16 * sc.n, with_backward=False)
        B.project(gs, probe.camc, probe.splats)
        B.bin_sort_views([probe], False, reach=reach)
        torch.cuda.synchronize()
        k = int(probe.k_total.item())
        del probe
        cap = int(math.ceil(k * CAPACITY_HEADROOM / 1024.0)) * 1024
        b = B.ViewBuffers(sc.n, cam, cap)
        b.k_total = k_all[v:v + 1]
        b.dL = f(sc.upstream(v))
        b.bwd_ws = torch.empty(B.render_bwd_screen_workspace_bytes(cap), dtype=torch.uint8, device=dev)
        b.g2 = torch.empty((sc.n, 9), dtype=torch.float32, device=dev)
        bufs.append(b)
        Ks.append(k)
        caps.append(cap)
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
    # the copy of K to the host runs beside the blends (the step's end waits for it)
    copy_stream = torch.cuda.Stream(device=dev)
    # a 2 GiB device copy (1 GiB read + 1 GiB written) before each cold step
    # pushes the step's inputs out of the 256 MB last-level cache and the L2
    n_cold = args.steps if args.cold_steps is None else args.cold_steps
    scrub = (torch.empty(1 << 28, dtype=torch.float32, device=dev),
             torch.empty(1 << 28, dtype=torch.float32, device=dev)) if n_cold > 0 else None
    # warm and cold steps carry only the step's own events; the per-call
    # events (two more per call) sit in a separate run of "calls" steps, so
    # the headline steps do not pay for them
    rec = {m: dict(ev={k: [] for k in names}, steps=[]) for m in ("warm", "calls", "cold")}
    # one pinned row of K per step run (warm-up, timed, per-call and cold steps)
    k_ring = torch.zeros((args.warmup + 2 * args.steps + n_cold, views), dtype=torch.int64).pin_memory()
    n_run = [0]

    def step(mode):
        for gr in grads.values():
            gr.zero_()
        if mode == "cold":
            scrub[1].copy_(scrub[0])
        R = rec[mode] if mode else None
        E = lambda: torch.cuda.Event(enable_timing=True)
        e_fwd0, e_sort0, e_sort1, e_fwd1, e_end = E(), E(), E(), E(), E()
        e_fwd0.record(stream)

        def timed(name, fn, st=stream):
            if mode != "calls":
                fn()
                return
            a, b = E(), E()
            a.record(st)
            fn()
            b.record(st)
            R["ev"][name].append((a, b))

        if use_mask:
            timed("active_mask", lambda: B.active_mask(scores, sc.n, keep, mask, mask_ws, stream))
        # the views' records in one pass over the Gaussians
        timed("project_batch", lambda: B.project_views(gs, [b.camc for b in bufs], [b.splats for b in bufs],
                                                       stream, bin_keys=[(b.depth_keys, None if reach else b.tile_rects)
                                                                         for b in bufs] if prebinned else None))
        e_sort0.record(stream)
        for st in side:
            st.wait_event(e_sort0)
        if args.sort == "batched":
            # the views split into one group per stream, each group sorted
            # by one gs_bin_sort_views call
            for i, st in enumerate(lanes):
                grp = bufs[i::len(lanes)]
                if grp:
                    timed("bin_sort_batch", lambda: B.bin_sort_views(grp, do_bwd, st, prebinned=prebinned,
                                                                     reach=reach), st)
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
        e_sort1.record(stream)
        # K of every view back to the host, without waiting for it: every
        # kernel clamps K to the view's capacity, so a step whose K passed a
        # capacity is memory-safe and only has to be run again with larger
        # buffers; the host checks each step's K once the steps are done
        copy_stream.wait_event(e_sort1)
        with torch.cuda.stream(copy_stream):
            k_ring[n_run[0]].copy_(k_all, non_blocking=True)
        e_copied = torch.cuda.Event()
        e_copied.record(copy_stream)
        n_run[0] += 1
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
                                                             [b.g2 for b in bufs], grads, stream,
                                                             depth_keys=[b.depth_keys for b in bufs]
                                                             if prebinned else None))
            if adam is not None:
                adam["t"] += 1
                timed("sh_adam", lambda: B.sh_adam_step(grads["sh"][1:], adam["val"], adam["m"], adam["v"],
                                                        adam["mb"], adam["vb"], step=adam["t"], lr=1e-3,
                                                        stream=stream))
        stream.wait_event(e_copied)
        e_end.record(stream)
        if R is not None:
            R["steps"].append((e_fwd0, e_sort0, e_sort1, e_fwd1, e_end))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print(f"# warmup done; K per view {Ks}", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step("warm")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for _ in range(args.steps):
        step("calls")
    torch.cuda.synchronize()
    for _ in range(n_cold):
        step("cold")
    torch.cuda.synchronize()
    del scrub
    # every step's K: within its capacity, and the K the probes measured
    for row in k_ring[:n_run[0]].tolist():
        if any(k > c for k, c in zip(row, caps)):
            raise RuntimeError(f"key capacity exceeded: K {row} capacities {caps}")
        if row != Ks:
            raise RuntimeError(f"K changed between passes: {row} vs {Ks}")
    ms_per_step = wall * 1e3 / args.steps
    print(f"# timed {args.steps} warm, {args.steps} per-call and {n_cold} cold steps", file=sys.stderr, flush=True)

    def stats(xs):
        if not xs:
            return None
        a = np.sort(np.asarray(xs, dtype=np.float64))
        return dict(median=round(float(np.median(a)), 4), p90=round(float(np.percentile(a, 90)), 4),
                    mean=round(float(a.mean()), 4))

    def summary(R):
        st = R["steps"]
        if not st:
            return None
        fwd = [a.elapsed_time(d) / views for a, _, _, d, _ in st]
        tot = [a.elapsed_time(e) / views for a, _, _, _, e in st]
        sort = [b.elapsed_time(c) for _, b, c, _, _ in st]
        calls = {k: stats([a.elapsed_time(b) for a, b in v]) for k, v in R["ev"].items()}
        out = dict(fwd_ms_per_frame=stats(fwd), fwd_bwd_ms_per_frame=stats(tot) if do_bwd else None,
                   sort_phase_ms=stats(sort))
        calls = {k: v for k, v in calls.items() if v is not None}
        if calls:
            out["per_call_ms"] = calls
        return out

    warm, calls, cold = summary(rec["warm"]), summary(rec["calls"]), summary(rec["cold"])
    fwd_ms = warm["fwd_ms_per_frame"]["median"]
    tot_ms = warm["fwd_bwd_ms_per_frame"]["median"] if do_bwd else None
    med = lambda k: calls["per_call_ms"][k]["median"] if k in calls["per_call_ms"] else None

    # algorithmic work of the blends per view, from the outputs (untimed)
    counts = [blend_pairs(torch, b) for b in bufs]
    p_eval = [c["eval"] for c in counts]
    p_need = [c["needed"] for c in counts]
    p_tile = [c["tile"] for c in counts]
    p_comp = [c["composited"] for c in counts]
    p_bwd = [c["bwd_examined"] for c in counts]
    vis = torch.zeros(sc.n, dtype=torch.bool, device=dev)
    n_vis = []
    for b in bufs:
        r = b.splats[: sc.n, 3].view(torch.int32) > 0
        n_vis.append(int(r.sum().item()))
        vis |= r
    n_any = int(vis.sum().item())
    del vis
    fma_meas = peaks_measured["fma32"] / 1e12 if peaks_measured else None
    copy_meas = peaks_measured["copy"] / 1e9 if peaks_measured else None

    def valu_roofline(kernel, pairs, slots, ms, note):
        ach = sum(pairs) * slots / (ms / 1e3) / 1e12
        out = {"kernel": kernel, "bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_T, 2),
               "unit": "Tslot/s", "frac": round(ach / VALU_PEAK_T, 4)}
        if fma_meas:
            out["peak_measured"] = round(fma_meas, 2)
            out["frac_measured"] = round(ach / fma_meas, 4)
        out["work_unit"] = note
        return out

    roof_fwd = valu_roofline(
        "render_fwd_kernel (forward blend)", p_need, BLEND_FWD_SLOTS_PER_PAIR, med("render_fwd_batch"),
        f"{BLEND_FWD_SLOTS_PER_PAIR} VALU lane-op slots per (pixel, Gaussian) pair whose entry can reach "
        f"alpha >= 1/255 in the pixel's 16x4 strip of its tile (P_needed), summed over the {views} views of one "
        f"launch, over the launch's median event-timed duration; a slot is one lane of a full-rate non-packed "
        f"VALU instruction (v_exp_f32, half rate, counts 2); peak = 256 CU x 64 lanes x 2.4 GHz, "
        f"peak_measured = non-packed fp32 FMA rate measured on this GPU")
    roof_fwd["traffic"] = measured_traffic() if args.workload == "scene_1m" else None
    roof_bwd = None
    if do_bwd:
        roof_bwd = valu_roofline(
            "render_bwd_kernel + sum_partials_kernel (one gs_render_bwd_screen_views call)", p_comp,
            BLEND_BWD_SLOTS_PER_PAIR, med("render_bwd_batch"),
            f"{BLEND_BWD_SLOTS_PER_PAIR} VALU lane-op slots per composited (pixel, Gaussian) pair (alpha >= 1/255 "
            f"before the pixel's last composited entry), summed over the {views} views, over the call's median "
            f"duration (the blend backward and the per-Gaussian sums of its partial rows)")

    # algorithmic HBM bytes of the memory-bound stages (what the method must
    # move once for the step's views: parameters and SH read once per batch,
    # one record per view written, gradients read-modified-written once)
    sh_b = {"f32": 12, "f16": 6, "q8": 3}["q8" if args.sh_q8 else ("f16" if sc.sh_fp16 is not None else "f32")]
    sh_bytes = sh_b * K_sh + (8.0 * 3 * K_sh / 256.0 if args.sh_q8 else 0.0)
    geo = 44 + (16 if sc.velocity is not None else 0)
    # + depth key (and tile rect, unless only reached tiles are listed) when
    # the projection writes them
    rec_b = 48 + ((4 if reach else 12) if prebinned else 0)
    bytes_proj = sc.n * geo + (sc.n if use_mask else 0) + views * sc.n * rec_b + n_any * sh_bytes
    # the sort: what this design must move once (depth digits on the visible
    # Gaussians, then the tile digits on the K keys): per Gaussian 20 B of its
    # record read and 12 B of depth key and tile rect written (none of it
    # when the projection writes those 12 B, counted there); per visible
    # Gaussian 4 depth passes of 20 B (4 B histogram read, 8 B read, 8 B
    # written), the slot scan's 24 B and the duplication's 16 B of reads; per
    # key 6 B written by the duplication, tile passes of 18 B (the first: the
    # slot is the index) and 22 B (2 B histogram read, 10 B read, 10 B
    # written) with 16-bit tile ids, and the 2 B read of the ranges
    def tile_passes(c):
        t, b = c.tiles_x * c.tiles_y, 0
        while (1 << b) < t:
            b += 1
        return (b + 7) // 8
    kb = 2 if all(c.tiles_x * c.tiles_y <= 65536 for c in sc.cameras[:views]) else 4
    per_g = 0 if prebinned else 32
    # the reach test: per visible Gaussian the mean and conic of its record
    # (32 B) read by the slot scan, and its tile mask written there and read
    # by the duplication (4 + 4 B)
    per_vis = 128 + (40 if reach else 0)
    bytes_sort = sum(per_g * sc.n + per_vis * nv + (6 + (tile_passes(c) > 0) * (kb + kb + 4 + kb + 8)
                                              + max(0, tile_passes(c) - 1) * (kb + kb + 8 + kb + 8) + kb) * k
                     for nv, k, c in zip(n_vis, Ks, sc.cameras[:views]))
    # the survey's per-unit model of a plain 64-bit LSB radix sort of the K
    # keys (scan 8 B x N, duplication 20 B x N + 12 B x K, 6 passes of 24 B +
    # an 8 B histogram read per key, ranges 8 B x K), which this design
    # does not move: reported beside it
    bytes_sort_lsb64 = sum(8 * sc.n + 20 * sc.n + 12 * k + (8 + 6 * 24) * k + 8 * k for k in Ks)
    bytes_pbwd = n_any * (geo + sh_bytes) + sum(nv * (48 + 36) for nv in n_vis) + n_any * 2 * (geo + 12 * K_sh)
    if prebinned:
        bytes_pbwd += views * sc.n * 4     # the depth keys (visibility of every Gaussian in every view)

    def hbm(name, nbytes, ms, model):
        if ms is None:
            return None
        gbps = nbytes / (ms / 1e3) / 1e9
        out = {"kernel": name, "bytes": int(nbytes), "ms": ms, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
               "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "model": model}
        if copy_meas:
            out["peak_measured_copy"] = round(copy_meas, 1)
            out["frac_measured"] = round(gbps / copy_meas, 4)
        return out

    hbm_stages = {
        "project": hbm("project_kernel (one launch, all views)", bytes_proj, med("project_batch"),
                       f"N x {geo} B parameters + {views} x N x {rec_b} B records"
                       + ((" (48 B + the sort's 4 B depth key)" if reach else
                           " (48 B + the sort's 12 B depth key and tile rect)") if prebinned else "") +
                       f" + {sh_bytes:g} B of SH per Gaussian visible in any view" + (" + N B mask" if use_mask else "")),
        "sort": hbm("gs_bin_sort_views (all views, 4 streams: the sort phase)",
                    bytes_sort, warm["sort_phase_ms"]["median"],
                    f"per view {per_g} B x N + {per_vis} B x visible + 48 B x K (depth passes on the visible Gaussians, "
                    f"scan, {'reach test, ' if reach else ''}duplication, 2 tile passes with 16-bit tile ids, "
                    "ranges); the survey's 64-bit "
                    f"6-pass model would be {bytes_sort_lsb64} B"),
        "project_bwd": (hbm("project_bwd_color_kernel + project_bwd_geom_kernel (one call, all views)",
                            bytes_pbwd, med("project_bwd_batch"),
                            f"per Gaussian visible in any view {geo} B + {sh_bytes:g} B parameters read and "
                            f"2 x ({geo} + {12 * K_sh}) B gradients read and written; per view and visible "
                            f"Gaussian 48 B record + 36 B screen-space sums"
                            + (f"; per view N x 4 B depth keys (visibility)" if prebinned else "")) if do_bwd else None),
    }

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
                           ("batched project writing the sort's depth keys and tile rects, " if prebinned
                            else "batched project, ") +
                           ("batched bin/sort" if args.sort == "batched" else "per view bin/sort") +
                           (" (each Gaussian listed in the tiles it reaches)" if reach else "") +
                           ", K copied to the host on a side stream (checked after the steps), batched blend fwd of all views" +
                           (" with per-Gaussian blending weights" if args.weights else "") +
                           (" (moving Gaussians, views spread over the time window)" if args.motion else "") +
                           (", then batched blend bwd of all views + one batched project bwd" if do_bwd else "") +
                           (f", then the fused SH Adam update ({args.sh_adam})" if adam is not None else "")},
        "fwd_ms_per_frame": round(fwd_ms, 4),
        "fwd_bwd_ms_per_frame": round(tot_ms, 4) if do_bwd else None,
        "timing": {"statistic": "median over steps (p90 and mean beside it); events on the streams the calls run on",
                   "warm": warm, "calls": calls, "cold": cold,
                   "calls_note": "per-call times from a separate run of as many steps with two events around "
                                 "every call; the warm and cold steps carry only the step's own events",
                   "cold_scrub": "2 GiB device copy (1 GiB read + 1 GiB written) before each cold step"},
        "per_call_ms": {k: med(k) for k in names},
        "K_per_view": Ks,
        "key_capacity_per_view": caps,
        "visible_per_view": n_vis,
        "visible_any_view": n_any,
        "P_eval_per_view": p_eval,
        "P_tile_per_view": p_tile,
        "P_needed_per_view": p_need,
        "P_composited_per_view": p_comp,
        "P_bwd_examined_per_view": p_bwd,
        "roofline": roof_fwd,
        "roofline_bwd": roof_bwd,
        "hbm_stages": hbm_stages,
        "peaks_measured": ({"fp32_fma_Tlane_per_s": round(peaks_measured["fma32"] / 1e12, 2),
                            "fp64_fma_Tlane_per_s": round(peaks_measured["fma64"] / 1e12, 2),
                            "exp_f32_Tlane_per_s": round(peaks_measured["exp32"] / 1e12, 2),
                            "exp_cost_slots_alone": round(peaks_measured["fma32"] / peaks_measured["exp32"], 2),
                            "exp_cost_slots_among_4_fma": round(peaks_measured["fma32"] / peaks_measured["mix"] - 4, 2),
                            "lds_read_TBps": round(peaks_measured["lds"] / 1e12, 1),
                            "copy_GBps": round(peaks_measured["copy"] / 1e9, 1),
                            "source": "csrc/peaks.hip, run once before the steps"}
                           if peaks_measured else None),
    }
    if adam is not None:
        t_adam = med("sh_adam") / 1e3
        gbps = adam["units"] * adam["bytes_per_unit"] / t_adam / 1e9
        res["sh_adam"] = {"kernel": "adam_q8_kernel" if args.sh_adam == "q8" else "adam_f32_kernel",
                          "state": "8-bit log-domain moments, fp16 values" if args.sh_adam == "q8"
                          else "fp32 moments and values",
                          "units": adam["units"], "ms": med("sh_adam"),
                          "bytes_per_unit": adam["bytes_per_unit"], "bound": "hbm",
                          "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gbps / HBM_PEAK_GBPS, 4),
                          "measured_copy_GBps": round(copy_meas, 1) if copy_meas else None,
                          "frac_of_measured_copy": round(gbps / copy_meas, 4) if copy_meas else None,
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
    """Per view, from its outputs: pairs examined under the compositing rule
    ("eval": a pixel that stopped examined n_contrib entries of its tile's
    list, otherwise all of them); among them those whose list entry can reach
    alpha >= 1/255 at some pixel centre of the pixel's 16x4 strip of its tile
    (rows 4r .. 4r+3, the strip a wave's pixel r covers: "needed"), the same
    with the whole tile ("tile"); the pairs the pixel composited ("composited":
    alpha >= 1/255 before its last composited entry) and the pairs the
    backward must examine ("bwd_examined": the entries before n_contrib)."""
    cam = b.cam
    TX, TY = cam.tiles_x, cam.tiles_y
    rng = b.ranges.long()
    L = rng[:, 1] - rng[:, 0]
    K = int(L.sum().item())
    start = rng[:, 0]
    Lpix = L.reshape(TY, TX).repeat_interleave(16, 0).repeat_interleave(16, 1)[: cam.height, : cam.width]
    nc = b.n_contrib.long()
    examined = torch.where(b.final_T < 1e-4, nc, Lpix)
    p_eval = int(examined.sum().item())
    p_bwd = int(nc.sum().item())
    tile = torch.repeat_interleave(torch.arange(TX * TY, device=rng.device), L)
    sp = b.splats[b.vals[:K].long()].double()
    u, v, a, bb, c, o = sp[:, 0], sp[:, 1], sp[:, 4], sp[:, 5], sp[:, 6], sp[:, 7]
    del sp
    tx0 = (tile % TX).double() * 16
    ty0 = (tile // TX).double() * 16
    dxl = tx0 + 0.5 - u
    dyl = ty0 + 0.5 - v
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
    del keep_tile
    # composited pairs: for each of the 256 pixel offsets of a tile, every
    # list entry whose position is before that pixel's n_contrib and whose
    # o exp(power) reaches 1/255 there
    pos = torch.arange(K, device=u.device) - start[tile]
    ncp = torch.zeros((TY * 16, TX * 16), dtype=torch.long, device=u.device)
    ncp[: cam.height, : cam.width] = nc
    txi, tyi = (tile % TX) * 16, (tile // TX) * 16
    p_comp = 0
    for oy in range(16):
        for ox in range(16):
            n_here = ncp[tyi + oy, txi + ox]
            dx = u - (tx0 + (ox + 0.5))
            dy = v - (ty0 + (oy + 0.5))
            power = -0.5 * (a * dx * dx + c * dy * dy) - bb * dx * dy
            p_comp += int(((pos < n_here) & (o * torch.exp(power) >= 1.0 / 255.0)).sum().item())
    return dict(eval=p_eval, needed=p_need, tile=p_tile, composited=p_comp, bwd_examined=p_bwd)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sc):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    project + bin + composite of whole views (forward) on all the threads
    OpenMP gives it (up to 4 views, ~10 s), then one whole view on one thread;
    reported in ms/frame."""
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
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    oracle.forward(sc, view=0)
    dt1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    return {"value": round(dt * 1e3 / frames, 1), "unit": "ms/frame", "cores": threads, "kind": "oracle",
            "sample": f"{frames} full forward view(s) of {sc.name} (project fp32-contract, brute-force "
                      f"binning + qsort, fp64 compositing), OpenMP; then view 0 on one thread",
            "one_core_ms_per_frame": round(dt1 * 1e3, 1),
            "cpu_model": cpu_model(), "cpus_visible": os.cpu_count()}


if __name__ == "__main__":
    main()
