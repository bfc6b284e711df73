"""GPU parity of the 8-bit block-quantized SH storage (GS_SH_Q8): the
quantizer's codes and bounds bit-exact against the oracle's; records, bins
and images from 8-bit SH against the oracle fed the decoded SH; gradients
against the oracle's (the SH gradient is taken with respect to the decoded
values)."""

import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_tile_amd import binding as B
from gaussian_splatting_tile_amd import scenes
from tests.gpu_util import compare_bins, compare_image, compare_records, run_view, say, splats_np
from tests.test_gpu_backward import NAMES, _compare, _upstream

pytestmark = pytest.mark.gpu


def _gpu_quantize(sh):
    t = torch.from_numpy(np.ascontiguousarray(sh, np.float32)).cuda()
    K, c3, n = sh.shape
    codes = torch.full((K, c3, n), 7, dtype=torch.uint8, device="cuda")
    bounds = torch.full((B.sh_q8_bounds_floats(n, K * c3),), float("nan"), device="cuda")
    B.sh_quantize8(t, codes, bounds)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), bounds.cpu().numpy().reshape(K * c3, -1, 2)


def test_sh_quantize8_matches_oracle():
    rng = np.random.default_rng(31)
    for n in (1, 255, 256, 257, 4097, 100_003):
        sh = rng.normal(0.0, 0.2, (16, 3, n)).astype(np.float32)
        sh[0] = rng.uniform(-1.0, 1.0, (3, n)).astype(np.float32)
        if n >= 512:
            sh[3, 2, 256:512] = np.float32(-0.125)                 # a constant block
        say(f"[gpu] sh_quantize8 n={n}")
        q, b = _gpu_quantize(sh)
        rq, rb = oracle.sh_quantize8(sh)
        assert np.array_equal(b, rb)
        assert np.array_equal(q, rq)


def test_projection_and_blend_from_q8_sh():
    sc = scenes.config(2, n_override=60_000)
    say("[gpu] 8-bit SH: box_60k forward")
    q, b = oracle.sh_quantize8(sc.sh)
    sh_dec = oracle.sh_dequantize8(q, b)
    buf, K = run_view(sc, 0, sh=(q, b))
    cam = sc.cameras[0]
    op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sh_dec, cam)
    ob = oracle.bin_sort(op, cam)
    compare_records(splats_np(buf), op, "q8 box_60k")
    compare_bins(buf, K, ob, "q8 box_60k")
    oo = oracle.render(op, ob, cam)
    st = compare_image(buf, cam, op, ob, oo)
    say(f"[gpu] q8 box_60k: K={K} {st}")
    assert st["unresolved"] == 0, st["details"]
    # the decoded colours stay close to the fp32 source's
    op32 = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sc.sh, cam)
    vis = op32["radius"] > 0
    assert np.abs(op32["rgb"][:, vis] - op["rgb"][:, vis]).max() < 0.02


def test_backward_from_q8_sh():
    sc = scenes.scene_like(seed=71, n=40_000, width=480, height=272, f=350.0, n_views=1)
    say("[gpu] 8-bit SH: backward")
    q, b = oracle.sh_quantize8(sc.sh)
    sh_dec = oracle.sh_dequantize8(q, b)
    cam = sc.cameras[0]
    op = oracle.project(sc.means, sc.scales, sc.quats, sc.opacities, 3, sh_dec, cam)
    ob = oracle.bin_sort(op, cam)
    oo = oracle.render(op, ob, cam)
    amb = (oo["events"] > 0) | (oo["capflag"] > 0)
    G = _upstream(cam, 701).astype(np.float64)
    G[:, amb] = 0.0
    g2 = oracle.render_bwd(op, ob, cam, G)
    ref = oracle.project_bwd(sc.means, sc.scales, sc.quats, sc.opacities, 3, sh_dec, cam, op, g2)
    near = np.abs(op["rgb_raw"]).min(axis=0) < 1e-5
    n = sc.n
    grads = dict(means=torch.zeros((3, n), device="cuda"), log_scales=torch.zeros((3, n), device="cuda"),
                 quats=torch.zeros((4, n), device="cuda"), opacity_logits=torch.zeros(n, device="cuda"),
                 sh=torch.zeros((16, 3, n), device="cuda"))
    buf, K = run_view(sc, 0, with_keys=False, sh=(q, b))
    g, act, gs = buf._keep
    ws = buf.backward_workspace()
    buf.backward(gs, torch.from_numpy(np.ascontiguousarray(G.astype(np.float32))).cuda(), grads, ws)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    _compare(gpu, ref, near, "bwd q8")
