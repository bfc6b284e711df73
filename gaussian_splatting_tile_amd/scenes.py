"""Seeded synthetic scenes for the tiled Gaussian-splatting rasterizer.

This module only draws inputs.  It holds none of the rasterizer's arithmetic:
no projection, no colour evaluation, no binning and no compositing.  Both the
GPU path and the CPU oracle are fed from here.

The per-Gaussian parameter set (position, scale, rotation, opacity and
spherical-harmonic colour) is the one the GlobalSplat page lists for the
Gaussians its geometry and appearance heads predict.  The five workloads are
synthetic stand-ins for the captured scenes the pages measure on (the "bicycle"
scene of the Spirula Studio page, the city-scale sets of the BlitzGS page);
none of those datasets is used.

Conventions
-----------
* Arrays are structure-of-arrays: ``means[3][N]``, ``scales[3][N]``,
  ``quats[4][N]`` as (w, x, y, z), ``opacities[N]``, ``sh[K][3][N]`` with
  ``K = (degree+1)**2`` coefficients ordered by band l = 0..3, m = -l..l.
* Scales and opacities are handed over activated (``exp`` of the drawn
  log-scale, ``sigmoid`` of the drawn logit, both in float32); the raw draws are
  kept so gradients can be taken with respect to them.
* ``N(mu, x)`` in a workload description is read with ``x`` as the variance.
* Cameras are pinhole, OpenCV axes (x right, y down, z forward); ``viewmat`` is
  the row-major 3x4 world-to-camera matrix ``[R | t]``.
* Random draws are float32 (``numpy.random.Generator``, PCG64) in a fixed
  order: means, log-scales, quaternions, opacity logits, SH, permutation,
  poses, importance scores, upstream image gradients.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

TILE = 16


@dataclasses.dataclass
class Camera:
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    viewmat: np.ndarray          # float32 [3][4], world -> camera, [R | t]
    znear: float = 0.2
    guard: float = 1.3
    lod_min_radius_px: float = 0.0   # 0 disables the distance-LOD gate
    time: float = 0.0                # the view's time (for moving Gaussians)

    @property
    def tiles_x(self) -> int:
        return (self.width + TILE - 1) // TILE

    @property
    def tiles_y(self) -> int:
        return (self.height + TILE - 1) // TILE

    @property
    def n_tiles(self) -> int:
        return self.tiles_x * self.tiles_y


@dataclasses.dataclass
class Scene:
    name: str
    means: np.ndarray            # f32 [3][N]
    log_scales: np.ndarray       # f32 [3][N]
    scales: np.ndarray           # f32 [3][N]  exp(log_scales)
    quats: np.ndarray            # f32 [4][N]  (w, x, y, z)
    opacity_logits: np.ndarray   # f32 [N]
    opacities: np.ndarray        # f32 [N]     sigmoid(logits)
    sh_degree: int
    sh: np.ndarray               # f32 [K][3][N]
    cameras: List[Camera]
    sh_fp16: Optional[np.ndarray] = None     # f16 [K][3][N] (storage form)
    importance: Optional[np.ndarray] = None  # f32 [N]
    keep_fraction: float = 1.0
    upstream_seed: Optional[int] = None      # seed of dL/dimage draws
    velocity: Optional[np.ndarray] = None    # f32 [3][N] motion vectors (moving scenes)
    t_offset: Optional[np.ndarray] = None    # f32 [N]    time offsets t_g

    @property
    def n(self) -> int:
        return int(self.means.shape[1])

    def sh_decoded(self) -> np.ndarray:
        """SH as the kernels see it: fp16 storage decoded exactly to fp32."""
        if self.sh_fp16 is None:
            return self.sh
        return self.sh_fp16.astype(np.float32)

    def upstream(self, view: int) -> np.ndarray:
        """dL/dimage ~ N(0, 1e-2) (std 0.1), f32 [3][H][W], one stream per view."""
        cam = self.cameras[view]
        rng = np.random.default_rng([self.upstream_seed or 0, view])
        return (rng.standard_normal((3, cam.height, cam.width), dtype=np.float32)
                * np.float32(0.1))


def _sigmoid32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _unit_quats(rng: np.random.Generator, n: int) -> np.ndarray:
    q = rng.standard_normal((4, n), dtype=np.float32)
    nrm = np.sqrt((q.astype(np.float64) ** 2).sum(axis=0))
    nrm[nrm == 0] = 1.0
    return (q / nrm).astype(np.float32)


def _sh(rng: np.random.Generator, degree: int, n: int) -> np.ndarray:
    k = (degree + 1) ** 2
    sh = np.empty((k, 3, n), dtype=np.float32)
    sh[0] = rng.random((3, n), dtype=np.float32)                 # DC ~ U(0,1)
    if k > 1:
        sh[1:] = rng.standard_normal((k - 1, 3, n), dtype=np.float32) * np.float32(0.2)
    return sh


def _uniform(rng, lo, hi, shape):
    return (np.float32(lo) + np.float32(hi - lo) * rng.random(shape, dtype=np.float32)).astype(np.float32)


def _random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random rotation from the QR factorisation of a Gaussian matrix."""
    a = rng.standard_normal((3, 3))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def look_at(eye: np.ndarray, target=(0.0, 0.0, 0.0), up=(0.0, 1.0, 0.0)) -> np.ndarray:
    """World-to-camera [R | t] for a camera at ``eye`` looking at ``target``
    (OpenCV axes: camera z toward the target, camera y pointing down)."""
    eye = np.asarray(eye, dtype=np.float64)
    zc = np.asarray(target, dtype=np.float64) - eye
    zc /= np.linalg.norm(zc)
    xc = np.cross(zc, np.asarray(up, dtype=np.float64))
    xc /= np.linalg.norm(xc)
    yc = np.cross(zc, xc)
    rot = np.stack([xc, yc, zc])
    t = -rot @ eye
    return np.concatenate([rot, t[:, None]], axis=1).astype(np.float32)


def _orbit_cameras(rng, n_views, radius, width, height, f, lod=0.0) -> List[Camera]:
    thetas = rng.random(n_views) * 2.0 * math.pi
    cams = []
    for th in thetas:
        eye = radius * np.array([math.sin(th), 0.0, math.cos(th)])
        cams.append(Camera(width, height, float(f), float(f), width / 2.0, height / 2.0,
                           look_at(eye), lod_min_radius_px=lod))
    return cams


def _scene_like_means(rng: np.random.Generator, n: int) -> np.ndarray:
    """90 %: 64 anisotropic Gaussian clusters; 10 %: a shell of radius 50."""
    n_shell = n // 10
    n_cl = n - n_shell
    centres = _uniform(rng, -10.0, 10.0, (64, 3)).astype(np.float64)
    rots = np.stack([_random_rotation(rng) for _ in range(64)])
    sig = _uniform(rng, 0.3, 3.0, (64, 3)).astype(np.float64)
    member = np.arange(n_cl) % 64
    z = rng.standard_normal((n_cl, 3), dtype=np.float32).astype(np.float64)
    pts = centres[member] + np.einsum("nij,nj->ni", rots[member], sig[member] * z)
    shell = rng.standard_normal((n_shell, 3), dtype=np.float32).astype(np.float64)
    shell = 50.0 * shell / np.linalg.norm(shell, axis=1, keepdims=True)
    return np.concatenate([pts, shell], axis=0).T.astype(np.float32)


def tiny(seed: int = 1, n: int = 1000, width: int = 128, height: int = 128) -> Scene:
    """1K Gaussians, SH degree 0, 128x128, fx = fy = 128, identity pose.
    Means x, y ~ U(-1,1), z ~ U(2,4); log-scales ~ U(-4,-2); quats normalised
    N(0, I4); opacity sigmoid(N(0,1)); DC colour ~ U(0,1)."""
    rng = np.random.default_rng(seed)
    means = np.empty((3, n), np.float32)
    means[0:2] = _uniform(rng, -1.0, 1.0, (2, n))
    means[2] = _uniform(rng, 2.0, 4.0, (n,))
    log_s = _uniform(rng, -4.0, -2.0, (3, n))
    quats = _unit_quats(rng, n)
    logit = rng.standard_normal(n, dtype=np.float32)
    sh = _sh(rng, 0, n)
    vm = np.concatenate([np.eye(3), np.zeros((3, 1))], axis=1).astype(np.float32)
    cam = Camera(width, height, 128.0 * width / 128, 128.0 * height / 128, width / 2.0, height / 2.0, vm)
    return Scene("tiny_1k_sh0_128", means, log_s, np.exp(log_s).astype(np.float32), quats,
                 logit, _sigmoid32(logit), 0, sh, [cam])


def box(seed: int = 2, n: int = 100_000, width: int = 1280, height: int = 720, f: float = 1000.0) -> Scene:
    """100K Gaussians, SH3, means U([-5,5]^3) seen from 15 units away
    (identity rotation, t = (0,0,15)), 1280x720, f = 1000; log-scales
    U(-5,-2); opacity sigmoid(N(0,1.5)); DC ~ U(0,1), higher bands N(0,0.2^2)."""
    rng = np.random.default_rng(seed)
    means = _uniform(rng, -5.0, 5.0, (3, n))
    log_s = _uniform(rng, -5.0, -2.0, (3, n))
    quats = _unit_quats(rng, n)
    logit = rng.standard_normal(n, dtype=np.float32) * np.float32(math.sqrt(1.5))
    sh = _sh(rng, 3, n)
    vm = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 15]], dtype=np.float32)
    cam = Camera(width, height, f, f, width / 2.0, height / 2.0, vm)
    return Scene(f"box_{n}_sh3_{width}x{height}", means, log_s, np.exp(log_s).astype(np.float32),
                 quats, logit, _sigmoid32(logit), 3, sh, [cam])


def scene_like(seed: int = 3, n: int = 1_000_000, width: int = 1920, height: int = 1080,
               f: float = 1400.0, n_views: int = 8, sh_fp16: bool = False,
               keep_fraction: float = 1.0, lod_px: float = 0.0, upstream: bool = False,
               name: Optional[str] = None) -> Scene:
    """Scene-like mixture: 64 anisotropic clusters (90 %) plus a background
    shell at radius 50 (10 %), randomly permuted; log-scales N(-4, 0.8)
    clipped at -1; opacity sigmoid(N(0,1.5)); SH3 as in :func:`box`; views on
    an orbit of radius 25 around the origin."""
    rng = np.random.default_rng(seed)
    means = _scene_like_means(rng, n)
    log_s = np.minimum(np.float32(-4.0) + np.float32(math.sqrt(0.8)) *
                       rng.standard_normal((3, n), dtype=np.float32), np.float32(-1.0)).astype(np.float32)
    quats = _unit_quats(rng, n)
    logit = rng.standard_normal(n, dtype=np.float32) * np.float32(math.sqrt(1.5))
    sh = _sh(rng, 3, n)
    perm = rng.permutation(n)
    means, log_s, quats = means[:, perm], log_s[:, perm], quats[:, perm]
    logit, sh = logit[perm], sh[:, :, perm]
    means = np.ascontiguousarray(means)
    log_s = np.ascontiguousarray(log_s)
    quats = np.ascontiguousarray(quats)
    sh = np.ascontiguousarray(sh)
    cams = _orbit_cameras(rng, n_views, 25.0, width, height, f, lod=lod_px)
    importance = None
    if keep_fraction < 1.0:
        importance = rng.exponential(1.0, n).astype(np.float32)
    sc = Scene(name or f"scene_{n}_sh3_{width}x{height}", means, log_s, np.exp(log_s).astype(np.float32),
               quats, logit, _sigmoid32(logit), 3, sh, cams,
               sh_fp16=sh.astype(np.float16) if sh_fp16 else None,
               importance=importance, keep_fraction=keep_fraction,
               upstream_seed=seed * 1000 + 7 if upstream else None)
    return sc


# The five workloads, smallest first.
def config(idx: int, n_override: Optional[int] = None) -> Scene:
    """Workload ``idx`` (1..5).  ``n_override`` shrinks N for quick tests while
    keeping the distribution."""
    if idx == 1:
        return tiny(n=n_override or 1000)
    if idx == 2:
        return box(n=n_override or 100_000)
    if idx == 3:
        return scene_like(seed=3, n=n_override or 1_000_000, name="scene_1m_sh3_1080p")
    if idx == 4:
        return scene_like(seed=4, n=n_override or 5_000_000, upstream=True, name="scene_5m_sh3_1080p_bwd")
    if idx == 5:
        return scene_like(seed=5, n=n_override or 10_000_000, width=3840, height=2160, f=2800.0,
                          sh_fp16=True, keep_fraction=0.3, lod_px=0.5, upstream=True,
                          name="scene_10m_sh3fp16_4k_cull")
    raise ValueError(f"unknown workload {idx}")


def keep_count(n: int, keep_fraction: float) -> int:
    """Number of Gaussians the importance mask keeps: floor(fraction * N)."""
    return int(math.floor(keep_fraction * n + 1e-9))


# ---------------------------------------------------------------------------
# Inputs of the fused SH Adam step: SH gradients, SH values and an optimizer
# state, all drawn at random (no optimizer arithmetic here).
def adam_inputs(seed: int, n: int, rows: int, state: str = "q8", value_dtype=np.float16,
                fresh: bool = False, visible: float = 0.6) -> dict:
    """Seeded inputs for one SH Adam step over ``rows`` x ``n`` units.

    * grad f32 [rows][n]: zero for Gaussians outside the step's views (a
      fraction ``1 - visible`` of them), else N(0, sigma) with a per-Gaussian
      sigma = 1e-6 * LogNormal(0, 1.5), ten times larger on the three DC rows.
    * value [rows][n] in ``value_dtype``: DC rows U(0, 1), the others N(0, 0.2).
    * state "f32": m ~ N(0, sigma_m), v = sigma_v^2 * LogNormal(0, 1)^2 per
      unit (both f32), or zeros when ``fresh``.
    * state "q8": m and s codes uniform on 0..255; per 256-unit block, m bounds
      (-a, b) with a, b = 1e-6 * LogNormal(0, 1.5), and s bounds
      (c - 3 + U(0, 1), c + U(0, 1)) around c = ln(max(a, b) / 1e-15), i.e.
      second-moment roots from e^-3 to e^1 times the block's first-moment
      scale; one block in 16 of each row has equal bounds.  ``fresh``: all
      codes and bounds 0.
    """
    rng = np.random.default_rng([seed, n, rows])
    nb = (n + 255) // 256
    sig = (1e-6 * np.exp(rng.standard_normal(n) * 1.5)).astype(np.float32)
    vis = rng.random(n) < visible
    grad = rng.standard_normal((rows, n), dtype=np.float32) * (sig * vis)[None, :]
    grad[:min(3, rows)] *= np.float32(10.0)
    value = np.empty((rows, n), dtype=np.float32)
    value[:min(3, rows)] = rng.random((min(3, rows), n), dtype=np.float32)
    if rows > 3:
        value[3:] = rng.standard_normal((rows - 3, n), dtype=np.float32) * np.float32(0.2)
    out = dict(grad=grad.astype(np.float32), value=value.astype(value_dtype))
    if state == "f32":
        if fresh:
            out["m"] = np.zeros((rows, n), dtype=np.float32)
            out["v"] = np.zeros((rows, n), dtype=np.float32)
        else:
            out["m"] = (rng.standard_normal((rows, n), dtype=np.float32) * sig[None, :]).astype(np.float32)
            sv = sig[None, :] * np.exp(rng.standard_normal((rows, n))).astype(np.float32)
            out["v"] = (sv * sv).astype(np.float32)
        return out
    if fresh:
        for k in ("m", "s"):
            out[k + "_codes"] = np.zeros((rows, n), dtype=np.uint8)
            out[k + "_bounds"] = np.zeros((rows, nb, 2), dtype=np.float32)
        return out
    out["m_codes"] = rng.integers(0, 256, (rows, n), dtype=np.uint8)
    out["s_codes"] = rng.integers(0, 256, (rows, n), dtype=np.uint8)
    a = 1e-6 * np.exp(rng.standard_normal((rows, nb)) * 1.5)
    b = 1e-6 * np.exp(rng.standard_normal((rows, nb)) * 1.5)
    mb = np.stack([-a, b], axis=2).astype(np.float32)
    c = np.log(np.maximum(a, b) / 1e-15)
    sb = np.stack([c - 3.0 + rng.random((rows, nb)), c + rng.random((rows, nb))], axis=2).astype(np.float32)
    const = rng.random((rows, nb)) < 1.0 / 16.0
    mb[const, 1] = mb[const, 0]
    sb[const, 1] = sb[const, 0]
    out["m_bounds"] = mb
    out["s_bounds"] = sb
    return out


# ---------------------------------------------------------------------------
def with_motion(sc: Scene, seed: int, speed: float = 0.5, span: float = 1.0) -> Scene:
    """The scene with a motion vector and a time offset per Gaussian (the
    VisionTech page's 4D record): v ~ N(0, speed^2) per axis in scene units
    per unit time, t_g ~ U(0, span), and view i of V at time span * i / (V - 1)
    (the views sweep the time window)."""
    import dataclasses
    rng = np.random.default_rng([seed, sc.n, 4])
    vel = (rng.standard_normal((3, sc.n), dtype=np.float32) * np.float32(speed)).astype(np.float32)
    t0 = _uniform(rng, 0.0, span, sc.n)
    V = len(sc.cameras)
    cams = [dataclasses.replace(c, time=float(np.float32(span * i / max(1, V - 1))))
            for i, c in enumerate(sc.cameras)]
    return dataclasses.replace(sc, velocity=vel, t_offset=t0, cameras=cams, name=sc.name + "_motion")
