"""Pins of the moving-Gaussian oracle (oracle/motion.py): a scene moving
uniformly renders as the static scene seen from a camera moved the other way
(which fixes the direction and the sign of tau - t_g), zero motion is the
static path, and the velocity and time-offset gradients match central finite
differences of the fp64 forward."""

import numpy as np

import oracle
from gaussian_splatting_tile_amd import scenes
from oracle import motion as M
from tests.test_oracle_pins import _fd_scene


def _render(means, sc, cam, precision="f64"):
    p = oracle.project(means, sc.scales, sc.quats, sc.opacities, sc.sh_degree, sc.sh, cam, precision=precision)
    return oracle.render(p, oracle.bin_sort(p, cam), cam)


def test_zero_motion_and_matching_time_are_static():
    sc = scenes.tiny(seed=3, n=500)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((3, sc.n)).astype(np.float32)
    t = rng.random(sc.n).astype(np.float32)
    assert np.array_equal(M.displaced_means(sc.means, np.zeros_like(v), t, 0.7), sc.means)
    assert np.array_equal(M.displaced_means(sc.means, v, t, 0.0)[:, t == 0], sc.means[:, t == 0])
    same = M.displaced_means(sc.means, v, np.full(sc.n, 0.25, np.float32), 0.25)
    assert np.array_equal(same, sc.means)


def test_uniform_motion_equals_a_camera_moved_the_other_way():
    """All Gaussians share v = u and t_g = c: at time tau the scene is the
    static one shifted by (tau - c) u, i.e. the static scene seen from a
    camera translated by (tau - c) u, whose world->camera translation is
    t - R (tau - c) u."""
    sc = scenes.tiny(seed=4, n=800)
    cam = sc.cameras[0]
    u = np.array([0.31, -0.22, 0.15])
    for c, tau in ((0.0, 0.8), (0.5, 0.2), (0.3, 0.3)):
        mp = M.displaced_means(sc.means, np.repeat(u[:, None], sc.n, axis=1), np.full(sc.n, c), tau,
                               precision="f64")
        moving = _render(mp, sc, cam)
        vm = np.asarray(cam.viewmat, dtype=np.float64).copy()
        vm[:, 3] = vm[:, 3] + vm[:, :3] @ ((tau - c) * u)
        cam2 = scenes.Camera(cam.width, cam.height, cam.fx, cam.fy, cam.cx, cam.cy, vm, cam.znear, cam.guard)
        still = _render(sc.means.astype(np.float64), sc, cam2)
        assert np.array_equal(moving["n_contrib"], still["n_contrib"])
        assert np.abs(moving["image"] - still["image"]).max() <= 1e-9
        if tau != c:                            # and it is not the unmoved picture
            base = _render(sc.means.astype(np.float64), sc, cam)
            assert np.abs(base["image"] - moving["image"]).max() > 1e-2


def test_velocity_and_time_offset_gradients_match_finite_differences():
    means, log_s, quats, logits, sh, cam, G = _fd_scene(seed=9)
    n = means.shape[1]
    rng = np.random.default_rng(10)
    vel = 0.2 * rng.standard_normal((3, n))
    t0 = rng.uniform(0.0, 1.0, n)
    tau = 0.6
    s, o = np.exp(log_s), 1.0 / (1.0 + np.exp(-logits))

    def loss(v, t):
        mp = M.displaced_means(means, v, t, tau, precision="f64")
        p = oracle.project(mp, s, quats, o, 3, sh, cam, precision="f64")
        b = oracle.bin_sort(p, cam)
        out = oracle.render(p, b, cam)
        return float((G * out["image"]).sum()), (tuple(b["vals"]), out["n_contrib"].tobytes()), mp, p, b

    L0, st0, mp, p, b = loss(vel, t0)
    assert (p["radius"] > 0).sum() >= 4
    g2 = oracle.render_bwd(p, b, cam, G)
    grads = oracle.project_bwd(mp, s, quats, o, 3, sh, cam, p, g2)
    d_vel, d_t = M.motion_grads(grads["means"], vel, t0, tau)
    h = 1e-6
    checked = 0
    for g in range(n):
        if p["radius"][g] == 0:
            continue
        for i in range(3):
            vals = []
            for sgn in (1, -1):
                v2 = vel.copy()
                v2[i, g] += sgn * h
                L, st, *_ = loss(v2, t0)
                assert st == st0
                vals.append(L)
            num = (vals[0] - vals[1]) / (2 * h)
            assert abs(num - d_vel[i, g]) <= 1e-6 * max(1.0, abs(num)) + 1e-7, ("v", i, g, num, d_vel[i, g])
        vals = []
        for sgn in (1, -1):
            t2 = t0.copy()
            t2[g] += sgn * h
            L, st, *_ = loss(vel, t2)
            assert st == st0
            vals.append(L)
        num = (vals[0] - vals[1]) / (2 * h)
        assert abs(num - d_t[g]) <= 1e-6 * max(1.0, abs(num)) + 1e-7, ("t", g, num, d_t[g])
        checked += 1
    assert checked >= 4
