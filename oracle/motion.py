"""Moving Gaussians -- CPU oracle (numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the GPU library,
and it shares no code with it.

What is computed (VisionTech page on its 4D Gaussian splatting renderer, the
section on the technical architecture: every Gaussian carries a position, a
time offset, a covariance, colour and opacity, and a motion vector).  The
page gives no formula; the reading taken is the plainest one: in a view at
time tau, Gaussian g is drawn at

    mu' = mu + (tau - t_g) v

and everything after that is the static path with mu' as the mean.  mu'
decides tiles, so in the "f32" form it is formed with one fp32 rounding per
operation in that order, dt = fp32(tau - t_g), mu' = fp32(mu + fp32(dt v));
the "f64" form is the smooth function the finite-difference pins
differentiate.  The gradients (fp64) follow from the chain rule:
dL/dmu = dL/dmu', dL/dv = dt dL/dmu', dL/dt_g = -v . dL/dmu', summed over
the views.
"""

from __future__ import annotations

import numpy as np


def displaced_means(means, velocity, t_offset, time, precision: str = "f32") -> np.ndarray:
    if precision == "f64":
        dt = float(time) - np.asarray(t_offset, dtype=np.float64)
        return np.asarray(means, dtype=np.float64) + dt[None, :] * np.asarray(velocity, dtype=np.float64)
    f = np.float32
    with np.errstate(invalid="ignore", over="ignore"):      # non-finite motion: culled downstream
        dt = (f(time) - np.asarray(t_offset, dtype=f)).astype(f)
        step = (dt[None, :] * np.asarray(velocity, dtype=f)).astype(f)
        return (np.asarray(means, dtype=f) + step).astype(f)


def motion_grads(d_means_displaced, velocity, t_offset, time):
    """(dL/dv [3][n], dL/dt_g [n]) of one view from its dL/dmu' (fp64)."""
    dm = np.asarray(d_means_displaced, dtype=np.float64)
    dt = float(np.float32(time)) - np.asarray(t_offset, dtype=np.float64)
    d_vel = dt[None, :] * dm
    d_t = -(np.asarray(velocity, dtype=np.float64) * dm).sum(axis=0)
    return d_vel, d_t
