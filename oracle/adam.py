"""Fused SH Adam step -- CPU oracle in numpy, fp64.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the GPU library,
and it shares no code with it.  Plain, slow and elementwise, so that it can be
checked against the sources by eye.

What is computed (Spirula Studio page on quantized training: the sections on
its one precision switch, on why an 8-bit Adam state keeps its accuracy, and on
the measured speed-up of its fused optimizer kernel):

* A "unit" is one SH coefficient of one colour channel of one Gaussian; the
  SH arrays are [rows][n] with rows = 3 K (K SH coefficients x 3 channels), so the
  256 consecutive Gaussians of one row form one block of 256 units -- the
  page's transposed 256-Gaussian layout.
* SH gradients stay fp32 and are never quantized.  SH values are stored in 16
  bits (fp16) at the page's default level, 32 bits at full precision.
* Adam itself is the standard bias-corrected form (Kingma and Ba); the page
  names Adam's two moments but prints no update formula:
      m' = b1 m + (1 - b1) g          v' = b2 v + (1 - b2) g^2
      theta' = theta - lr * (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps)
  applied to every unit (lazy=False: the dense rule of torch.optim.Adam,
  where a unit with a zero gradient still decays both moments and moves by
  its first moment) or lazily (lazy=True: a unit whose gradient is exactly
  zero in this step, a Gaussian none of the step's views saw, keeps its
  value and both moments, as in torch.optim.SparseAdam).  t counts all
  steps.  The page states neither rule; lazy is the reading taken with the
  8-bit state, where zero is in general not a code of the first moment and a
  dense step would move every unseen Gaussian by about lr * (quantization
  residue) / eps.
* Full-precision state: m and v as fp32.
* 8-bit state: both moments 8-bit with one (min, max) float pair per block of
  256 consecutive units, decoded lo + q * step, step = (hi - lo) * fp32(1/255)
  (the block-quantized decode the same page describes, taken in fp32 exactly
  as for 8-bit SH storage).  The first moment is stored as itself; the second
  as s = log1p(sqrt(v) / eps), the page's log-domain encoding, so that
  v = (eps * expm1(s))^2.  After the update each block takes the min and max
  of its new values as its bounds and codes round to nearest,
  q = floor((x - lo) * 255 / (hi - lo) + 0.5), 0 for a block with hi == lo.
  A fresh state is all codes 0 with bounds (0, 0), i.e. m = v = 0.

Everything after the fp32 decode of the input state is fp64.  The new value is
rounded to nearest (ties to even) into its storage type; the new bounds are
returned both in fp64 and rounded to fp32, and the codes are decided in fp64
with the unrounded code position t returned beside them, so that a test can
tell which codes sit so close to a rounding boundary that an fp32 evaluation
may legitimately land on the other side.
"""

from __future__ import annotations

import numpy as np

BLOCK = 256


def n_blocks(n: int) -> int:
    return (int(n) + BLOCK - 1) // BLOCK


def decode8(codes: np.ndarray, bounds: np.ndarray) -> np.ndarray:
    """fp32 decode of [rows][n] codes with [rows][nb][2] bounds: lo + q * step,
    step = (hi - lo) * fp32(1/255), every operation one fp32 rounding."""
    rows, n = codes.shape
    nb = n_blocks(n)
    b = np.asarray(bounds, dtype=np.float32).reshape(rows, nb, 2)
    blk = np.arange(n) // BLOCK
    lo = b[:, blk, 0]
    hi = b[:, blk, 1]
    step = (hi - lo) * np.float32(1.0 / 255.0)
    return lo + codes.astype(np.float32) * step


def encode8(x: np.ndarray):
    """Block min/max and round-to-nearest codes of fp64 [rows][n] values.
    Returns codes (uint8), bounds (fp64 [rows][nb][2]) and the unrounded code
    positions t (fp64; 0 in blocks with hi == lo)."""
    x = np.asarray(x, dtype=np.float64)
    rows, n = x.shape
    nb = n_blocks(n)
    pad = nb * BLOCK - n
    xp = np.pad(x, ((0, 0), (0, pad)), constant_values=np.nan).reshape(rows, nb, BLOCK)
    lo = np.nanmin(xp, axis=2) if n else np.zeros((rows, 0))
    hi = np.nanmax(xp, axis=2) if n else np.zeros((rows, 0))
    bounds = np.stack([lo, hi], axis=2)
    blk = np.arange(n) // BLOCK
    d = (hi - lo)[:, blk]
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(d > 0, (x - lo[:, blk]) * 255.0 / np.where(d > 0, d, 1.0), 0.0)
    codes = np.clip(np.floor(t + 0.5), 0, 255).astype(np.uint8)
    return codes, bounds, t


def _adam(theta, m, v, g, step, lr, beta1, beta2, eps, lazy):
    """One bias-corrected Adam update in fp64 of every unit (lazy=False) or
    of the units with g != 0 (lazy=True, the others unchanged); returns
    theta', m', v'."""
    live = (g != 0) if lazy else np.ones(np.shape(g), dtype=bool)
    m1 = np.where(live, beta1 * m + (1.0 - beta1) * g, m)
    v1 = np.where(live, beta2 * v + (1.0 - beta2) * g * g, v)
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    theta1 = np.where(live, theta - lr * (m1 / bc1) / (np.sqrt(v1 / bc2) + eps), theta)
    return theta1, m1, v1


def adam_step_f32(grad, value, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-15, lazy=True):
    """Full-precision state: m and v fp32 [rows][n].  value is fp32 or fp16;
    the new value is rounded into the same type."""
    g = np.asarray(grad, dtype=np.float64)
    th, m1, v1 = _adam(np.asarray(value, dtype=np.float64), np.asarray(m, dtype=np.float64),
                       np.asarray(v, dtype=np.float64), g, step, lr, beta1, beta2, eps, lazy)
    return dict(value=th.astype(value.dtype), value64=th, m=m1.astype(np.float32), m64=m1,
                v=v1.astype(np.float32), v64=v1)


def adam_step_q8(grad, value, m_codes, m_bounds, s_codes, s_bounds, step, lr,
                 beta1=0.9, beta2=0.999, eps=1e-15, lazy=True):
    """8-bit state: m and s = log1p(sqrt(v)/eps) as codes [rows][n] (uint8)
    with bounds [rows][nb][2] (fp32).  value is fp32 or fp16."""
    g = np.asarray(grad, dtype=np.float64)
    m = decode8(m_codes, m_bounds).astype(np.float64)
    s = decode8(s_codes, s_bounds).astype(np.float64)
    v = (eps * np.expm1(s)) ** 2
    th, m1, v1 = _adam(np.asarray(value, dtype=np.float64), m, v, g, step, lr, beta1, beta2, eps, lazy)
    live = (g != 0) if lazy else np.ones(g.shape, dtype=bool)
    s1 = np.where(live, np.log1p(np.sqrt(v1) / eps), s)          # an untouched unit keeps its s
    mc, mb, mt = encode8(m1)
    sc, sb, st = encode8(s1)
    return dict(value=th.astype(value.dtype), value64=th, m64=m1, s64=s1,
                m_codes=mc, m_bounds=mb.astype(np.float32), m_bounds64=mb, m_t=mt,
                s_codes=sc, s_bounds=sb.astype(np.float32), s_bounds64=sb, s_t=st)
