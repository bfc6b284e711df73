"""Pins of the fused SH Adam oracle (oracle/adam.py) to things other than
itself: torch's own Adam (the dense rule, zero gradients included) and
SparseAdam (the lazy rule) -- independent library implementations of the
same update, Adam also fed the oracle's decoded 8-bit state -- closed
forms of a first step, the scale invariance of Adam, exact codes of a
log-encoded ramp, block locality and the round-trip bound of the 8-bit
encoding."""

import numpy as np
import pytest
import torch

from gaussian_splatting_tile_amd import scenes
from oracle import adam as A

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-15


def _torch_adam(theta, grads, m0=None, v0=None, step0=0, lr=LR, eps=EPS):
    """Run torch.optim.Adam (CPU, float64) over ``grads`` from the state
    (m0, v0) that ``step0`` earlier steps left; returns the parameter and
    the final moments."""
    p = torch.nn.Parameter(torch.from_numpy(np.array(theta, dtype=np.float64)))
    opt = torch.optim.Adam([p], lr=lr, betas=(B1, B2), eps=eps)
    if m0 is not None:
        opt.state[p] = dict(step=torch.tensor(float(step0), dtype=torch.float64),
                            exp_avg=torch.from_numpy(np.array(m0, dtype=np.float64)),
                            exp_avg_sq=torch.from_numpy(np.array(v0, dtype=np.float64)))
    for g in grads:
        p.grad = torch.from_numpy(np.array(g, dtype=np.float64))
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def test_full_precision_matches_torch_adam_over_steps():
    """Every gradient non-zero: the lazy update is plain Adam."""
    d = scenes.adam_inputs(11, 700, 6, state="f32", value_dtype=np.float64, fresh=True)
    rng = np.random.default_rng(5)
    grads = [rng.standard_normal((6, 700)) * 1e-5 * (1 + rng.random()) for _ in range(5)]
    th, m, v = d["value"].astype(np.float64), d["m"].astype(np.float64), d["v"].astype(np.float64)
    for t, g in enumerate(grads, start=1):
        r = A.adam_step_f32(g, th, m, v, step=t, lr=LR)
        th, m, v = r["value64"], r["m64"], r["v64"]
    tp, tm, tv = _torch_adam(d["value"].astype(np.float64), grads)
    np.testing.assert_allclose(th, tp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-25)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-30)


def test_zero_gradient_units_follow_torch_sparse_adam():
    """Units with a zero gradient are skipped and t counts every step, as in
    torch.optim.SparseAdam (fed the non-zero entries).  SparseAdam adds eps
    before the bias correction, so eps is made negligible here."""
    d = scenes.adam_inputs(19, 700, 6, state="f32", value_dtype=np.float64, fresh=True)
    rng = np.random.default_rng(6)
    grads = [d["grad"] * rng.random() * 3 for _ in range(5)]
    grads[2] = np.zeros_like(grads[2])                       # a step with no gradient at all
    assert np.mean(grads[0] == 0) > 0.2
    eps = 1e-300
    th, m, v = d["value"].astype(np.float64), d["m"].astype(np.float64), d["v"].astype(np.float64)
    for t, g in enumerate(grads, start=1):
        r = A.adam_step_f32(g, th, m, v, step=t, lr=LR, eps=eps)
        th, m, v = r["value64"], r["m64"], r["v64"]
    p = torch.nn.Parameter(torch.from_numpy(d["value"].astype(np.float64)))
    opt = torch.optim.SparseAdam([p], lr=LR, betas=(B1, B2), eps=eps)
    for g in grads:
        p.grad = torch.from_numpy(np.array(g, dtype=np.float64)).to_sparse()
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-25)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-30)
    never = np.all([g == 0 for g in grads], axis=0)
    assert never.any() and np.array_equal(th[never], d["value"][never])


def test_dense_rule_matches_torch_adam_with_zero_gradient_units():
    """lazy=False is torch.optim.Adam's rule: units whose gradient is zero
    (about 40 % here, and a whole step without any gradient) still decay both
    moments and move by their first moment."""
    d = scenes.adam_inputs(23, 700, 6, state="f32", value_dtype=np.float64, fresh=True)
    rng = np.random.default_rng(7)
    grads = [d["grad"] * rng.random() * 3 for _ in range(5)]
    grads[3] = np.zeros_like(grads[3])
    assert np.mean(grads[0] == 0) > 0.2
    th, m, v = d["value"].astype(np.float64), d["m"].astype(np.float64), d["v"].astype(np.float64)
    for t, g in enumerate(grads, start=1):
        r = A.adam_step_f32(g, th, m, v, step=t, lr=LR, lazy=False)
        th, m, v = r["value64"], r["m64"], r["v64"]
    tp, tm, tv = _torch_adam(d["value"].astype(np.float64), grads)
    np.testing.assert_allclose(th, tp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-25)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-30)
    # the lazy rule leaves exactly the never-seen units where they were; the
    # dense one moves the units seen once and then left alone
    lz = dict(th=d["value"].astype(np.float64), m=d["m"].astype(np.float64), v=d["v"].astype(np.float64))
    for t, g in enumerate(grads, start=1):
        r = A.adam_step_f32(g, lz["th"], lz["m"], lz["v"], step=t, lr=LR, lazy=True)
        lz = dict(th=r["value64"], m=r["m64"], v=r["v64"])
    seen = np.any([g != 0 for g in grads], axis=0)
    assert seen.any() and np.all(np.abs(th - lz["th"])[seen] > 0)


def test_dense_eight_bit_step_matches_torch_adam_on_the_decoded_state():
    """The dense rule on the 8-bit state: torch's Adam from the decoded
    moments on every unit, zero gradients included."""
    d = scenes.adam_inputs(13, 900, 6)
    t = 5
    r = A.adam_step_q8(d["grad"], d["value"], d["m_codes"], d["m_bounds"], d["s_codes"], d["s_bounds"],
                       step=t, lr=LR, lazy=False)
    m0 = A.decode8(d["m_codes"], d["m_bounds"]).astype(np.float64)
    s0 = A.decode8(d["s_codes"], d["s_bounds"]).astype(np.float64)
    v0 = (EPS * np.expm1(s0)) ** 2
    tp, tm, tv = _torch_adam(d["value"].astype(np.float64), [d["grad"]], m0, v0, step0=t - 1)
    assert 0.2 < np.mean(d["grad"] == 0) < 0.6
    np.testing.assert_allclose(r["value64"], tp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["m64"], tm, rtol=1e-12, atol=1e-25)
    np.testing.assert_allclose(r["s64"], np.log1p(np.sqrt(tv) / EPS), rtol=1e-12, atol=1e-12)
    zero = d["grad"] == 0
    assert np.all(r["value64"][zero] != d["value"][zero].astype(np.float64)) or not np.any(m0[zero])


def test_eight_bit_step_matches_torch_adam_on_the_decoded_state():
    """The Adam arithmetic of the 8-bit path: torch's Adam started from the
    decoded moments (v = (eps expm1(s))^2) at the same step count, on the
    units with a gradient; the others keep their value and decoded moments."""
    d = scenes.adam_inputs(12, 900, 6)
    t = 7
    r = A.adam_step_q8(d["grad"], d["value"], d["m_codes"], d["m_bounds"], d["s_codes"], d["s_bounds"],
                       step=t, lr=LR)
    m0 = A.decode8(d["m_codes"], d["m_bounds"]).astype(np.float64)
    s0 = A.decode8(d["s_codes"], d["s_bounds"]).astype(np.float64)
    v0 = (EPS * np.expm1(s0)) ** 2
    tp, tm, tv = _torch_adam(d["value"].astype(np.float64), [d["grad"]], m0, v0, step0=t - 1)
    live = d["grad"] != 0
    assert 0.2 < np.mean(~live) < 0.6
    np.testing.assert_allclose(r["value64"][live], tp[live], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["m64"][live], tm[live], rtol=1e-12, atol=1e-25)
    np.testing.assert_allclose(r["s64"][live], np.log1p(np.sqrt(tv[live]) / EPS), rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["value64"][~live], d["value"][~live].astype(np.float64))
    assert np.array_equal(r["m64"][~live], m0[~live]) and np.array_equal(r["s64"][~live], s0[~live])
    assert np.all(np.abs(r["value"].astype(np.float64) - r["value64"])
                  <= 0.5 * np.spacing(np.abs(r["value"])).astype(np.float64) * (1 + 1e-9))


def test_decode_endpoints():
    d = scenes.adam_inputs(13, 600, 3)
    nb = A.n_blocks(600)
    q = np.zeros((3, 600), dtype=np.uint8)
    lo = np.repeat(d["m_bounds"][:, :, 0], 256, axis=1)[:, :600]
    hi = np.repeat(d["m_bounds"][:, :, 1], 256, axis=1)[:, :600]
    assert np.array_equal(A.decode8(q, d["m_bounds"]), lo)
    top = A.decode8(q + 255, d["m_bounds"]).astype(np.float64)
    scale = np.maximum(np.abs(lo), np.abs(hi)).astype(np.float32)
    assert np.all(np.abs(top - hi) <= 4 * np.spacing(scale))
    assert d["m_bounds"].shape == (3, nb, 2)


@pytest.mark.parametrize("state", ["f32", "q8"])
def test_first_step_from_a_fresh_state_moves_by_lr_times_sign(state):
    """t = 1 from m = v = 0: m' = (1-b1) g, v' = (1-b2) g^2, so the bias-
    corrected step is lr g / (|g| + eps), i.e. lr in the direction -sign(g)."""
    d = scenes.adam_inputs(14, 1000, 6, state=state, value_dtype=np.float32, fresh=True)
    g = d["grad"].astype(np.float64)
    if state == "f32":
        r = A.adam_step_f32(d["grad"], d["value"], d["m"], d["v"], step=1, lr=LR)
    else:
        r = A.adam_step_q8(d["grad"], d["value"], d["m_codes"], d["m_bounds"], d["s_codes"], d["s_bounds"],
                           step=1, lr=LR)
        np.testing.assert_allclose(r["s64"], np.log1p(np.sqrt(1 - B2) * np.abs(g) / EPS), rtol=1e-12)
    np.testing.assert_allclose(r["m64"], (1 - B1) * g, rtol=1e-12, atol=0)
    expect = d["value"].astype(np.float64) - LR * g / (np.abs(g) + EPS)
    np.testing.assert_allclose(r["value64"], expect, rtol=1e-12, atol=1e-18)
    moved = g != 0
    assert np.all(np.sign(d["value"].astype(np.float64) - r["value64"])[moved] == np.sign(g)[moved])
    assert np.all(r["value64"][~moved] == d["value"][~moved])


def test_adam_update_is_invariant_to_gradient_scale():
    """With eps negligible, scaling g and m by c and v by c^2 leaves the
    step unchanged (a transposed moment or a dropped root breaks this)."""
    d = scenes.adam_inputs(15, 500, 3, state="f32", value_dtype=np.float64)
    a = A.adam_step_f32(d["grad"], d["value"], d["m"], d["v"], step=4, lr=LR, eps=1e-300)
    c = 37.5
    g, m, v = (d[k].astype(np.float64) for k in ("grad", "m", "v"))
    b = A.adam_step_f32(g * c, d["value"], m * c, v * c * c, step=4, lr=LR, eps=1e-300)
    upd_a = a["value64"] - d["value"]
    upd_b = b["value64"] - d["value"]
    np.testing.assert_allclose(upd_b, upd_a, rtol=1e-9, atol=1e-18)


def test_log_encoded_ramp_gives_exact_codes():
    """From a fresh state with 1 - b2 = 1/4 (b2 = 0.75) and g chosen so that
    sqrt(v') / eps = e^(0.1 i) - 1, the log-domain value is s' = 0.1 i: the
    block's bounds are (0, 25.5) and unit i gets code i."""
    i = np.arange(256, dtype=np.float64)
    eps = 1e-12
    g = (eps * np.expm1(0.1 * i) / 0.5)[None, :]
    value = np.zeros((1, 256), dtype=np.float32)
    z8 = np.zeros((1, 256), dtype=np.uint8)
    zb = np.zeros((1, 1, 2), dtype=np.float32)
    r = A.adam_step_q8(g, value, z8, zb, z8, zb, step=1, lr=LR, beta2=0.75, eps=eps)
    np.testing.assert_allclose(r["s64"][0], 0.1 * i, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["s_bounds64"][0, 0], [0.0, 25.5], rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["s_codes"][0], np.arange(256, dtype=np.uint8))
    # the first moment (1 - b1) g rises with i too: codes 0 .. 255, never falling
    assert r["m_codes"][0, 0] == 0 and r["m_codes"][0, -1] == 255
    assert np.all(np.diff(r["m_codes"][0].astype(int)) >= 0)


def test_blocks_are_local_and_the_tail_block_is_its_own():
    n = 1000                                      # blocks of 256, 256, 256, 232
    d = scenes.adam_inputs(16, n, 3)
    args = (d["value"], d["m_codes"], d["m_bounds"], d["s_codes"], d["s_bounds"])
    r = A.adam_step_q8(d["grad"], *args, step=3, lr=LR)
    for key, x in (("m", r["m64"]), ("s", r["s64"])):
        for b in range(4):
            sl = slice(b * 256, min(n, b * 256 + 256))
            assert r[key + "_bounds64"][1, b, 0] == x[1, sl].min()
            assert r[key + "_bounds64"][1, b, 1] == x[1, sl].max()
            c = r[key + "_codes"][1, sl]
            assert c[np.argmin(x[1, sl])] == 0 and c[np.argmax(x[1, sl])] == 255
    g2 = d["grad"].copy()
    g2[1, 520] *= -50.0                           # one unit of block 2 of row 1
    r2 = A.adam_step_q8(g2, *args, step=3, lr=LR)
    for key in ("m_codes", "s_codes"):
        same = np.ones((3, n), dtype=bool)
        same[1, 512:768] = False
        assert np.array_equal(r[key][same], r2[key][same])
        assert not np.array_equal(r[key][1, 512:768], r2[key][1, 512:768])
    # permuting the units of one block permutes their codes
    perm = np.random.default_rng(3).permutation(256)
    gp, vp = d["grad"].copy(), d["value"].copy()
    mcp, scp = d["m_codes"].copy(), d["s_codes"].copy()
    for a_ in (gp, vp, mcp, scp):
        a_[0, 256:512] = a_[0, 256:512][perm]
    r3 = A.adam_step_q8(gp, vp, mcp, d["m_bounds"], scp, d["s_bounds"], step=3, lr=LR)
    assert np.array_equal(r3["m_codes"][0, 256:512], r["m_codes"][0, 256:512][perm])
    assert np.array_equal(r3["s_codes"][0, 256:512], r["s_codes"][0, 256:512][perm])


def test_round_trip_error_is_at_most_half_a_step():
    d = scenes.adam_inputs(17, 3000, 6)
    r = A.adam_step_q8(d["grad"], d["value"], d["m_codes"], d["m_bounds"], d["s_codes"], d["s_bounds"],
                       step=50, lr=LR)
    blk = np.arange(3000) // 256
    for key in ("m", "s"):
        x = r[key + "64"]
        dec = A.decode8(r[key + "_codes"], r[key + "_bounds"]).astype(np.float64)
        b = r[key + "_bounds64"]
        half = 0.5 * (b[:, blk, 1] - b[:, blk, 0]) / 255.0
        scale = np.maximum(np.abs(b[:, blk, 0]), np.abs(b[:, blk, 1]))
        assert np.all(np.abs(dec - x) <= half * (1 + 1e-5) + 1e-6 * scale), key
    # constant blocks of the input decode to their bound, and a block whose new
    # values are all equal gets codes 0 with lo == hi
    z = scenes.adam_inputs(18, 256, 1, fresh=True)
    rz = A.adam_step_q8(np.zeros((1, 256), np.float32), z["value"], z["m_codes"], z["m_bounds"],
                        z["s_codes"], z["s_bounds"], step=2, lr=LR)
    assert np.all(rz["m_codes"] == 0) and np.all(rz["s_codes"] == 0)
    assert np.all(rz["m_bounds64"] == 0) and np.all(rz["s_bounds64"] == 0)
    assert np.array_equal(rz["value"], z["value"])
