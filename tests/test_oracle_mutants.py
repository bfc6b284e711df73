"""Planted mistakes: each case copies the oracle's C sources, plants one
plausible mistake (a dropped term, a flipped sign, a removed branch, a
transposed index), builds the copy with the oracle's own flags and runs the
pins of tests/test_oracle_pins.py against it in a subprocess.  The pins must
fail on every mutant; a mutant that passes is a part of the oracle that no
pin guards.  CPU only; the broken copies live in a temporary directory and
are loaded through GS_ORACLE_LIB, never by anything else."""

import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

# (id, file, text as written, the mistake, -k expression of the pins to run)
MUTANTS = [
    # the backward branches that hold a forward decision
    ("guard_x_clamped_sign", "gs_oracle.c",
     "dp[2] += dJ[0][2] * (fx * (xg / z) / (z * z));", "dp[2] -= dJ[0][2] * (fx * (xg / z) / (z * z));",
     "finite"),
    ("guard_y_clamped_sign", "gs_oracle.c",
     "dp[2] += dJ[1][2] * (fy * (yg / z) / (z * z));", "dp[2] -= dJ[1][2] * (fy * (yg / z) / (z * z));",
     "finite"),
    ("guard_x_clamped_dropped", "gs_oracle.c",
     "dp[2] += dJ[0][2] * (fx * (xg / z) / (z * z));", "(void)xg;", "finite"),
    ("guard_x_unclamped_as_clamped", "gs_oracle.c", "if (!clx) {", "if (0) {", "finite"),
    ("cap_test_removed", "gs_oracle.c", "if (raw < cap) {", "if (1) {", "finite"),
    ("colour_clamp_skip_removed", "gs_oracle.c", "if ((clamped[g] >> ch) & 1u) continue;", "", "finite"),
    # backward arithmetic
    ("alpha_grad_suffix_sign", "gs_oracle.c", "dl_dalpha += Tk * (col - S) * G[ch];",
     "dl_dalpha += Tk * (col + S) * G[ch];", "finite"),
    ("conic_b_factor", "gs_oracle.c", "ac[3] += dl_dpower * (-dx * dy);",
     "ac[3] += dl_dpower * (-0.5 * dx * dy);", "finite"),
    ("inverse_grad_sign", "gs_oracle.c", "dS2[i][j] = -(QA[i][0] * Q[0][j] + QA[i][1] * Q[1][j]);",
     "dS2[i][j] = (QA[i][0] * Q[0][j] + QA[i][1] * Q[1][j]);", "finite"),
    ("quat_normalisation_projection_dropped", "gs_oracle.c", "(dqh[r] - qh[r] * dot) / qn", "dqh[r] / qn",
     "finite"),
    ("logit_chain_dropped", "gs_oracle.c", "opac[g] * (1.0 - opac[g]) * go", "opac[g] * go", "finite"),
    ("view_direction_tangent_dropped", "gs_oracle.c", "(dd[r] - d[r] * ddot) / dn", "dd[r] / dn", "finite"),
    ("scale_grad_transposed", "gs_oracle.c", "ds[j] += R[i][j] * dM[i][j];", "ds[j] += R[j][i] * dM[i][j];",
     "finite"),
    # forward
    ("dilation_value", "project_real.h", "const REAL p00 = C00 + (REAL)0.3;", "const REAL p00 = C00 + (REAL)0.35;",
     "closed_form or analytic"),
    ("jacobian_third_column_sign", "project_real.h", "const REAL J02 = -((fx * xg) / zz);",
     "const REAL J02 = ((fx * xg) / zz);", "monte_carlo"),
    ("guard_not_applied", "project_real.h", "const REAL xg = FMIN(FMAX(tx, -lx), lx) * z;",
     "const REAL xg = tx * z;", "guard"),
    ("alpha_cap_value", "gs_oracle.c", "const double a_thr = 1.0 / 255.0, t_thr = 1e-4, cap = 0.99;\n    double T",
     "const double a_thr = 1.0 / 255.0, t_thr = 1e-4, cap = 0.995;\n    double T", "occlusion or analytic"),
    ("transmittance_not_applied", "gs_oracle.c", "for (int ch = 0; ch < 3; ch++) C[ch] += alpha * T * rgb[ch * n + g];",
     "for (int ch = 0; ch < 3; ch++) C[ch] += alpha * rgb[ch * n + g];", "occlusion or unity"),
    ("stop_after_instead_of_before", "gs_oracle.c", "int stop = T < t_thr;", "int stop = T * 0.5 < t_thr;",
     "occlusion or brute_force"),
    ("sh_basis_sign", "gs_oracle.c", "Y[5] = -c2a * y * z;", "Y[5] = c2a * y * z;", "sh_basis"),
    ("depth_ties_reversed", "gs_oracle.c", "if (a->g != b->g) return a->g < b->g ? -1 : 1;",
     "if (a->g != b->g) return a->g > b->g ? -1 : 1;", "binning"),
    ("radius_sqrt_dropped", "project_real.h", "REAL rf = CEIL((REAL)3.0 * SQRT(lam));",
     "REAL rf = CEIL((REAL)3.0 * lam);", "closed_form or rect"),
    # the reached-tile binning
    ("reach_edge_vertex_sign", "gs_oracle.c", "const double dy = fmin(fmax(-b * dx / c, y0), y1);",
     "const double dy = fmin(fmax(b * dx / c, y0), y1);", "reach"),
    ("reach_cross_term_factor", "gs_oracle.c",
     "        best = fmin(best, a * dx * dx + 2.0 * b * dx * dy + c * dy * dy);\n    }\n    for",
     "        best = fmin(best, a * dx * dx + b * dx * dy + c * dy * dy);\n    }\n    for", "reach"),
    ("reach_inside_test_dropped", "gs_oracle.c",
     "if (x0 <= 0.0 && 0.0 <= x1 && y0 <= 0.0 && 0.0 <= y1) return 0.0;", "", "reach"),
    ("reach_box_one_pixel_short", "gs_oracle.c", "return o * exp(-0.5 * box_min_q(a, b, c, x0, x0 + 15.0, y0, y0 + 15.0));",
     "return o * exp(-0.5 * box_min_q(a, b, c, x0, x0 + 14.0, y0, y0 + 15.0));", "reach"),
    ("reach_threshold_without_margin", "gs_oracle.c", "const double reach_min = (1.0 / 255.0) * (1.0 - 1e-3);",
     "const double reach_min = (1.0 / 255.0) * (1.0 + 1e-3);", "reach"),
]


def _build_mutant(tmp, fname, old, new):
    for f in obuild.SOURCES + obuild.HEADERS:
        shutil.copy(os.path.join(ORACLE, f), os.path.join(tmp, f))
    path = os.path.join(tmp, fname)
    src = open(path).read()
    assert src.count(old) == 1, f"the text to mutate must occur once in {fname}: {old!r}"
    open(path, "w").write(src.replace(old, new))
    lib = os.path.join(tmp, "liboracle_mutant.so")
    subprocess.run(["gcc"] + obuild.CFLAGS + ["-o", lib] + [os.path.join(tmp, s) for s in obuild.SOURCES] + ["-lm"],
                   check=True, capture_output=True)
    return lib


@pytest.mark.slow
@pytest.mark.parametrize("mid,fname,old,new,kexpr", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_fail_on_planted_mistake(mid, fname, old, new, kexpr):
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, fname, old, new)
        env = dict(os.environ, GS_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                            "-x", "-q", "-p", "no:cacheprovider", "-k", kexpr],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    tail = (r.stdout + r.stderr)[-1500:]
    assert "passed" in tail or "failed" in tail or "error" in tail, tail
    assert r.returncode == 1 and " failed" in tail, f"pins did not catch mutant {mid}:\n{tail}"
