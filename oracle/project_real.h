/*
 * Projection of one Gaussian, written once for a scalar type REAL and
 * included twice by gs_oracle.c (REAL = float: the fp32 op-order contract;
 * REAL = double: the smooth fp64 function).  TEST INFRASTRUCTURE ONLY.
 *
 * Every line is one operation at a time, left to right as written, with no
 * fused multiply-add (the file is compiled with -ffp-contract=off).  Both
 * types use correctly rounded +, -, *, / and sqrt.
 *
 * The steps, in order (readings, since the pages give no formulas):
 *   P0 cull non-finite inputs, a zero quaternion, and inactive Gaussians;
 *   P1 camera space p = R mu + t; cull z <= znear (near plane 0.2);
 *   P1b distance-LOD gate (when enabled): cull when the undilated 3-sigma
 *       pinhole radius 3 f max(s) / |mu - c| is below lod_px (BlitzGS
 *       page, section 2.3: far Gaussians that cover too few pixels leave the
 *       per-view active set);
 *   P2 image mean u = fx x/z + cx, v = fy y/z + cy (pixel (i,j) covers
 *       [i,i+1) x [j,j+1));
 *   P3 Sigma = M M^T with M = R(q/|q|) diag(s);
 *   P4 Jacobian of the pinhole map at the mean, with x/z and y/z clamped to
 *       guard x the half field of view (keeps Gaussians just past the near
 *       plane at the frame edge from blowing up);
 *   P5 Sigma2 = (J W) Sigma (J W)^T, W the camera rotation (EWA);
 *   P6 Sigma' = Sigma2 + 0.3 I (low-pass dilation, px^2);
 *   P7 conic = inverse of Sigma'; cull det <= 0;
 *   P8 r = ceil(3 sqrt(lambda_max(Sigma'))), at most 2^24;
 *   P9 tile rect of the square [u-r, u+r] x [v-r, v+r], half-open, clamped
 *       to the tile grid; cull when empty;
 *   P10 colour max(0, 0.5 + sum_j k_j Y_j(d)), d the unit view direction
 *       (fp64 in both builds).
 */

static int FN(project_one)(int64_t g, int64_t n, const REAL *means,
                           const REAL *scales, const REAL *quats,
                           const REAL *opac, const uint8_t *active,
                           const orc_cam *cam, REAL out_f[8], int32_t out_i[6])
{
    /* out_f: u, v, z, conic a, b, c, opacity, (unused)
     * out_i: radius, x0, x1, y0, y1, tiles */
    const REAL mx = means[g], my = means[n + g], mz = means[2 * n + g];
    const REAL sx = scales[g], sy = scales[n + g], sz = scales[2 * n + g];
    const REAL qw = quats[g], qx = quats[n + g], qy = quats[2 * n + g], qz = quats[3 * n + g];
    const REAL o = opac[g];

    /* P0 */
    if (active && !active[g]) return 0;
    if (!isfinite(mx) || !isfinite(my) || !isfinite(mz) || !isfinite(sx) ||
        !isfinite(sy) || !isfinite(sz) || !isfinite(qw) || !isfinite(qx) ||
        !isfinite(qy) || !isfinite(qz) || !isfinite(o))
        return 0;

    const REAL R00 = (REAL)cam->viewmat[0], R01 = (REAL)cam->viewmat[1], R02 = (REAL)cam->viewmat[2];
    const REAL t0 = (REAL)cam->viewmat[3];
    const REAL R10 = (REAL)cam->viewmat[4], R11 = (REAL)cam->viewmat[5], R12 = (REAL)cam->viewmat[6];
    const REAL t1 = (REAL)cam->viewmat[7];
    const REAL R20 = (REAL)cam->viewmat[8], R21 = (REAL)cam->viewmat[9], R22 = (REAL)cam->viewmat[10];
    const REAL t2 = (REAL)cam->viewmat[11];
    const REAL fx = (REAL)cam->fx, fy = (REAL)cam->fy, cx = (REAL)cam->cx, cy = (REAL)cam->cy;

    /* P1 */
    REAL x = R00 * mx;  x = x + R01 * my;  x = x + R02 * mz;  x = x + t0;
    REAL y = R10 * mx;  y = y + R11 * my;  y = y + R12 * mz;  y = y + t1;
    REAL z = R20 * mx;  z = z + R21 * my;  z = z + R22 * mz;  z = z + t2;
    if (!(z > (REAL)cam->znear)) return 0;

    /* P1b: camera centre c = -R^T t, distance |mu - c| */
    if (cam->lod_px > 0.0) {
        REAL ccx = R00 * t0;  ccx = ccx + R10 * t1;  ccx = ccx + R20 * t2;  ccx = -ccx;
        REAL ccy = R01 * t0;  ccy = ccy + R11 * t1;  ccy = ccy + R21 * t2;  ccy = -ccy;
        REAL ccz = R02 * t0;  ccz = ccz + R12 * t1;  ccz = ccz + R22 * t2;  ccz = -ccz;
        const REAL dx = mx - ccx, dy = my - ccy, dz = mz - ccz;
        REAL d2 = dx * dx;  d2 = d2 + dy * dy;  d2 = d2 + dz * dz;
        const REAL dist = SQRT(d2);
        const REAL smax = FMAX(FMAX(sx, sy), sz);
        const REAL f = FMAX(fx, fy);
        const REAL lhs = ((REAL)3.0 * f) * smax;      /* 3 f max(s)        */
        const REAL rhs = (REAL)cam->lod_px * dist;      /* lod_px |mu - c|   */
        if (lhs < rhs) return 0;
    }

    /* P2 */
    const REAL tx = x / z, ty = y / z;
    const REAL u = fx * tx + cx;
    const REAL v = fy * ty + cy;

    /* P3: normalised quaternion, rotation, M = R diag(s), Sigma = M M^T */
    REAL nq2 = qw * qw;  nq2 = nq2 + qx * qx;  nq2 = nq2 + qy * qy;  nq2 = nq2 + qz * qz;
    if (!(nq2 > (REAL)0.0)) return 0;
    const REAL nq = SQRT(nq2);
    const REAL w = qw / nq, a = qx / nq, b = qy / nq, c = qz / nq;
    /* rotation of the unit quaternion (w, a, b, c) */
    const REAL q00 = (REAL)1.0 - (REAL)2.0 * (b * b + c * c);
    const REAL q01 = (REAL)2.0 * (a * b - w * c);
    const REAL q02 = (REAL)2.0 * (a * c + w * b);
    const REAL q10 = (REAL)2.0 * (a * b + w * c);
    const REAL q11 = (REAL)1.0 - (REAL)2.0 * (a * a + c * c);
    const REAL q12 = (REAL)2.0 * (b * c - w * a);
    const REAL q20 = (REAL)2.0 * (a * c - w * b);
    const REAL q21 = (REAL)2.0 * (b * c + w * a);
    const REAL q22 = (REAL)1.0 - (REAL)2.0 * (a * a + b * b);
    const REAL M00 = q00 * sx, M01 = q01 * sy, M02 = q02 * sz;
    const REAL M10 = q10 * sx, M11 = q11 * sy, M12 = q12 * sz;
    const REAL M20 = q20 * sx, M21 = q21 * sy, M22 = q22 * sz;
    const REAL S00 = (M00 * M00 + M01 * M01) + M02 * M02;
    const REAL S01 = (M00 * M10 + M01 * M11) + M02 * M12;
    const REAL S02 = (M00 * M20 + M01 * M21) + M02 * M22;
    const REAL S11 = (M10 * M10 + M11 * M11) + M12 * M12;
    const REAL S12 = (M10 * M20 + M11 * M21) + M12 * M22;
    const REAL S22 = (M20 * M20 + M21 * M21) + M22 * M22;

    /* P4 */
    const REAL lx = (REAL)cam->guard * (((REAL)0.5 * (REAL)cam->width) / fx);
    const REAL ly = (REAL)cam->guard * (((REAL)0.5 * (REAL)cam->height) / fy);
    const REAL xg = FMIN(FMAX(tx, -lx), lx) * z;
    const REAL yg = FMIN(FMAX(ty, -ly), ly) * z;
    const REAL zz = z * z;
    const REAL J00 = fx / z;
    const REAL J02 = -((fx * xg) / zz);
    const REAL J11 = fy / z;
    const REAL J12 = -((fy * yg) / zz);

    /* P5: T = J W (2x3), U = T Sigma, Sigma2 = U T^T */
    const REAL T00 = J00 * R00 + J02 * R20, T01 = J00 * R01 + J02 * R21, T02 = J00 * R02 + J02 * R22;
    const REAL T10 = J11 * R10 + J12 * R20, T11 = J11 * R11 + J12 * R21, T12 = J11 * R12 + J12 * R22;
    const REAL U00 = (T00 * S00 + T01 * S01) + T02 * S02;
    const REAL U01 = (T00 * S01 + T01 * S11) + T02 * S12;
    const REAL U02 = (T00 * S02 + T01 * S12) + T02 * S22;
    const REAL U10 = (T10 * S00 + T11 * S01) + T12 * S02;
    const REAL U11 = (T10 * S01 + T11 * S11) + T12 * S12;
    const REAL U12 = (T10 * S02 + T11 * S12) + T12 * S22;
    const REAL C00 = (U00 * T00 + U01 * T01) + U02 * T02;
    const REAL C01 = (U00 * T10 + U01 * T11) + U02 * T12;
    const REAL C11 = (U10 * T10 + U11 * T11) + U12 * T12;

    /* P6 */
    const REAL p00 = C00 + (REAL)0.3;
    const REAL p01 = C01;
    const REAL p11 = C11 + (REAL)0.3;

    /* P7 */
    const REAL det = p00 * p11 - p01 * p01;
    if (!(det > (REAL)0.0)) return 0;
    const REAL ca = p11 / det;
    const REAL cb = -(p01 / det);
    const REAL cc = p00 / det;

    /* P8 */
    const REAL mid = (REAL)0.5 * (p00 + p11);
    const REAL disc = FMAX((REAL)0.0, mid * mid - det);
    const REAL lam = mid + SQRT(disc);
    REAL rf = CEIL((REAL)3.0 * SQRT(lam));
    rf = FMIN(rf, (REAL)16777216.0);

    /* P9 */
    const REAL TXf = (REAL)((cam->width + 15) / 16), TYf = (REAL)((cam->height + 15) / 16);
    REAL fx0 = FLOOR((u - rf) / (REAL)16.0);
    REAL fx1 = FLOOR((u + rf) / (REAL)16.0) + (REAL)1.0;
    REAL fy0 = FLOOR((v - rf) / (REAL)16.0);
    REAL fy1 = FLOOR((v + rf) / (REAL)16.0) + (REAL)1.0;
    fx0 = FMIN(FMAX(fx0, (REAL)0.0), TXf);
    fx1 = FMIN(FMAX(fx1, (REAL)0.0), TXf);
    fy0 = FMIN(FMAX(fy0, (REAL)0.0), TYf);
    fy1 = FMIN(FMAX(fy1, (REAL)0.0), TYf);
    const int32_t x0 = (int32_t)fx0, x1 = (int32_t)fx1, y0 = (int32_t)fy0, y1 = (int32_t)fy1;
    if (x0 >= x1 || y0 >= y1) return 0;

    out_f[0] = u;  out_f[1] = v;  out_f[2] = z;
    out_f[3] = ca; out_f[4] = cb; out_f[5] = cc; out_f[6] = o; out_f[7] = 0;
    out_i[0] = (int32_t)rf;
    out_i[1] = x0; out_i[2] = x1; out_i[3] = y0; out_i[4] = y1;
    out_i[5] = (x1 - x0) * (y1 - y0);
    return 1;
}

void FN(orc_project)(int64_t n, const REAL *means, const REAL *scales,
                     const REAL *quats, const REAL *opac, int sh_degree,
                     const REAL *sh, const uint8_t *active, const orc_cam *cam,
                     orc_proj_out *out)
{
    const int K = (sh_degree + 1) * (sh_degree + 1);
    double cc[3];
    camera_centre(cam, cc);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n; g++) {
        REAL f[8];
        int32_t iv[6];
        const int vis = FN(project_one)(g, n, means, scales, quats, opac, active, cam, f, iv);
        out->clamped[g] = 0;
        if (!vis) {
            /* P11 reading: a culled Gaussian has every record field zero */
            out->u[g] = out->v[g] = out->z[g] = 0.0;
            out->radius[g] = 0;
            for (int k = 0; k < 4; k++) out->rect[k * n + g] = 0;
            for (int k = 0; k < 3; k++) {
                out->conic[k * n + g] = 0.0;
                out->rgb[k * n + g] = 0.0;
                out->rgb_raw[k * n + g] = 0.0;
            }
            out->opacity[g] = 0.0;
            out->tiles[g] = 0;
            continue;
        }
        out->u[g] = (double)f[0];
        out->v[g] = (double)f[1];
        out->z[g] = (double)f[2];
        out->conic[g] = (double)f[3];
        out->conic[n + g] = (double)f[4];
        out->conic[2 * n + g] = (double)f[5];
        out->opacity[g] = (double)f[6];
        out->radius[g] = iv[0];
        for (int k = 0; k < 4; k++) out->rect[k * n + g] = iv[1 + k];
        out->tiles[g] = iv[5];

        /* P10, fp64: unit view direction from the camera centre */
        double d[3] = {(double)means[g] - cc[0], (double)means[n + g] - cc[1],
                       (double)means[2 * n + g] - cc[2]};
        const double dn = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
        d[0] /= dn; d[1] /= dn; d[2] /= dn;
        double Y[16], dY[48];
        orc_sh_basis(d, Y, dY);
        for (int ch = 0; ch < 3; ch++) {
            double s = 0.0;
            for (int j = 0; j < K; j++) s += (double)sh[((int64_t)j * 3 + ch) * n + g] * Y[j];
            const double val = 0.5 + s;
            out->rgb_raw[ch * n + g] = val;
            if (val < 0.0) out->clamped[g] |= (uint8_t)(1u << ch);
            out->rgb[ch * n + g] = val < 0.0 ? 0.0 : val;
        }
    }
}
