// Projection + SH colour (forward) and its chain rule (backward), gfx950.
//
// One lane per Gaussian; the parameters are structure-of-arrays so every load
// of a wave is one contiguous 256-byte (fp32) or 128-byte (fp16 SH) segment.
// The projection is HBM-bound: 44 bytes of geometry in, 48 bytes of record
// out, plus the SH block (12 K or 6 K bytes) for Gaussians that survive the
// culls.
//
// Numerics: everything here is compiled without floating-point contraction,
// so each +, -, * is one correctly rounded fp32 operation taken in the written
// order; / and sqrt are correctly rounded (the HIP default on gfx950).  The
// quantities that decide the tile lists (camera-space position, u, v, the 2D
// covariance, conic, radius, rect) are therefore reproducible bit for bit by
// any IEEE fp32 evaluation of the same sequence.  The sequence (EWA splatting
// with a dilation of the 2D covariance; the pages name the method but give no
// formula) is:
//   p = R mu + t                          (sums left to right)
//   u = fx (x/z) + cx,  v = fy (y/z) + cy
//   q <- q / |q|,  Rq from q,  M = Rq diag(s),  Sigma = M M^T
//   J = [[fx/z, 0, -fx xg/z^2], [0, fy/z, -fy yg/z^2]],
//       xg = clamp(x/z, +-guard*W/(2 fx)) z, likewise yg
//   T = J R,  Sigma2 = T Sigma T^T,  Sigma' = Sigma2 + 0.3 I
//   conic = Sigma'^-1,  r = ceil(3 sqrt(m + sqrt(max(0, m^2 - det)))), m the
//   mean of the diagonal.
#pragma clang fp contract(off)

#include "gs_internal.h"

namespace gsi {
namespace {

struct Geo {
    float x, y, z, tx, ty;
    float w, qa, qb, qc, nq;          // normalised quaternion and |q|
    float Rq[9];
    float M[9];
    float S[6];                      // Sigma: 00 01 02 11 12 22
    float J00, J02, J11, J12;
    bool clx, cly;
    float T[6];                      // T = J R, rows 0 and 1
    float p00, p01, p11, det;
    float u, v;
};

// Geometry of one Gaussian; returns false when it is culled before the rect.
__device__ __forceinline__ bool geometry(const Cam &cam, float mx, float my, float mz, float sx,
                                         float sy, float sz, float qw, float qx, float qy, float qz,
                                         Geo &o)
{
    const float *R = cam.R;
    float x = R[0] * mx;  x = x + R[1] * my;  x = x + R[2] * mz;  x = x + cam.t[0];
    float y = R[3] * mx;  y = y + R[4] * my;  y = y + R[5] * mz;  y = y + cam.t[1];
    float z = R[6] * mx;  z = z + R[7] * my;  z = z + R[8] * mz;  z = z + cam.t[2];
    if (!(z > cam.znear)) return false;
    o.x = x; o.y = y; o.z = z;

    o.tx = x / z;
    o.ty = y / z;
    o.u = cam.fx * o.tx + cam.cx;
    o.v = cam.fy * o.ty + cam.cy;

    float nq2 = qw * qw;  nq2 = nq2 + qx * qx;  nq2 = nq2 + qy * qy;  nq2 = nq2 + qz * qz;
    if (!(nq2 > 0.0f)) return false;
    const float nq = sqrtf(nq2);
    const float w = qw / nq, a = qx / nq, b = qy / nq, c = qz / nq;
    o.w = w; o.qa = a; o.qb = b; o.qc = c; o.nq = nq;
    float *Q = o.Rq;
    Q[0] = 1.0f - 2.0f * (b * b + c * c);
    Q[1] = 2.0f * (a * b - w * c);
    Q[2] = 2.0f * (a * c + w * b);
    Q[3] = 2.0f * (a * b + w * c);
    Q[4] = 1.0f - 2.0f * (a * a + c * c);
    Q[5] = 2.0f * (b * c - w * a);
    Q[6] = 2.0f * (a * c - w * b);
    Q[7] = 2.0f * (b * c + w * a);
    Q[8] = 1.0f - 2.0f * (a * a + b * b);
    float *M = o.M;
    M[0] = Q[0] * sx; M[1] = Q[1] * sy; M[2] = Q[2] * sz;
    M[3] = Q[3] * sx; M[4] = Q[4] * sy; M[5] = Q[5] * sz;
    M[6] = Q[6] * sx; M[7] = Q[7] * sy; M[8] = Q[8] * sz;
    float *S = o.S;
    S[0] = (M[0] * M[0] + M[1] * M[1]) + M[2] * M[2];
    S[1] = (M[0] * M[3] + M[1] * M[4]) + M[2] * M[5];
    S[2] = (M[0] * M[6] + M[1] * M[7]) + M[2] * M[8];
    S[3] = (M[3] * M[3] + M[4] * M[4]) + M[5] * M[5];
    S[4] = (M[3] * M[6] + M[4] * M[7]) + M[5] * M[8];
    S[5] = (M[6] * M[6] + M[7] * M[7]) + M[8] * M[8];

    const float lx = cam.guard * ((0.5f * (float)cam.width) / cam.fx);
    const float ly = cam.guard * ((0.5f * (float)cam.height) / cam.fy);
    o.clx = (o.tx < -lx) || (o.tx > lx);
    o.cly = (o.ty < -ly) || (o.ty > ly);
    const float xg = fminf(fmaxf(o.tx, -lx), lx) * z;
    const float yg = fminf(fmaxf(o.ty, -ly), ly) * z;
    const float zz = z * z;
    o.J00 = cam.fx / z;
    o.J02 = -((cam.fx * xg) / zz);
    o.J11 = cam.fy / z;
    o.J12 = -((cam.fy * yg) / zz);

    float *T = o.T;
    T[0] = o.J00 * R[0] + o.J02 * R[6];
    T[1] = o.J00 * R[1] + o.J02 * R[7];
    T[2] = o.J00 * R[2] + o.J02 * R[8];
    T[3] = o.J11 * R[3] + o.J12 * R[6];
    T[4] = o.J11 * R[4] + o.J12 * R[7];
    T[5] = o.J11 * R[5] + o.J12 * R[8];
    // U = T Sigma (Sigma symmetric: S01 = S10 ...)
    const float U00 = (T[0] * S[0] + T[1] * S[1]) + T[2] * S[2];
    const float U01 = (T[0] * S[1] + T[1] * S[3]) + T[2] * S[4];
    const float U02 = (T[0] * S[2] + T[1] * S[4]) + T[2] * S[5];
    const float U10 = (T[3] * S[0] + T[4] * S[1]) + T[5] * S[2];
    const float U11 = (T[3] * S[1] + T[4] * S[3]) + T[5] * S[4];
    const float U12 = (T[3] * S[2] + T[4] * S[4]) + T[5] * S[5];
    const float C00 = (U00 * T[0] + U01 * T[1]) + U02 * T[2];
    const float C01 = (U00 * T[3] + U01 * T[4]) + U02 * T[5];
    const float C11 = (U10 * T[3] + U11 * T[4]) + U12 * T[5];
    o.p00 = C00 + 0.3f;
    o.p01 = C01;
    o.p11 = C11 + 0.3f;
    o.det = o.p00 * o.p11 - o.p01 * o.p01;
    return o.det > 0.0f;
}

__device__ __forceinline__ bool all_finite(float a, float b, float c, float d, float e, float f,
                                           float g, float h, float i, float j, float k)
{
    return isfinite(a) && isfinite(b) && isfinite(c) && isfinite(d) && isfinite(e) && isfinite(f) &&
           isfinite(g) && isfinite(h) && isfinite(i) && isfinite(j) && isfinite(k);
}

// Real SH basis, degree <= 3, band order l = 0..3, m = -l..l, with the sign
// (-1)^|m| relative to the phase-free textbook basis (the convention of
// common 3DGS coefficient files).  Constants: sqrt((2l+1)/(4 pi)
// (l-|m|)!/(l+|m|)!) times the Legendre factors.
struct SH {
    static constexpr float c0 = 0.282094791773878f;
    static constexpr float c1 = 0.488602511902920f;
    static constexpr float c2a = 1.092548430592079f;
    static constexpr float c2b = 0.315391565252520f;
    static constexpr float c2c = 0.546274215296040f;
    static constexpr float c3a = 0.590043589926644f;
    static constexpr float c3b = 2.890611442640554f;
    static constexpr float c3c = 0.457045799464466f;
    static constexpr float c3d = 0.373176332590115f;
    static constexpr float c3e = 1.445305721320277f;
};

__device__ __forceinline__ void sh_basis(int K, float x, float y, float z, float *Y)
{
    Y[0] = SH::c0;
    if (K > 1) {
        Y[1] = -SH::c1 * y;
        Y[2] = SH::c1 * z;
        Y[3] = -SH::c1 * x;
    }
    if (K > 4) {
        const float xx = x * x, yy = y * y, zz = z * z;
        Y[4] = SH::c2a * (x * y);
        Y[5] = -SH::c2a * (y * z);
        Y[6] = SH::c2b * (2.0f * zz - xx - yy);
        Y[7] = -SH::c2a * (x * z);
        Y[8] = SH::c2c * (xx - yy);
        if (K > 9) {
            Y[9] = -SH::c3a * y * (3.0f * xx - yy);
            Y[10] = SH::c3b * (x * y) * z;
            Y[11] = -SH::c3c * y * (4.0f * zz - xx - yy);
            Y[12] = SH::c3d * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
            Y[13] = -SH::c3c * x * (4.0f * zz - xx - yy);
            Y[14] = SH::c3e * z * (xx - yy);
            Y[15] = -SH::c3a * x * (xx - 3.0f * yy);
        }
    }
}

// d Y_j / d(x, y, z) for the same basis.
__device__ __forceinline__ void sh_basis_grad(int K, float x, float y, float z, float (*g)[3])
{
    for (int j = 0; j < 16; j++) g[j][0] = g[j][1] = g[j][2] = 0.0f;
    if (K > 1) {
        g[1][1] = -SH::c1;
        g[2][2] = SH::c1;
        g[3][0] = -SH::c1;
    }
    if (K > 4) {
        const float xx = x * x, yy = y * y, zz = z * z;
        g[4][0] = SH::c2a * y;  g[4][1] = SH::c2a * x;
        g[5][1] = -SH::c2a * z; g[5][2] = -SH::c2a * y;
        g[6][0] = -2.0f * SH::c2b * x; g[6][1] = -2.0f * SH::c2b * y; g[6][2] = 4.0f * SH::c2b * z;
        g[7][0] = -SH::c2a * z; g[7][2] = -SH::c2a * x;
        g[8][0] = 2.0f * SH::c2c * x; g[8][1] = -2.0f * SH::c2c * y;
        if (K > 9) {
            g[9][0] = -SH::c3a * 6.0f * x * y;
            g[9][1] = -SH::c3a * 3.0f * (xx - yy);
            g[10][0] = SH::c3b * y * z; g[10][1] = SH::c3b * x * z; g[10][2] = SH::c3b * x * y;
            g[11][0] = 2.0f * SH::c3c * x * y;
            g[11][1] = -SH::c3c * (4.0f * zz - xx - 3.0f * yy);
            g[11][2] = -8.0f * SH::c3c * y * z;
            g[12][0] = -6.0f * SH::c3d * x * z;
            g[12][1] = -6.0f * SH::c3d * y * z;
            g[12][2] = SH::c3d * (6.0f * zz - 3.0f * xx - 3.0f * yy);
            g[13][0] = -SH::c3c * (4.0f * zz - 3.0f * xx - yy);
            g[13][1] = 2.0f * SH::c3c * x * y;
            g[13][2] = -8.0f * SH::c3c * x * z;
            g[14][0] = 2.0f * SH::c3e * x * z; g[14][1] = -2.0f * SH::c3e * y * z;
            g[14][2] = SH::c3e * (xx - yy);
            g[15][0] = -SH::c3a * 3.0f * (xx - yy);
            g[15][1] = 6.0f * SH::c3a * x * y;
        }
    }
}

template <typename T>
__device__ __forceinline__ float ld_sh(const T *p);
template <>
__device__ __forceinline__ float ld_sh<float>(const float *p) { return __builtin_nontemporal_load(p); }
template <>
__device__ __forceinline__ float ld_sh<__half>(const __half *p) { return __half2float(*p); }

// Camera centre c = -R^T t, sums left to right.
__device__ __forceinline__ void cam_centre(const Cam &cam, float &ccx, float &ccy, float &ccz)
{
    const float *R = cam.R;
    ccx = R[0] * cam.t[0];  ccx = ccx + R[3] * cam.t[1];  ccx = ccx + R[6] * cam.t[2];  ccx = -ccx;
    ccy = R[1] * cam.t[0];  ccy = ccy + R[4] * cam.t[1];  ccy = ccy + R[7] * cam.t[2];  ccy = -ccy;
    ccz = R[2] * cam.t[0];  ccz = ccz + R[5] * cam.t[1];  ccz = ccz + R[8] * cam.t[2];  ccz = -ccz;
}

template <typename TSH>
__global__ __launch_bounds__(kBlock) void project_kernel(
    int n, int K, const float *__restrict__ means, const float *__restrict__ scales,
    const float *__restrict__ quats, const float *__restrict__ opac, const TSH *__restrict__ sh,
    const uint8_t *__restrict__ active, Cam cam, Splat *__restrict__ out)
{
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= n) return;
    const float mx = means[g], my = means[n + g], mz = means[2 * n + g];
    const float sx = scales[g], sy = scales[n + g], sz = scales[2 * n + g];
    const float qw = quats[g], qx = quats[n + g], qy = quats[2 * n + g], qz = quats[3 * n + g];
    const float o = opac[g];

    Splat rec;
    rec.a = rec.b = rec.c = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool vis = (active == nullptr || active[g] != 0) && all_finite(mx, my, mz, sx, sy, sz, qw, qx, qy, qz, o);
    float ccx, ccy, ccz;
    cam_centre(cam, ccx, ccy, ccz);
    Geo G;
    if (vis) vis = geometry(cam, mx, my, mz, sx, sy, sz, qw, qx, qy, qz, G);
    if (vis && cam.lod > 0.0f) {
        // distance-LOD gate: undilated 3-sigma pinhole radius below lod px
        const float dx = mx - ccx, dy = my - ccy, dz = mz - ccz;
        float d2 = dx * dx;  d2 = d2 + dy * dy;  d2 = d2 + dz * dz;
        const float dist = sqrtf(d2);
        const float smax = fmaxf(fmaxf(sx, sy), sz);
        const float f = fmaxf(cam.fx, cam.fy);
        const float lhs = (3.0f * f) * smax;
        const float rhs = cam.lod * dist;
        vis = !(lhs < rhs);
    }
    if (vis) {
        const float ca = G.p11 / G.det;
        const float cb = -(G.p01 / G.det);
        const float cc = G.p00 / G.det;
        const float mid = 0.5f * (G.p00 + G.p11);
        const float disc = fmaxf(0.0f, mid * mid - G.det);
        const float lam = mid + sqrtf(disc);
        float rf = ceilf(3.0f * sqrtf(lam));
        rf = fminf(rf, 16777216.0f);
        const Rect r = tile_rect(G.u, G.v, rf, (float)cam.tiles_x, (float)cam.tiles_y);
        if (r.x0 < r.x1 && r.y0 < r.y1) {
            // colour: SH at the unit view direction
            float dx = mx - ccx, dy = my - ccy, dz = mz - ccz;
            const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
            dx = dx / dn; dy = dy / dn; dz = dz / dn;
            float Y[16];
            sh_basis(K, dx, dy, dz, Y);
            float col[3];
#pragma unroll
            for (int ch = 0; ch < 3; ch++) {
                float s = 0.0f;
                for (int j = 0; j < K; j++) s = s + ld_sh(sh + ((size_t)(j * 3 + ch)) * n + g) * Y[j];
                const float val = 0.5f + s;
                col[ch] = val < 0.0f ? 0.0f : val;
            }
            rec.a = make_float4(G.u, G.v, G.z, __int_as_float((int)rf));
            rec.b = make_float4(ca, cb, cc, o);
            rec.c = make_float4(col[0], col[1], col[2],
                                __uint_as_float((uint32_t)((r.x1 - r.x0) * (r.y1 - r.y0))));
        }
    }
    out[g] = rec;
}

// ---------------------------------------------------------------------------
// Backward: grad2d[9][n] = d/du, d/dv, d/da, d/db, d/dc, d/dopacity, d/drgb
// (from the compositing pass) -> raw parameter gradients, +=.  The forward
// sequence above is recomputed; the guard clamp and the colour clamp keep the
// branch the forward took.
template <typename TSH>
__global__ __launch_bounds__(kBlock) void project_bwd_kernel(
    int n, int K, const float *__restrict__ means, const float *__restrict__ scales,
    const float *__restrict__ quats, const float *__restrict__ opac, const TSH *__restrict__ sh,
    Cam cam, const Splat *__restrict__ splats, const float *__restrict__ grad2d,
    float *__restrict__ d_means, float *__restrict__ d_log_scales, float *__restrict__ d_quats,
    float *__restrict__ d_logits, float *__restrict__ d_sh)
{
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= n) return;
    // culled Gaussians have radius 0 and receive nothing
    const float4 ra = splats[g].a;
    if (__float_as_int(ra.w) == 0) return;
    const float gu = grad2d[g], gv = grad2d[n + g];
    const float ga = grad2d[2 * n + g], gb = grad2d[3 * n + g], gc = grad2d[4 * n + g];
    const float go = grad2d[5 * n + g];
    const float grgb[3] = {grad2d[6 * n + g], grad2d[7 * n + g], grad2d[8 * n + g]};

    const float mx = means[g], my = means[n + g], mz = means[2 * n + g];
    const float s[3] = {scales[g], scales[n + g], scales[2 * n + g]};
    const float qw = quats[g], qx = quats[n + g], qy = quats[2 * n + g], qz = quats[3 * n + g];
    const float o = opac[g];
    Geo G;
    geometry(cam, mx, my, mz, s[0], s[1], s[2], qw, qx, qy, qz, G);
    const float *R = cam.R;
    const float z = G.z;

    // conic = Q = Sigma'^-1:  dSigma' = -Q A Q,  A = [[ga, gb/2], [gb/2, gc]]
    const float q00 = G.p11 / G.det, q01 = -(G.p01 / G.det), q11 = G.p00 / G.det;
    const float A00 = ga, A01 = 0.5f * gb, A11 = gc;
    const float QA00 = q00 * A00 + q01 * A01, QA01 = q00 * A01 + q01 * A11;
    const float QA10 = q01 * A00 + q11 * A01, QA11 = q01 * A01 + q11 * A11;
    const float D00 = -(QA00 * q00 + QA01 * q01);
    const float D01 = -(QA00 * q01 + QA01 * q11);
    const float D11 = -(QA10 * q01 + QA11 * q11);
    // Sigma2 = T Sigma T^T:  dSigma = T^T D T,  dT = 2 D T Sigma
    const float *T = G.T;
    float dS[3][3];
#pragma unroll
    for (int k = 0; k < 3; k++)
#pragma unroll
        for (int l = 0; l < 3; l++)
            dS[k][l] = T[k] * (D00 * T[l] + D01 * T[3 + l]) + T[3 + k] * (D01 * T[l] + D11 * T[3 + l]);
    const float Sg[3][3] = {{G.S[0], G.S[1], G.S[2]}, {G.S[1], G.S[3], G.S[4]}, {G.S[2], G.S[4], G.S[5]}};
    float DT[2][3];
#pragma unroll
    for (int l = 0; l < 3; l++) {
        DT[0][l] = D00 * T[l] + D01 * T[3 + l];
        DT[1][l] = D01 * T[l] + D11 * T[3 + l];
    }
    float dT[2][3];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int k = 0; k < 3; k++)
            dT[i][k] = 2.0f * (DT[i][0] * Sg[0][k] + DT[i][1] * Sg[1][k] + DT[i][2] * Sg[2][k]);
    // T = J R:  dJ = dT R^T (only the non-zero entries of J matter)
    const float dJ00 = dT[0][0] * R[0] + dT[0][1] * R[1] + dT[0][2] * R[2];
    const float dJ02 = dT[0][0] * R[6] + dT[0][1] * R[7] + dT[0][2] * R[8];
    const float dJ11 = dT[1][0] * R[3] + dT[1][1] * R[4] + dT[1][2] * R[5];
    const float dJ12 = dT[1][0] * R[6] + dT[1][1] * R[7] + dT[1][2] * R[8];

    const float fx = cam.fx, fy = cam.fy;
    const float iz = 1.0f / z, iz2 = iz * iz;
    float dpx = gu * fx * iz;
    float dpy = gv * fy * iz;
    float dpz = -(gu * fx * G.x + gv * fy * G.y) * iz2;
    dpz = dpz - (dJ00 * fx + dJ11 * fy) * iz2;
    if (!G.clx) {
        dpx = dpx - dJ02 * fx * iz2;
        dpz = dpz + dJ02 * 2.0f * fx * G.x * iz2 * iz;
    } else {
        dpz = dpz + dJ02 * fx * (G.J02 * (-z / fx)) * iz2;   // fx * (xg/z) / z^2
    }
    if (!G.cly) {
        dpy = dpy - dJ12 * fy * iz2;
        dpz = dpz + dJ12 * 2.0f * fy * G.y * iz2 * iz;
    } else {
        dpz = dpz + dJ12 * fy * (G.J12 * (-z / fy)) * iz2;
    }
    float dmu[3];
#pragma unroll
    for (int j = 0; j < 3; j++) dmu[j] = R[j] * dpx + R[3 + j] * dpy + R[6 + j] * dpz;

    // Sigma = M M^T:  dM = 2 dSigma M,  ds_j = sum_i Rq_ij dM_ij,  dRq = dM diag(s)
    const float *M = G.M, *Q = G.Rq;
    float dM[9];
#pragma unroll
    for (int i = 0; i < 3; i++)
#pragma unroll
        for (int j = 0; j < 3; j++)
            dM[i * 3 + j] = 2.0f * (dS[i][0] * M[j] + dS[i][1] * M[3 + j] + dS[i][2] * M[6 + j]);
    float ds[3];
#pragma unroll
    for (int j = 0; j < 3; j++) ds[j] = Q[j] * dM[j] + Q[3 + j] * dM[3 + j] + Q[6 + j] * dM[6 + j];
    float dR[9];
#pragma unroll
    for (int i = 0; i < 3; i++)
#pragma unroll
        for (int j = 0; j < 3; j++) dR[i * 3 + j] = dM[i * 3 + j] * s[j];
    const float w = G.w, a = G.qa, b = G.qb, c = G.qc;
    float dq[4];
    dq[0] = 2.0f * (-c * dR[1] + b * dR[2] + c * dR[3] - a * dR[5] - b * dR[6] + a * dR[7]);
    dq[1] = 2.0f * (b * dR[1] + c * dR[2] + b * dR[3] - w * dR[5] + c * dR[6] + w * dR[7]) -
            4.0f * a * (dR[4] + dR[8]);
    dq[2] = 2.0f * (a * dR[1] + w * dR[2] + a * dR[3] + c * dR[5] - w * dR[6] + c * dR[7]) -
            4.0f * b * (dR[0] + dR[8]);
    dq[3] = 2.0f * (-w * dR[1] + a * dR[2] + w * dR[3] + b * dR[5] + a * dR[6] + b * dR[7]) -
            4.0f * c * (dR[0] + dR[4]);
    const float qdot = w * dq[0] + a * dq[1] + b * dq[2] + c * dq[3];
    const float qh[4] = {w, a, b, c};

    // colour: rgb_ch = max(0, 0.5 + sum_j k_j Y_j(d)); clamped channels get 0
    float ccx, ccy, ccz;
    cam_centre(cam, ccx, ccy, ccz);
    float dx = mx - ccx, dy = my - ccy, dz = mz - ccz;
    const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
    dx = dx / dn; dy = dy / dn; dz = dz / dn;
    float Y[16];
    sh_basis(K, dx, dy, dz, Y);
    float dY[16][3];
    sh_basis_grad(K, dx, dy, dz, dY);
    float dd[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ch = 0; ch < 3; ch++) {
        float kv[16];
        float sum = 0.0f;
        for (int j = 0; j < K; j++) {
            kv[j] = ld_sh(sh + ((size_t)(j * 3 + ch)) * n + g);
            sum = sum + kv[j] * Y[j];
        }
        if (0.5f + sum < 0.0f) continue;
        const float gr = grgb[ch];
        for (int j = 0; j < K; j++) {
            float *p = d_sh + ((size_t)(j * 3 + ch)) * n + g;
            *p = *p + Y[j] * gr;
            dd[0] = dd[0] + kv[j] * dY[j][0] * gr;
            dd[1] = dd[1] + kv[j] * dY[j][1] * gr;
            dd[2] = dd[2] + kv[j] * dY[j][2] * gr;
        }
    }
    const float ddot = dx * dd[0] + dy * dd[1] + dz * dd[2];
    dmu[0] = dmu[0] + (dd[0] - dx * ddot) / dn;
    dmu[1] = dmu[1] + (dd[1] - dy * ddot) / dn;
    dmu[2] = dmu[2] + (dd[2] - dz * ddot) / dn;

#pragma unroll
    for (int r = 0; r < 3; r++) d_means[r * n + g] += dmu[r];
#pragma unroll
    for (int r = 0; r < 3; r++) d_log_scales[r * n + g] += s[r] * ds[r];
#pragma unroll
    for (int r = 0; r < 4; r++) d_quats[r * n + g] += (dq[r] - qh[r] * qdot) / G.nq;
    d_logits[g] += o * (1.0f - o) * go;
}

}  // namespace

hipError_t launch_project(const gs_gaussians &g, const Cam &cam, Splat *splats, hipStream_t s)
{
    const int n = (int)g.n;
    if (n == 0) return hipSuccess;
    const int K = (g.sh_degree + 1) * (g.sh_degree + 1);
    dim3 grid((n + kBlock - 1) / kBlock);
    if (g.sh_dtype == GS_SH_F16)
        project_kernel<__half><<<grid, kBlock, 0, s>>>(n, K, g.means, g.scales, g.quats, g.opacities,
                                                       (const __half *)g.sh, g.active, cam, splats);
    else
        project_kernel<float><<<grid, kBlock, 0, s>>>(n, K, g.means, g.scales, g.quats, g.opacities,
                                                      (const float *)g.sh, g.active, cam, splats);
    return hipGetLastError();
}

hipError_t launch_project_bwd(const gs_gaussians &g, const Cam &cam, const Splat *splats,
                              const float *grad2d, const gs_grads &out, hipStream_t s)
{
    const int n = (int)g.n;
    if (n == 0) return hipSuccess;
    const int K = (g.sh_degree + 1) * (g.sh_degree + 1);
    dim3 grid((n + kBlock - 1) / kBlock);
    if (g.sh_dtype == GS_SH_F16)
        project_bwd_kernel<__half><<<grid, kBlock, 0, s>>>(
            n, K, g.means, g.scales, g.quats, g.opacities, (const __half *)g.sh, cam, splats, grad2d,
            out.means, out.log_scales, out.quats, out.opacity_logits, out.sh);
    else
        project_bwd_kernel<float><<<grid, kBlock, 0, s>>>(
            n, K, g.means, g.scales, g.quats, g.opacities, (const float *)g.sh, cam, splats, grad2d,
            out.means, out.log_scales, out.quats, out.opacity_logits, out.sh);
    return hipGetLastError();
}

}  // namespace gsi
