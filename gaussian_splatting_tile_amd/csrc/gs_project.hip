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

template <typename R>
struct GeoT {
    R x, y, z, tx, ty;
    R w, qa, qb, qc, nq;             // normalised quaternion and |q|
    R Rq[9];
    R M[9];
    R S[6];                          // Sigma: 00 01 02 11 12 22
    R J00, J02, J11, J12;
    bool clx, cly;
    R T[6];                          // T = J R, rows 0 and 1
    R p00, p01, p11, det;
    R u, v;
};
using Geo = GeoT<float>;

__device__ __forceinline__ float rmin(float a, float b) { return fminf(a, b); }
__device__ __forceinline__ float rmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ double rmin(double a, double b) { return fmin(a, b); }
__device__ __forceinline__ double rmax(double a, double b) { return fmax(a, b); }

// The view-independent part: normalised quaternion, its rotation Rq and
// M = Rq diag(s); false for a zero quaternion.
template <typename R>
__device__ __forceinline__ bool rot_scale(R sx, R sy, R sz, R qw, R qx, R qy, R qz, GeoT<R> &o)
{
    R nq2 = qw * qw;  nq2 = nq2 + qx * qx;  nq2 = nq2 + qy * qy;  nq2 = nq2 + qz * qz;
    if (!(nq2 > (R)0)) return false;
    const R nq = sqrt(nq2);
    const R w = qw / nq, a = qx / nq, b = qy / nq, c = qz / nq;
    o.w = w; o.qa = a; o.qb = b; o.qc = c; o.nq = nq;
    const R one = (R)1, two = (R)2;
    R *Q = o.Rq;
    Q[0] = one - two * (b * b + c * c);
    Q[1] = two * (a * b - w * c);
    Q[2] = two * (a * c + w * b);
    Q[3] = two * (a * b + w * c);
    Q[4] = one - two * (a * a + c * c);
    Q[5] = two * (b * c - w * a);
    Q[6] = two * (a * c - w * b);
    Q[7] = two * (b * c + w * a);
    Q[8] = one - two * (a * a + b * b);
    R *M = o.M;
    M[0] = Q[0] * sx; M[1] = Q[1] * sy; M[2] = Q[2] * sz;
    M[3] = Q[3] * sx; M[4] = Q[4] * sy; M[5] = Q[5] * sz;
    M[6] = Q[6] * sx; M[7] = Q[7] * sy; M[8] = Q[8] * sz;
    return true;
}

// Geometry of one Gaussian in scalar type R (float: the op-order contract of
// the forward; double: the backward's recomputation); returns false when it
// is culled before the rect.
template <typename R>
__device__ __forceinline__ bool geometry(const Cam &cam, R mx, R my, R mz, R sx, R sy, R sz, R qw,
                                         R qx, R qy, R qz, GeoT<R> &o)
{
    R Rc[9], t[3];
    for (int i = 0; i < 9; i++) Rc[i] = (R)cam.R[i];
    for (int i = 0; i < 3; i++) t[i] = (R)cam.t[i];
    const R fx = (R)cam.fx, fy = (R)cam.fy;
    R x = Rc[0] * mx;  x = x + Rc[1] * my;  x = x + Rc[2] * mz;  x = x + t[0];
    R y = Rc[3] * mx;  y = y + Rc[4] * my;  y = y + Rc[5] * mz;  y = y + t[1];
    R z = Rc[6] * mx;  z = z + Rc[7] * my;  z = z + Rc[8] * mz;  z = z + t[2];
    if (!(z > (R)cam.znear)) return false;
    o.x = x; o.y = y; o.z = z;

    o.tx = x / z;
    o.ty = y / z;
    o.u = fx * o.tx + (R)cam.cx;
    o.v = fy * o.ty + (R)cam.cy;

    if (!rot_scale(sx, sy, sz, qw, qx, qy, qz, o)) return false;
    const R *M = o.M;
    R *S = o.S;
    S[0] = (M[0] * M[0] + M[1] * M[1]) + M[2] * M[2];
    S[1] = (M[0] * M[3] + M[1] * M[4]) + M[2] * M[5];
    S[2] = (M[0] * M[6] + M[1] * M[7]) + M[2] * M[8];
    S[3] = (M[3] * M[3] + M[4] * M[4]) + M[5] * M[5];
    S[4] = (M[3] * M[6] + M[4] * M[7]) + M[5] * M[8];
    S[5] = (M[6] * M[6] + M[7] * M[7]) + M[8] * M[8];

    const R lx = (R)cam.guard * (((R)0.5 * (R)cam.width) / fx);
    const R ly = (R)cam.guard * (((R)0.5 * (R)cam.height) / fy);
    o.clx = (o.tx < -lx) || (o.tx > lx);
    o.cly = (o.ty < -ly) || (o.ty > ly);
    const R xg = rmin(rmax(o.tx, -lx), lx) * z;
    const R yg = rmin(rmax(o.ty, -ly), ly) * z;
    const R zz = z * z;
    o.J00 = fx / z;
    o.J02 = -((fx * xg) / zz);
    o.J11 = fy / z;
    o.J12 = -((fy * yg) / zz);

    R *T = o.T;
    T[0] = o.J00 * Rc[0] + o.J02 * Rc[6];
    T[1] = o.J00 * Rc[1] + o.J02 * Rc[7];
    T[2] = o.J00 * Rc[2] + o.J02 * Rc[8];
    T[3] = o.J11 * Rc[3] + o.J12 * Rc[6];
    T[4] = o.J11 * Rc[4] + o.J12 * Rc[7];
    T[5] = o.J11 * Rc[5] + o.J12 * Rc[8];
    // U = T Sigma (Sigma symmetric: S01 = S10 ...)
    const R U00 = (T[0] * S[0] + T[1] * S[1]) + T[2] * S[2];
    const R U01 = (T[0] * S[1] + T[1] * S[3]) + T[2] * S[4];
    const R U02 = (T[0] * S[2] + T[1] * S[4]) + T[2] * S[5];
    const R U10 = (T[3] * S[0] + T[4] * S[1]) + T[5] * S[2];
    const R U11 = (T[3] * S[1] + T[4] * S[3]) + T[5] * S[4];
    const R U12 = (T[3] * S[2] + T[4] * S[4]) + T[5] * S[5];
    const R C00 = (U00 * T[0] + U01 * T[1]) + U02 * T[2];
    const R C01 = (U00 * T[3] + U01 * T[4]) + U02 * T[5];
    const R C11 = (U10 * T[3] + U11 * T[4]) + U12 * T[5];
    o.p00 = C00 + (R)0.3;
    o.p01 = C01;
    o.p11 = C11 + (R)0.3;
    o.det = o.p00 * o.p11 - o.p01 * o.p01;
    return o.det > (R)0;
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

// Basis values Y[0 .. (DEG+1)^2) at the unit direction (x, y, z).
template <int DEG>
__device__ __forceinline__ void sh_basis(float x, float y, float z, float *Y)
{
    Y[0] = SH::c0;
    if (DEG >= 1) {
        Y[1] = -SH::c1 * y;
        Y[2] = SH::c1 * z;
        Y[3] = -SH::c1 * x;
    }
    if (DEG >= 2) {
        const float xx = x * x, yy = y * y, zz = z * z;
        Y[4] = SH::c2a * (x * y);
        Y[5] = -SH::c2a * (y * z);
        Y[6] = SH::c2b * (2.0f * zz - xx - yy);
        Y[7] = -SH::c2a * (x * z);
        Y[8] = SH::c2c * (xx - yy);
        if (DEG >= 3) {
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

// sum_j w_j grad Y_j at (x, y, z): the gradient of the basis with respect to
// the three components of the direction, folded with the weights w_j.
template <int DEG>
__device__ __forceinline__ void sh_dir_grad(const float *w, float x, float y, float z, float dd[3])
{
    float gx = 0.0f, gy = 0.0f, gz = 0.0f;
    if (DEG >= 1) {
        gy += -SH::c1 * w[1];
        gz += SH::c1 * w[2];
        gx += -SH::c1 * w[3];
    }
    if (DEG >= 2) {
        gx += SH::c2a * y * w[4];                gy += SH::c2a * x * w[4];
        gy += -SH::c2a * z * w[5];               gz += -SH::c2a * y * w[5];
        gx += -2.0f * SH::c2b * x * w[6];        gy += -2.0f * SH::c2b * y * w[6];
        gz += 4.0f * SH::c2b * z * w[6];
        gx += -SH::c2a * z * w[7];               gz += -SH::c2a * x * w[7];
        gx += 2.0f * SH::c2c * x * w[8];         gy += -2.0f * SH::c2c * y * w[8];
        if (DEG >= 3) {
            const float xx = x * x, yy = y * y, zz = z * z;
            gx += -6.0f * SH::c3a * x * y * w[9];
            gy += -3.0f * SH::c3a * (xx - yy) * w[9];
            gx += SH::c3b * y * z * w[10];  gy += SH::c3b * x * z * w[10];  gz += SH::c3b * x * y * w[10];
            gx += 2.0f * SH::c3c * x * y * w[11];
            gy += -SH::c3c * (4.0f * zz - xx - 3.0f * yy) * w[11];
            gz += -8.0f * SH::c3c * y * z * w[11];
            gx += -6.0f * SH::c3d * x * z * w[12];
            gy += -6.0f * SH::c3d * y * z * w[12];
            gz += SH::c3d * (6.0f * zz - 3.0f * xx - 3.0f * yy) * w[12];
            gx += -SH::c3c * (4.0f * zz - 3.0f * xx - yy) * w[13];
            gy += 2.0f * SH::c3c * x * y * w[13];
            gz += -8.0f * SH::c3c * x * z * w[13];
            gx += 2.0f * SH::c3e * x * z * w[14];
            gy += -2.0f * SH::c3e * y * z * w[14];
            gz += SH::c3e * (xx - yy) * w[14];
            gx += -3.0f * SH::c3a * (xx - yy) * w[15];
            gy += 6.0f * SH::c3a * x * y * w[15];
        }
    }
    dd[0] = gx; dd[1] = gy; dd[2] = gz;
}

// SH coefficient `row` of Gaussian g; blk = g / 256 (the projection passes
// its workgroup index, which is that block for every lane, so the 8-bit
// bounds are read with scalar loads)
template <typename T>
__device__ __forceinline__ float ld_sh(const T *sh, const float *bounds, size_t row, int n, int g, int blk);
template <>
__device__ __forceinline__ float ld_sh<float>(const float *sh, const float *, size_t row, int n, int g, int)
{
    return sh[row * n + g];
}
template <>
__device__ __forceinline__ float ld_sh<__half>(const __half *sh, const float *, size_t row, int n, int g, int)
{
    return __half2float(sh[row * n + g]);
}
// 8-bit codes: lo + q step, step = (hi - lo) * fp32(1/255), with the
// (lo, hi) of the row's 256-Gaussian block, each step one fp32 operation
template <>
__device__ __forceinline__ float ld_sh<uint8_t>(const uint8_t *sh, const float *bounds, size_t row, int n, int g,
                                                int blk)
{
#pragma clang fp contract(off)
    const size_t nb = ((size_t)n + 255) / 256;
    const float *b = bounds + (row * nb + (size_t)blk) * 2;
    const float lo = b[0], hi = b[1];
    const float step = (hi - lo) * (1.0f / 255.0f);
    return lo + (float)sh[row * n + g] * step;
}

// Camera centre c = -R^T t, sums left to right.
__device__ __forceinline__ void cam_centre(const Cam &cam, float &ccx, float &ccy, float &ccz)
{
    const float *R = cam.R;
    ccx = R[0] * cam.t[0];  ccx = ccx + R[3] * cam.t[1];  ccx = ccx + R[6] * cam.t[2];  ccx = -ccx;
    ccy = R[1] * cam.t[0];  ccy = ccy + R[4] * cam.t[1];  ccy = ccy + R[7] * cam.t[2];  ccy = -ccy;
    ccz = R[2] * cam.t[0];  ccz = ccz + R[5] * cam.t[1];  ccz = ccz + R[8] * cam.t[2];  ccz = -ccz;
}

// Unit view direction from the camera centre and its length.
__device__ __forceinline__ void view_dir(const Cam &cam, float mx, float my, float mz, float &dx,
                                         float &dy, float &dz, float &dn)
{
    float ccx, ccy, ccz;
    cam_centre(cam, ccx, ccy, ccz);
    dx = mx - ccx; dy = my - ccy; dz = mz - ccz;
    dn = sqrtf(dx * dx + dy * dy + dz * dz);
    dx = dx / dn; dy = dy / dn; dz = dz / dn;
}

// Moving Gaussians (a motion vector v and a time offset t_g each): in a view
// at time tau the mean is mu + (tau - t_g) v, one fp32 rounding per
// operation in that order (contraction is off in this file).  The backward
// adds dL/dv = sum_views dt dL/dmu' and dL/dt_g = -v . sum_views dL/dmu'.
struct Motion {
    const float *v;               // [3][n]
    const float *t;               // [n]
    float *dv;                    // [3][n] (backward)
    float *dt;                    // [n]    (backward)
};

__device__ __forceinline__ float displace(float mu, float dt, float v) { return mu + dt * v; }

template <int DEG, typename TSH, bool kMotion>
__global__ __launch_bounds__(kBlock) void project_kernel(
    int n, const float *__restrict__ means, const float *__restrict__ scales,
    const float *__restrict__ quats, const float *__restrict__ opac, const TSH *__restrict__ sh,
    const float *__restrict__ sh_bounds, const uint8_t *__restrict__ active, const Motion mo,
    const ProjBatch views)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= n) return;
    const float mx = means[g], my = means[n + g], mz = means[2 * n + g];
    const float sx = scales[g], sy = scales[n + g], sz = scales[2 * n + g];
    const float qw = quats[g], qx = quats[n + g], qy = quats[2 * n + g], qz = quats[3 * n + g];
    const float o = opac[g];
    float vx = 0.0f, vy = 0.0f, vz = 0.0f, tg = 0.0f;
    if constexpr (kMotion) {
        vx = mo.v[g];
        vy = mo.v[n + g];
        vz = mo.v[2 * n + g];
        tg = mo.t[g];
    }
    // with motion the mean's finiteness is that of each view's displaced mean
    const bool act = active == nullptr || active[g] != 0;
    const bool on = act && all_finite(kMotion ? 0.0f : mx, kMotion ? 0.0f : my, kMotion ? 0.0f : mz, sx, sy, sz,
                                      qw, qx, qy, qz, o);

    // the views of the batch, parameters and SH coefficients read once (all
    // lanes load, g < n; a masked-out Gaussian's coefficients go unused, and
    // with a random mask nearly every line of a row holds a kept Gaussian)
    float shc[3 * K];
    static_assert(kBlock == 256, "a projection workgroup is one 256-Gaussian SH block");
#pragma unroll
    for (int i = 0; i < 3 * K; i++) shc[i] = ld_sh(sh, sh_bounds, (size_t)i, n, g, (int)blockIdx.x);
    for (int v = 0; v < views.count; v++) {
    const Cam &cam = views.cam[v];
    Splat *__restrict__ out = views.out[v];
    Splat rec;
    rec.a = rec.b = rec.c = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool vis = on;
    float px = mx, py = my, pz = mz;
    if constexpr (kMotion) {
        const float dt = cam.time - tg;
        px = displace(mx, dt, vx);
        py = displace(my, dt, vy);
        pz = displace(mz, dt, vz);
        vis = vis && isfinite(px) && isfinite(py) && isfinite(pz);
    }
    uint32_t dkey = kSentinel;
    uint2 grect = make_uint2(0u, 0u);
    Geo G;
    if (vis) vis = geometry(cam, px, py, pz, sx, sy, sz, qw, qx, qy, qz, G);
    if (vis && cam.lod > 0.0f) {
        // distance-LOD gate: undilated 3-sigma pinhole radius below lod px
        float ccx, ccy, ccz;
        cam_centre(cam, ccx, ccy, ccz);
        const float dx = px - ccx, dy = py - ccy, dz = pz - ccz;
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
            // colour: SH at the unit view direction (read only for survivors)
            float dx, dy, dz, dn;
            view_dir(cam, px, py, pz, dx, dy, dz, dn);
            float Y[K];
            sh_basis<DEG>(dx, dy, dz, Y);
            float col[3];
#pragma unroll
            for (int ch = 0; ch < 3; ch++) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < K; j++) s = s + shc[j * 3 + ch] * Y[j];
                const float val = 0.5f + s;
                col[ch] = val < 0.0f ? 0.0f : val;
            }
            rec.a = make_float4(G.u, G.v, G.z, __int_as_float((int)rf));
            rec.b = make_float4(ca, cb, cc, o);
            rec.c = make_float4(col[0], col[1], col[2],
                                __uint_as_float((uint32_t)((r.x1 - r.x0) * (r.y1 - r.y0))));
            dkey = __float_as_uint(G.z);
            grect = pack_rect(r);
        }
    }
    // With the sort's keys requested, the record of a Gaussian outside the
    // importance mask is not written: the sort takes visibility from the
    // depth key, the blend reads listed Gaussians only and the projection
    // backward skips Gaussians outside the mask.
    if (act || views.dkeys[v] == nullptr) out[g] = rec;
    // the sort's inputs from the same values (the binning would otherwise
    // read them back from the record)
    if (views.dkeys[v] != nullptr) {
        views.dkeys[v][g] = dkey;
        if (views.grect[v] != nullptr) views.grect[v][g] = grect;
    }
    }   // views
}

// ---------------------------------------------------------------------------
// Backward: the screen-space gradients d/du, d/dv, d/dSigma' (xx, xy, yy,
// per element of the symmetric matrix), d/dopacity, d/drgb (summed from the
// compositing pass's per-tile partials) -> raw parameter gradients, +=.  The
// forward sequence above is recomputed; the guard clamp and the colour clamp
// keep the branch the forward took.  The compositing pass already carried
// the conic's gradient through the record's conic per pixel; the fp64
// inverse replaces it below.
//   Sigma' = Sigma2 + 0.3 I: dSigma2 = dSigma'
//   Sigma2 = T Sigma T^T:   dSigma = T^T dSigma2 T,  dT = 2 dSigma2 T Sigma
//   T = J W:                dJ = dT W^T;  J and (u, v) differentiated in (x, y, z)
//   Sigma = M M^T:          dM = 2 dSigma M;  ds_j = sum_i Rq_ij dM_ij;  dRq = dM diag(s)
//   q_hat = q / |q|:        dq = (I - q_hat q_hat^T) dq_hat / |q|
//   colour:                 dk_j = Y_j drgb (unclamped channels),
//                           dmu += (I - d d^T) / |mu - c| sum_j k_j grad Y_j drgb
//   raw outputs:            dlog s = s ds,  dlogit = o (1 - o) do.
// The screen-space gradients of each Gaussian visible in a view: the sum of
// its per-tile partial rows, which sit at its tiles_touched contiguous
// duplication slots.  Gaussians are taken in depth order, 63 per wave (the
// slots of consecutive depth ranks are consecutive, so a wave reads one
// contiguous stretch of rows and needs no record), in nine rounds of seven.
// A Gaussian with at most kSumSmall slots is summed by nine lanes, one
// component each, in slot order; the few larger ones (near the camera they
// span thousands of tiles) by the whole wave in turn: lane (j, q) takes slots
// j, j + 7, ... of component q, then the seven partial sums are added in j
// order.  Both orders are fixed, so the result is reproducible.  The rows of
// round r + 1 (their first four slots) are loaded while round r is summed.
// (Loading a group of 21 Gaussians' contiguous rows into LDS with 16-byte
// loads first, then summing from LDS in the same order, measured 5 % slower:
// the scattered 36-byte reads are not what limits this kernel.)
// Slots at or past the capacity were never written and are left out.
// Output: g2[g][9], visible Gaussians only, components 2..4 halved (the
// rows hold the second moments sum dp w' w'^T).
constexpr int kSumPerRound = 7;
constexpr int kSumRounds = 9;
constexpr int kSumPerWave = kSumPerRound * kSumRounds;   // 63
constexpr uint32_t kSumSmall = 32;     // slots a lane sums on its own
constexpr int kSumAhead = 4;           // slots per lane loaded one round ahead (a
                                       // Gaussian has ~4 at 1080p; 8 was 1-2 % slower)

struct SumRound {
    uint32_t g, first, count;
    bool valid;
    float v[kSumAhead];
};

__global__ __launch_bounds__(kBlock) void sum_partials_kernel(const SumBatch batch)
{
    const SumView &V = batch.v[blockIdx.y];
    const float *__restrict__ partial = V.partial;
    const uint64_t k_capacity = V.k_capacity;
    float *__restrict__ g2 = V.g2;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * (unsigned)kBlock + threadIdx.x) >> 6;
    const uint32_t n_vis = *V.count;
    const uint32_t j0 = wave * kSumPerWave;
    if (j0 >= n_vis) return;
    // lane L < 63 holds depth rank j0 + L: its Gaussian, first slot, slot count
    uint32_t my_g = 0, my_first = 0, my_count = 0;
    if (lane < kSumPerWave && j0 + lane < n_vis) {
        const uint32_t j = j0 + lane;
        my_g = V.order[j];
        const uint64_t s0 = V.off[j], s1 = V.off[j + 1];
        const uint64_t a = s0 < k_capacity ? s0 : k_capacity, b = s1 < k_capacity ? s1 : k_capacity;
        my_first = (uint32_t)a;
        my_count = (uint32_t)(b - a);
    }
    const int gl = lane / 9, q = lane - 9 * gl;
    // round r: lane (gl, q) takes rank j0 + 7 r + gl; its first eight slots
    // are loaded unpredicated (indices past the last slot re-read it)
    auto fetch = [&](int r, SumRound &R) {
        const int src = r * kSumPerRound + (gl < kSumPerRound ? gl : 0);
        R.g = (uint32_t)__shfl((int)my_g, src, 64);
        R.first = (uint32_t)__shfl((int)my_first, src, 64);
        R.count = (uint32_t)__shfl((int)my_count, src, 64);
        R.valid = gl < kSumPerRound && j0 + (uint32_t)src < n_vis;
        if (R.valid && R.count > 0 && R.count <= kSumSmall) {
            const uint32_t last = R.first + R.count - 1;
#pragma unroll
            for (int t = 0; t < kSumAhead; t++) R.v[t] = partial[(size_t)min(R.first + t, last) * 9 + q];
        }
    };
    const int cj = lane / 9, cq = lane - 9 * (lane / 9);       // cooperative layout (63 lanes)
    SumRound cur, nxt;
    fetch(0, cur);
    for (int r = 0; r < kSumRounds; r++) {
        if (j0 + (uint32_t)(r * kSumPerRound) >= n_vis) break;   // wave-uniform
        if (r + 1 < kSumRounds) fetch(r + 1, nxt);
        // fp64: the sums run over up to thousands of partials
        double acc = 0.0;
        const bool big = cur.count > kSumSmall;
        if (cur.valid && !big && cur.count > 0) {
#pragma unroll
            for (int t = 0; t < kSumAhead; t++) acc += (uint32_t)t < cur.count ? (double)cur.v[t] : 0.0;
            const uint32_t last = cur.first + cur.count;
            for (uint32_t sl = cur.first + kSumAhead; sl < last; sl += 8) {
                float v[8];
#pragma unroll
                for (int t = 0; t < 8; t++) v[t] = partial[(size_t)min(sl + t, last - 1) * 9 + q];
#pragma unroll
                for (int t = 0; t < 8; t++) acc += sl + t < last ? (double)v[t] : 0.0;
            }
        }
        // the round's large Gaussians, one after another
        uint64_t bigs = __ballot(cur.valid && big && q == 0);
        while (bigs) {
            const int src = __builtin_ctzll(bigs);                 // lane (gl_b, 0) of that Gaussian
            bigs &= bigs - 1;
            const uint32_t bfirst = (uint32_t)__shfl((int)cur.first, src, 64);
            const uint32_t bcount = (uint32_t)__shfl((int)cur.count, src, 64);
            double part = 0.0;
            if (cj < kSumPerRound) {
                // four rows in flight per step; the sum stays in slot order
                uint32_t t = cj;
                for (; t + 3 * kSumPerRound < bcount; t += 4 * kSumPerRound) {
                    const float *row = partial + ((size_t)bfirst + t) * 9 + cq;
                    const float r0 = row[0], r1 = row[9 * kSumPerRound], r2 = row[18 * kSumPerRound],
                                r3 = row[27 * kSumPerRound];
                    part += (double)r0;
                    part += (double)r1;
                    part += (double)r2;
                    part += (double)r3;
                }
                for (; t < bcount; t += kSumPerRound) part += (double)partial[((size_t)bfirst + t) * 9 + cq];
            }
            // lane (gl_b, q) collects component q: sum over j = 0..6 in order
            double tot = 0.0;
            for (int t = 0; t < kSumPerRound; t++) tot += __shfl(part, t * 9 + q, 64);
            if (gl == src / 9) acc = tot;
        }
        // the rows carry sum dp w' w'^T; d/dSigma' takes half of it (exact)
        if (cur.valid) g2[(size_t)cur.g * 9 + q] = (float)(q >= 2 && q <= 4 ? 0.5 * acc : acc);
        cur = nxt;
    }
}

// The projection backward runs as two kernels over a batch of views, one
// thread per Gaussian each: the colour part (SH gradients and the view
// direction's share of the mean gradient, fp32 like the forward's colour)
// and the geometry part (the fp64 chain rule).  Each reads the Gaussian's
// parameters once for the whole batch and sums its gradients in registers
// in view order; the SH gradients are updated in place per view (the lines
// stay in cache between views).
// Colour part: one lane per (Gaussian, channel), 21 Gaussians per wave with
// the channel fastest.  A lane holds its channel's K coefficients and their
// gradient sums in registers for the whole batch, so the SH rows are read
// once and their gradients updated once.  Per view, for an unclamped channel:
//   dk_j += Y_j(d) dL/drgb,   d(direction) += dL/drgb grad_d sum_j k_j Y_j(d);
// the three channels' shares of the mean gradient are added across lanes.
constexpr int kColourPerWave = 21;
// Gaussians of a wave's range that the projection backward must visit: in
// the importance mask (if any) and visible in at least one view of the batch.
// With a mask most are not, and a wave of mostly idle lanes costs as much as
// a full one, so each wave first compacts its range (64 per ballot) into a
// per-wave list in LDS and then works through the list densely.
constexpr int kMaxCompact = 1024;             // Gaussians per wave range, at most

// Was Gaussian g visible in view v?  From the view's depth keys when the
// projection wrote them (4 bytes per Gaussian, not a sentinel), else from
// the record's radius (non-zero): the projection sets both together, so the
// two agree.  The keys spare the colour part a read of every record line.
__device__ __forceinline__ bool seen(const ViewBatch &views, int v, long long g)
{
    const uint32_t *k = views.dkeys[v];
    return k != nullptr ? k[g] != kSentinel : __float_as_int(views.splats[v][g].a.w) != 0;
}
__device__ __forceinline__ int compact_range(long long g_begin, long long g_end, const uint8_t *__restrict__ active,
                                             const ViewBatch &views, uint32_t *list)
{
    const int lane = threadIdx.x & 63;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int cnt = 0;
    for (long long base = g_begin; base < g_end; base += 64) {
        const long long g = base + lane;
        bool keep = g < g_end && (active == nullptr || active[g] != 0);
        if (keep) {
            bool any = false;
            for (int v = 0; v < views.count; v++) any = any | seen(views, v, g);
            keep = any;
        }
        const uint64_t m = __ballot(keep);
        if (keep) list[cnt + __popcll(m & lt)] = (uint32_t)g;
        cnt += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return cnt;
}

// One round of the colour part: lane (gl, ch) takes Gaussian g (valid lanes
// only; every lane of the wave calls this, for the cross-lane sums).
template <int DEG, typename TSH, bool kMotion>
__device__ __forceinline__ void colour_backward(int n_, int g, bool valid, int ch, const float *__restrict__ means,
                                                const TSH *__restrict__ sh, const float *__restrict__ sh_bounds,
                                                const Motion &mo, const ViewBatch &views,
                                                float *__restrict__ d_means, float *__restrict__ d_sh)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int lane = threadIdx.x & 63;
    // opaque copies of the row pointers and the row stride: the 2 K row
    // offsets are invariant across the caller's rounds and would otherwise
    // be held in registers
    const TSH *shr = sh;
    float *dshr = d_sh;
    int n = n_;
    asm volatile("" : "+s"(shr), "+s"(dshr), "+s"(n));
    float kv[K], acc[K];
    float mx = 0.0f, my = 0.0f, mz = 0.0f;
#pragma unroll
    for (int j = 0; j < K; j++) {
        kv[j] = valid ? ld_sh(shr, sh_bounds, (size_t)(j * 3 + ch), n, g, g >> 8) : 0.0f;
        acc[j] = 0.0f;
    }
    float vx = 0.0f, vy = 0.0f, vz = 0.0f, tg = 0.0f;
    if (valid) {
        mx = means[g];
        my = means[n + g];
        mz = means[2 * n + g];
        if constexpr (kMotion) {
            vx = mo.v[g];
            vy = mo.v[n + g];
            vz = mo.v[2 * n + g];
            tg = mo.t[g];
        }
    }
    float dm[3] = {0.0f, 0.0f, 0.0f};
    float dmv[3] = {0.0f, 0.0f, 0.0f};          // sum over views of dt dL/dmu'

    bool visible = false;
    // the next view's visibility and gradient are loaded one view ahead (a
    // culled Gaussian's gradient row holds no value and is not used)
    bool seen_next = false;
    float gr_next = 0.0f;
    if (valid && views.count > 0) {
        seen_next = seen(views, 0, g);
        gr_next = views.g2[0][(size_t)g * 9 + 6 + ch];
    }
    for (int v = 0; v < views.count; v++) {
        const bool in_view = seen_next;
        const float gr = gr_next;
        if (valid && v + 1 < views.count) {
            seen_next = seen(views, v + 1, g);
            gr_next = views.g2[v + 1][(size_t)g * 9 + 6 + ch];
        }
        // culled Gaussians receive nothing
        if (!valid || !in_view) continue;
        visible = true;
        const Cam &cam = views.cam[v];
        float px = mx, py = my, pz = mz, dtv = 0.0f;
        if constexpr (kMotion) {
            dtv = cam.time - tg;
            px = displace(mx, dtv, vx);
            py = displace(my, dtv, vy);
            pz = displace(mz, dtv, vz);
        }
        float dx, dy, dz, dn;
        view_dir(cam, px, py, pz, dx, dy, dz, dn);
        float Y[K];
        sh_basis<DEG>(dx, dy, dz, Y);
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < K; j++) sum = sum + kv[j] * Y[j];
        // the forward's clamp at 0 keeps its branch
        if (0.5f + sum < 0.0f) continue;
#pragma unroll
        for (int j = 0; j < K; j++) acc[j] = acc[j] + Y[j] * gr;
        float dd[3];
        sh_dir_grad<DEG>(kv, dx, dy, dz, dd);
        dd[0] *= gr;
        dd[1] *= gr;
        dd[2] *= gr;
        const float ddot = dx * dd[0] + dy * dd[1] + dz * dd[2];
        const float c0 = (dd[0] - dx * ddot) / dn;
        const float c1 = (dd[1] - dy * ddot) / dn;
        const float c2 = (dd[2] - dz * ddot) / dn;
        dm[0] += c0;
        dm[1] += c1;
        dm[2] += c2;
        if constexpr (kMotion) {
            dmv[0] += dtv * c0;
            dmv[1] += dtv * c1;
            dmv[2] += dtv * c2;
        }
    }
    // channel lanes 3 gl + 1 and 3 gl + 2 hand their mean shares to 3 gl
    float tot[3], totv[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 3; j++) {
        const float a1 = __shfl(dm[j], lane + 1, 64), a2 = __shfl(dm[j], lane + 2, 64);
        tot[j] = (dm[j] + a1) + a2;
        if constexpr (kMotion) {
            const float b1 = __shfl(dmv[j], lane + 1, 64), b2 = __shfl(dmv[j], lane + 2, 64);
            totv[j] = (dmv[j] + b1) + b2;
        }
    }
    if (!visible) return;
#pragma unroll
    for (int j = 0; j < K; j++) {
        float *p = dshr + (size_t)(j * 3 + ch) * n + g;
        *p = *p + acc[j];
    }
    if (ch == 0) {
#pragma unroll
        for (int j = 0; j < 3; j++) d_means[j * n + g] += tot[j];
        if constexpr (kMotion) {
#pragma unroll
            for (int j = 0; j < 3; j++) mo.dv[j * n + g] += totv[j];
            mo.dt[g] -= (vx * tot[0] + vy * tot[1]) + vz * tot[2];
        }
    }
}

// Without a mask (COMPACT false) wave w takes Gaussians 21 w .. 21 w + 20 and
// Gaussians culled in every view drop out lane by lane; with one, each wave
// compacts its range of per_wave Gaussians first and takes rounds of 21.
template <int DEG, typename TSH, bool COMPACT, bool kMotion>
__global__ __launch_bounds__(kBlock) void project_bwd_color_kernel(int n, int per_wave,
                                                                   const float *__restrict__ means,
                                                                   const TSH *__restrict__ sh,
                                                                   const float *__restrict__ sh_bounds,
                                                                   const uint8_t *__restrict__ active,
                                                                   const Motion mo, const ViewBatch views,
                                                                   float *__restrict__ d_means,
                                                                   float *__restrict__ d_sh)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gl = lane / 3, ch = lane - 3 * gl;
    if constexpr (COMPACT) {
        __shared__ uint32_t s_list[kBlock / 64][kMaxCompact];
        const long long g_begin = ((long long)blockIdx.x * (kBlock / 64) + wv) * per_wave;
        const long long g_end = g_begin + per_wave < n ? g_begin + per_wave : n;
        const int cnt = compact_range(g_begin, g_end, active, views, s_list[wv]);
        for (int r0 = 0; r0 < cnt; r0 += kColourPerWave) {
            const int idx = r0 + gl;
            const bool valid = gl < kColourPerWave && idx < cnt;
            const int g = valid ? (int)s_list[wv][idx] : 0;
            colour_backward<DEG, TSH, kMotion>(n, g, valid, ch, means, sh, sh_bounds, mo, views, d_means, d_sh);
        }
    } else {
        const long long wave = (long long)blockIdx.x * (kBlock / 64) + wv;
        const long long gg = wave * kColourPerWave + gl;
        bool valid = gl < kColourPerWave && gg < n && (active == nullptr || active[gg] != 0);
        // culled in every view of the batch: leave the SH rows untouched
        if (valid) {
            bool any = false;
            for (int v = 0; v < views.count; v++) any = any | seen(views, v, gg);
            valid = any;
        }
        colour_backward<DEG, TSH, kMotion>(n, valid ? (int)gg : 0, valid, ch, means, sh, sh_bounds, mo, views,
                                           d_means, d_sh);
    }
}

// The geometry part for one Gaussian (visible in at least one view).
template <bool kMotion>
__device__ __forceinline__ void geom_backward(
    int n, int g, const float *__restrict__ means, const float *__restrict__ scales, const float *__restrict__ quats,
    const float *__restrict__ opac, const Motion &mo, const ViewBatch &views, float *__restrict__ d_means,
    float *__restrict__ d_log_scales, float *__restrict__ d_quats, float *__restrict__ d_logits)
{
    const float mx0 = means[g], my0 = means[n + g], mz0 = means[2 * n + g];
    float vx = 0.0f, vy = 0.0f, vz = 0.0f, tg = 0.0f;
    if constexpr (kMotion) {
        vx = mo.v[g];
        vy = mo.v[n + g];
        vz = mo.v[2 * n + g];
        tg = mo.t[g];
    }
    float acc_vel[3] = {0.0f, 0.0f, 0.0f};
    const float s0 = scales[g], s1 = scales[n + g], s2 = scales[2 * n + g];
    const float qw0 = quats[g], qx0 = quats[n + g], qy0 = quats[2 * n + g], qz0 = quats[3 * n + g];
    const float o = opac[g];
    float acc_mean[3] = {0.0f, 0.0f, 0.0f}, acc_ls[3], acc_q[4], acc_logit = 0.0f;
    double dS_sum[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    bool touched = false;
    // the next view's radius, conic and gradients are loaded one view ahead
    // (a culled Gaussian's gradient row holds no value and is not used)
    int rad_next = 0;
    float4 cr_next = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float g2_next[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (views.count > 0) {
        rad_next = __float_as_int(views.splats[0][g].a.w);
        cr_next = views.splats[0][g].b;
#pragma unroll
        for (int q = 0; q < 6; q++) g2_next[q] = views.g2[0][(size_t)g * 9 + q];
    }
    for (int v = 0; v < views.count; v++) {
    const int rad = rad_next;
    const float4 cr = cr_next;
    float g2[6];
#pragma unroll
    for (int q = 0; q < 6; q++) g2[q] = g2_next[q];
    if (v + 1 < views.count) {
        rad_next = __float_as_int(views.splats[v + 1][g].a.w);
        cr_next = views.splats[v + 1][g].b;
#pragma unroll
        for (int q = 0; q < 6; q++) g2_next[q] = views.g2[v + 1][(size_t)g * 9 + q];
    }
    if (rad == 0) continue;
    touched = true;
    // The view-independent part (rotation, 3D covariance) is recomputed per
    // view from opaque copies of the parameters: held across views in fp64
    // it would cost ~50 registers.  Its gradient chain runs once, after the
    // views, on the summed Sigma gradient.
    float mx = mx0, my = my0, mz = mz0, qw = qw0, qx = qx0, qy = qy0, qz = qz0;
    float s[3] = {s0, s1, s2};
    asm volatile("" : "+v"(mx), "+v"(my), "+v"(mz), "+v"(qw), "+v"(qx), "+v"(qy), "+v"(qz));
    asm volatile("" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]));
    const Cam &cam = views.cam[v];
    float dtv = 0.0f;
    if constexpr (kMotion) {
        dtv = cam.time - tg;
        mx = displace(mx, dtv, vx);
        my = displace(my, dtv, vy);
        mz = displace(mz, dtv, vz);
    }

    // The compositing pass worked in the principal frame V of the record's
    // conic Qr: mean gradient V (g0, g1), covariance gradient V W V^T.
    double ex, ey;
    {
        double l1, l2;
        conic_frame(cr.x, cr.y, cr.z, ex, ey, l1, l2);
    }
    const double gu = ex * (double)g2[0] - ey * (double)g2[1];
    const double gv = ey * (double)g2[0] + ex * (double)g2[1];
    const float go = g2[5];
    // The chain rule runs in fp64 on a fp64 recomputation of the geometry:
    // for thin Gaussians the conic is ill-conditioned (eigenvalue ratios up
    // to ~1e5), and fp32 intermediates would cost several digits.
    GeoT<double> G;
    geometry<double>(cam, mx, my, mz, s[0], s[1], s[2], qw, qx, qy, qz, G);
    double R[9];
#pragma unroll
    for (int i = 0; i < 9; i++) R[i] = cam.R[i];
    const double z = G.z;

    // dL/dSigma' (= dL/dSigma2, the dilation is additive), per element.  The
    // compositing pass summed W = V^T Qr (-A) Qr V with the record's fp32
    // conic Qr (A = dL/dconic); the derivative through the exact inverse is
    // -Q A Q = F W F^T with Q = Sigma'^-1 in fp64 and F = Q Qr^-1 V, a
    // rotation up to the rounding of the fp32 conic.
    double D00, D01, D11;
    {
        const double q00 = G.p11 / G.det, q01 = -(G.p01 / G.det), q11 = G.p00 / G.det;
        const double ra = cr.x, rb = cr.y, rc = cr.z;
        const double rdet = ra * rc - rb * rb;
        const double i00 = rc / rdet, i01 = -rb / rdet, i11 = ra / rdet;   // Qr^-1
        const double E00 = q00 * i00 + q01 * i01, E01 = q00 * i01 + q01 * i11;
        const double E10 = q01 * i00 + q11 * i01, E11 = q01 * i01 + q11 * i11;
        // F = E V, V = [[ex, -ey], [ey, ex]]
        const double F00 = E00 * ex + E01 * ey, F01 = -(E00 * ey) + E01 * ex;
        const double F10 = E10 * ex + E11 * ey, F11 = -(E10 * ey) + E11 * ex;
        const double W00 = g2[2], W01 = g2[3], W11 = g2[4];
        const double P00 = F00 * W00 + F01 * W01, P01 = F00 * W01 + F01 * W11;
        const double P10 = F10 * W00 + F11 * W01, P11 = F10 * W01 + F11 * W11;
        D00 = P00 * F00 + P01 * F01;
        D01 = P00 * F10 + P01 * F11;
        D11 = P10 * F10 + P11 * F11;
    }
    const double *T = G.T;
    const double Sg[3][3] = {{G.S[0], G.S[1], G.S[2]}, {G.S[1], G.S[3], G.S[4]}, {G.S[2], G.S[4], G.S[5]}};
    double DT[2][3];
#pragma unroll
    for (int l = 0; l < 3; l++) {
        DT[0][l] = D00 * T[l] + D01 * T[3 + l];
        DT[1][l] = D01 * T[l] + D11 * T[3 + l];
    }
    double dT[2][3];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int k = 0; k < 3; k++)
            dT[i][k] = 2.0 * (DT[i][0] * Sg[0][k] + DT[i][1] * Sg[1][k] + DT[i][2] * Sg[2][k]);
    const double dJ00 = dT[0][0] * R[0] + dT[0][1] * R[1] + dT[0][2] * R[2];
    const double dJ02 = dT[0][0] * R[6] + dT[0][1] * R[7] + dT[0][2] * R[8];
    const double dJ11 = dT[1][0] * R[3] + dT[1][1] * R[4] + dT[1][2] * R[5];
    const double dJ12 = dT[1][0] * R[6] + dT[1][1] * R[7] + dT[1][2] * R[8];

    const double fx = cam.fx, fy = cam.fy;
    const double iz = 1.0 / z, iz2 = iz * iz;
    double dpx = gu * fx * iz;
    double dpy = gv * fy * iz;
    double dpz = -(gu * fx * G.x + gv * fy * G.y) * iz2;
    dpz = dpz - (dJ00 * fx + dJ11 * fy) * iz2;
    if (!G.clx) {
        dpx = dpx - dJ02 * fx * iz2;
        dpz = dpz + dJ02 * 2.0 * fx * G.x * iz2 * iz;
    } else {
        dpz = dpz + dJ02 * fx * (G.J02 * (-z / fx)) * iz2;   // fx * (xg/z) / z^2
    }
    if (!G.cly) {
        dpy = dpy - dJ12 * fy * iz2;
        dpz = dpz + dJ12 * 2.0 * fy * G.y * iz2 * iz;
    } else {
        dpz = dpz + dJ12 * fy * (G.J12 * (-z / fy)) * iz2;
    }

    // Sigma's gradient T^T D T (symmetric: its upper triangle, 00 01 02 11
    // 12 22) is summed over the views in fp64; the rest of the chain (Sigma =
    // M M^T, M = Rq diag(s), the quaternion) is linear in it and
    // view-independent, so it runs once after the loop
#pragma unroll
    for (int k = 0, e = 0; k < 3; k++)
#pragma unroll
        for (int l = k; l < 3; l++, e++) dS_sum[e] += T[k] * DT[0][l] + T[3 + k] * DT[1][l];

#pragma unroll
    for (int j = 0; j < 3; j++) {
        const float c = (float)(R[j] * dpx + R[3 + j] * dpy + R[6 + j] * dpz);
        acc_mean[j] += c;
        if constexpr (kMotion) acc_vel[j] += dtv * c;
    }
    acc_logit += o * (1.0f - o) * go;
    }   // views
    if (!touched) return;
    {
        GeoT<double> H;
        rot_scale<double>(s0, s1, s2, qw0, qx0, qy0, qz0, H);   // a touched Gaussian has a non-zero quaternion
        const double *M = H.M, *Q = H.Rq;
        const double sd[3] = {s0, s1, s2};
        const double dSg[3][3] = {{dS_sum[0], dS_sum[1], dS_sum[2]},
                                  {dS_sum[1], dS_sum[3], dS_sum[4]},
                                  {dS_sum[2], dS_sum[4], dS_sum[5]}};
        double dM[9];
#pragma unroll
        for (int i = 0; i < 3; i++)
#pragma unroll
            for (int j = 0; j < 3; j++)
                dM[i * 3 + j] = 2.0 * (dSg[i][0] * M[j] + dSg[i][1] * M[3 + j] + dSg[i][2] * M[6 + j]);
        double ds[3];
#pragma unroll
        for (int j = 0; j < 3; j++) ds[j] = Q[j] * dM[j] + Q[3 + j] * dM[3 + j] + Q[6 + j] * dM[6 + j];
        double dR[9];
#pragma unroll
        for (int i = 0; i < 3; i++)
#pragma unroll
            for (int j = 0; j < 3; j++) dR[i * 3 + j] = dM[i * 3 + j] * sd[j];
        const double w = H.w, a = H.qa, b = H.qb, c = H.qc;
        double dq[4];
        dq[0] = 2.0 * (-c * dR[1] + b * dR[2] + c * dR[3] - a * dR[5] - b * dR[6] + a * dR[7]);
        dq[1] = 2.0 * (b * dR[1] + c * dR[2] + b * dR[3] - w * dR[5] + c * dR[6] + w * dR[7]) -
                4.0 * a * (dR[4] + dR[8]);
        dq[2] = 2.0 * (a * dR[1] + w * dR[2] + a * dR[3] + c * dR[5] - w * dR[6] + c * dR[7]) -
                4.0 * b * (dR[0] + dR[8]);
        dq[3] = 2.0 * (-w * dR[1] + a * dR[2] + w * dR[3] + b * dR[5] + a * dR[6] + b * dR[7]) -
                4.0 * c * (dR[0] + dR[4]);
        const double qdot = w * dq[0] + a * dq[1] + b * dq[2] + c * dq[3];
        const double qh[4] = {w, a, b, c};
#pragma unroll
        for (int r = 0; r < 3; r++) acc_ls[r] = (float)(sd[r] * ds[r]);
#pragma unroll
        for (int r = 0; r < 4; r++) acc_q[r] = (float)((dq[r] - qh[r] * qdot) / H.nq);
    }
#pragma unroll
    for (int j = 0; j < 3; j++) d_means[j * n + g] += acc_mean[j];
    if constexpr (kMotion) {
#pragma unroll
        for (int j = 0; j < 3; j++) mo.dv[j * n + g] += acc_vel[j];
        mo.dt[g] -= (vx * acc_mean[0] + vy * acc_mean[1]) + vz * acc_mean[2];
    }
#pragma unroll
    for (int j = 0; j < 3; j++) d_log_scales[j * n + g] += acc_ls[j];
#pragma unroll
    for (int j = 0; j < 4; j++) d_quats[j * n + g] += acc_q[j];
    d_logits[g] += acc_logit;
}

template <bool COMPACT, bool kMotion>
__global__ __launch_bounds__(kBlock) void project_bwd_geom_kernel(
    int n, int per_wave, const float *__restrict__ means, const float *__restrict__ scales,
    const float *__restrict__ quats, const float *__restrict__ opac, const uint8_t *__restrict__ active,
    const Motion mo, const ViewBatch views, float *__restrict__ d_means, float *__restrict__ d_log_scales,
    float *__restrict__ d_quats, float *__restrict__ d_logits)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if constexpr (COMPACT) {
        __shared__ uint32_t s_list[kBlock / 64][kMaxCompact];
        const long long g_begin = ((long long)blockIdx.x * (kBlock / 64) + wv) * per_wave;
        const long long g_end = g_begin + per_wave < n ? g_begin + per_wave : n;
        const int cnt = compact_range(g_begin, g_end, active, views, s_list[wv]);
        for (int r0 = 0; r0 < cnt; r0 += 64) {
            const int idx = r0 + lane;
            if (idx < cnt)
                geom_backward<kMotion>(n, (int)s_list[wv][idx], means, scales, quats, opac, mo, views, d_means,
                                       d_log_scales, d_quats, d_logits);
        }
    } else {
        const long long g = (long long)blockIdx.x * kBlock + threadIdx.x;
        if (g >= n || (active != nullptr && active[g] == 0)) return;
        bool any = false;   // culled in every view: nothing to read or write
        for (int v = 0; v < views.count; v++) any = any | seen(views, v, g);
        if (!any) return;
        geom_backward<kMotion>(n, (int)g, means, scales, quats, opac, mo, views, d_means, d_log_scales, d_quats,
                               d_logits);
    }
}


Motion motion_of(const gs_gaussians &g, const gs_grads *out)
{
    Motion m;
    m.v = g.velocity;
    m.t = g.t_offset;
    m.dv = out ? out->velocity : nullptr;
    m.dt = out ? out->t_offset : nullptr;
    return m;
}

template <int DEG, typename TSH, bool kMotion>
void launch_project_m(const gs_gaussians &g, const ProjBatch &views, hipStream_t s)
{
    const int n = (int)g.n;
    project_kernel<DEG, TSH, kMotion><<<(n + kBlock - 1) / kBlock, kBlock, 0, s>>>(
        n, g.means, g.scales, g.quats, g.opacities, (const TSH *)g.sh, g.sh_bounds, g.active, motion_of(g, nullptr),
        views);
}

template <int DEG, typename TSH>
void launch_project_t(const gs_gaussians &g, const ProjBatch &views, hipStream_t s)
{
    if (g.velocity)
        launch_project_m<DEG, TSH, true>(g, views, s);
    else
        launch_project_m<DEG, TSH, false>(g, views, s);
}

template <int DEG, typename TSH, bool kMotion>
void launch_project_bwd_m(const gs_gaussians &g, const ViewBatch &views, const gs_grads &out, hipStream_t s)
{
    const int n = (int)g.n;
    const Motion mo = motion_of(g, &out);
    if (g.active == nullptr) {
        const long long colour_waves = (n + kColourPerWave - 1) / kColourPerWave;
        project_bwd_color_kernel<DEG, TSH, false, kMotion>
            <<<(unsigned)((colour_waves + kBlock / 64 - 1) / (kBlock / 64)), kBlock, 0, s>>>(
                n, 0, g.means, (const TSH *)g.sh, g.sh_bounds, nullptr, mo, views, out.means, out.sh);
        project_bwd_geom_kernel<false, kMotion><<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(
            n, 0, g.means, g.scales, g.quats, g.opacities, nullptr, mo, views, out.means, out.log_scales, out.quats,
            out.opacity_logits);
        return;
    }
    // With a mask: ranges large enough that a compacted wave is mostly full,
    // while keeping ~16K waves
    long long m = (long long)n / (64LL * 16384);
    if (m < 1) m = 1;
    if (m > kMaxCompact / 64) m = kMaxCompact / 64;
    const int per_wave = (int)(64 * m);
    const long long waves = (n + per_wave - 1) / per_wave;
    const unsigned blocks = (unsigned)((waves + kBlock / 64 - 1) / (kBlock / 64));
    project_bwd_color_kernel<DEG, TSH, true, kMotion><<<blocks, kBlock, 0, s>>>(
        n, per_wave, g.means, (const TSH *)g.sh, g.sh_bounds, g.active, mo, views, out.means, out.sh);
    project_bwd_geom_kernel<true, kMotion><<<blocks, kBlock, 0, s>>>(n, per_wave, g.means, g.scales, g.quats,
                                                                     g.opacities, g.active, mo, views, out.means,
                                                                     out.log_scales, out.quats, out.opacity_logits);
}

template <int DEG, typename TSH>
void launch_project_bwd_t(const gs_gaussians &g, const ViewBatch &views, const gs_grads &out, hipStream_t s)
{
    if (g.velocity)
        launch_project_bwd_m<DEG, TSH, true>(g, views, out, s);
    else
        launch_project_bwd_m<DEG, TSH, false>(g, views, out, s);
}

template <typename TSH>
void dispatch_project(int deg, const gs_gaussians &g, const ProjBatch &views, hipStream_t s)
{
    switch (deg) {
    case 0: launch_project_t<0, TSH>(g, views, s); break;
    case 1: launch_project_t<1, TSH>(g, views, s); break;
    case 2: launch_project_t<2, TSH>(g, views, s); break;
    default: launch_project_t<3, TSH>(g, views, s); break;
    }
}

template <typename TSH>
void dispatch_project_bwd(int deg, const gs_gaussians &g, const ViewBatch &views, const gs_grads &out,
                          hipStream_t s)
{
    switch (deg) {
    case 0: launch_project_bwd_t<0, TSH>(g, views, out, s); break;
    case 1: launch_project_bwd_t<1, TSH>(g, views, out, s); break;
    case 2: launch_project_bwd_t<2, TSH>(g, views, out, s); break;
    default: launch_project_bwd_t<3, TSH>(g, views, out, s); break;
    }
}

}  // namespace

hipError_t launch_project(const gs_gaussians &g, const ProjBatch &views, hipStream_t s)
{
    if (g.n == 0 || views.count == 0) return hipSuccess;
    if (g.sh_dtype == GS_SH_F16)
        dispatch_project<__half>(g.sh_degree, g, views, s);
    else if (g.sh_dtype == GS_SH_Q8)
        dispatch_project<uint8_t>(g.sh_degree, g, views, s);
    else
        dispatch_project<float>(g.sh_degree, g, views, s);
    return hipGetLastError();
}

namespace {
// 8-bit block quantization of SH rows: one block per (256-Gaussian block,
// row); the block's min and max by wave and block reductions, then every
// code in fp32 with the documented order of operations.
__global__ __launch_bounds__(kBlock) void sh_quantize8_kernel(const float *__restrict__ x, int n, int nb,
                                                             uint8_t *__restrict__ q, float *__restrict__ bounds)
{
#pragma clang fp contract(off)
    __shared__ float s_lo[kBlock / 64], s_hi[kBlock / 64];
    const int row = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
    const int g0 = b * 256;
    const int g = g0 + tid;
    const bool valid = g < n;
    const float *xr = x + (size_t)row * n;
    const float v = xr[valid ? g : g0];        // padding lanes repeat the block's first value
    float lo = v, hi = v;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    if ((tid & 63) == 0) {
        s_lo[tid >> 6] = lo;
        s_hi[tid >> 6] = hi;
    }
    __syncthreads();
    lo = s_lo[0];
    hi = s_hi[0];
#pragma unroll
    for (int w = 1; w < kBlock / 64; w++) {
        lo = fminf(lo, s_lo[w]);
        hi = fmaxf(hi, s_hi[w]);
    }
    if (tid == 0) {
        bounds[((size_t)row * nb + b) * 2] = lo;
        bounds[((size_t)row * nb + b) * 2 + 1] = hi;
    }
    if (!valid) return;
    const float d = hi - lo;
    uint8_t c = 0;
    if (d > 0.0f) {
        const float t = ((v - lo) * 255.0f) / d;
        const float f = floorf(t + 0.5f);
        c = f >= 255.0f ? (uint8_t)255 : (uint8_t)f;
    }
    q[(size_t)row * n + g] = c;
}
}  // namespace

hipError_t launch_sh_quantize8(const float *sh, int64_t n, int rows, uint8_t *codes, float *bounds, hipStream_t s)
{
    const int nb = (int)((n + 255) / 256);
    sh_quantize8_kernel<<<dim3(nb, rows), kBlock, 0, s>>>(sh, (int)n, nb, codes, bounds);
    return hipGetLastError();
}

hipError_t launch_sum_partials(const SumBatch &batch, hipStream_t s)
{
    int n_max = 0;
    for (int i = 0; i < batch.count; i++) n_max = batch.v[i].n > n_max ? batch.v[i].n : n_max;
    if (batch.count == 0 || n_max == 0) return hipSuccess;
    const long long waves = (n_max + kSumPerWave - 1) / kSumPerWave;
    const unsigned blocks = (unsigned)((waves * 64 + kBlock - 1) / kBlock);
    sum_partials_kernel<<<dim3(blocks, batch.count), kBlock, 0, s>>>(batch);
    return hipGetLastError();
}

hipError_t launch_project_bwd(const gs_gaussians &g, const ViewBatch &views, const gs_grads &out, hipStream_t s)
{
    if (g.n == 0 || views.count == 0) return hipSuccess;
    if (g.sh_dtype == GS_SH_F16)
        dispatch_project_bwd<__half>(g.sh_degree, g, views, out, s);
    else if (g.sh_dtype == GS_SH_Q8)
        dispatch_project_bwd<uint8_t>(g.sh_degree, g, views, out, s);
    else
        dispatch_project_bwd<float>(g.sh_degree, g, views, out, s);
    return hipGetLastError();
}

}  // namespace gsi
