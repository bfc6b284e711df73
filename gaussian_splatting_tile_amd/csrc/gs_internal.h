// Internal declarations of the gfx950 rasterizer library (not installed; the
// public interface is include/gs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "gs.h"

namespace gsi {

constexpr int kTile = 16;                 // tile side in pixels
constexpr int kTilePixels = kTile * kTile;
constexpr int kBlock = 256;               // threads per block (4 wave64)

// Tile rectangle of a splat: the half-open range of 16x16 tiles meeting the
// square [u - r, u + r] x [v - r, v + r], clamped to the grid.  Every step is
// exact or one correctly rounded fp32 operation, so the projection and the
// binning kernels (and any other IEEE fp32 implementation of the same steps)
// agree bit for bit.
struct Rect { int x0, x1, y0, y1; };

__device__ __forceinline__ Rect tile_rect(float u, float v, float rf, float tiles_x, float tiles_y)
{
#pragma clang fp contract(off)
    float fx0 = floorf((u - rf) / 16.0f);
    float fx1 = floorf((u + rf) / 16.0f) + 1.0f;
    float fy0 = floorf((v - rf) / 16.0f);
    float fy1 = floorf((v + rf) / 16.0f) + 1.0f;
    fx0 = fminf(fmaxf(fx0, 0.0f), tiles_x);
    fx1 = fminf(fmaxf(fx1, 0.0f), tiles_x);
    fy0 = fminf(fmaxf(fy0, 0.0f), tiles_y);
    fy1 = fminf(fmaxf(fy1, 0.0f), tiles_y);
    return Rect{(int)fx0, (int)fx1, (int)fy0, (int)fy1};
}

// Can any pixel centre of the box of pixels [x0, x0 + w] x [y0, y0 + h]
// (inclusive, pixel indices) reach alpha >= 1/255?  The minimum of
// Q(d) = a dx^2 + 2 b dx dy + c dy^2 over the box of pixel centres is at the
// mean if it lies inside, else on an edge, where Q is a 1D quadratic
// minimised in closed form.  A record is dropped only when o exp(-Q_min / 2)
// is below 1/255 by a relative margin of 1e-3, far above the error of the
// per-pixel evaluation.
// The edge minimiser is located in fp32 and clamped into the box; Q is then
// evaluated there in fp64.  Q at any point of the box is >= its minimum, and
// the location error only adds c * O(ulp)^2 (Q is stationary there), far
// inside the margin.
__device__ __forceinline__ bool box_may_contribute(float fu, float fv, const float4 &conic_o, int x0, int y0, int w,
                                                   int h)
{
    const double a = conic_o.x, b = conic_o.y, c = conic_o.z;
    const double W = (double)w, H = (double)h;
    const double dxl = (double)x0 + 0.5 - (double)fu, dyl = (double)y0 + 0.5 - (double)fv;
    if (dxl <= 0.0 && dxl + W >= 0.0 && dyl <= 0.0 && dyl + H >= 0.0) return true;
    const float rb_c = -conic_o.y / conic_o.z, rb_a = -conic_o.y / conic_o.x;
    const float fxl = (float)dxl, fyl = (float)dyl;
    double best = 1e300;
#pragma unroll 1
    for (int e = 0; e < 4; e++) {
        double dx, dy;
        if (e < 2) {                   // edges x = const: minimise over dy
            dx = dxl + W * e;
            dy = (double)fminf(fmaxf(rb_c * (float)dx, fyl), fyl + (float)h);
            dy = fmin(fmax(dy, dyl), dyl + H);
        } else {                       // edges y = const: minimise over dx
            dy = dyl + H * (e - 2);
            dx = (double)fminf(fmaxf(rb_a * (float)dy, fxl), fxl + (float)w);
            dx = fmin(fmax(dx, dxl), dxl + W);
        }
        best = fmin(best, a * dx * dx + 2.0 * b * dx * dy + c * dy * dy);
    }
    const float amax = conic_o.w * __expf((float)(-0.5 * best));
    return amax >= (1.0f / 255.0f) * (1.0f - 1e-3f);
}

// The sort's per-Gaussian inputs: the depth key (fp32 depth bits; the
// sentinel, which no finite depth has, for a Gaussian that touches no tile)
// and the tile rect packed as (x0 | y0 << 16, width | height << 16).
constexpr uint32_t kSentinel = 0xFFFFFFFFu;

__device__ __forceinline__ uint2 pack_rect(const Rect &r)
{
    return make_uint2((uint32_t)r.x0 | ((uint32_t)r.y0 << 16),
                      (uint32_t)(r.x1 - r.x0) | ((uint32_t)(r.y1 - r.y0) << 16));
}

// Principal frame of a 2D conic [[a, b], [b, c]] in fp64: the unit
// eigenvector (ex, ey) of the larger eigenvalue l1 and the smaller one l2;
// the second axis is (-ey, ex).  Each component of the eigenvector is formed
// without cancellation; an isotropic conic gets the x axis.  The blend
// backward expresses the covariance gradient in this frame and the
// projection backward maps it back with the same frame.
__device__ __forceinline__ void conic_frame(double a, double b, double c, double &ex, double &ey, double &l1,
                                            double &l2)
{
    const double hd = 0.5 * (a - c);
    const double h = sqrt(hd * hd + b * b);
    l1 = 0.5 * (a + c) + h;
    l2 = 0.5 * (a + c) - h;       // relative error ~1e-16 l1 / l2, ample in fp64
    double vx, vy;
    if (hd >= 0.0) {
        vx = hd + h;
        vy = b;
    } else {
        vx = b;
        vy = h - hd;
    }
    const double nrm = sqrt(vx * vx + vy * vy);
    if (nrm > 0.0) {
        const double inv = 1.0 / nrm;
        ex = vx * inv;
        ey = vy * inv;
    } else {
        ex = 1.0;
        ey = 0.0;
    }
}

// Camera as the kernels take it (by value, in the kernel argument segment).
struct Cam {
    int width, height, tiles_x, tiles_y;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    float znear, guard, lod;
    float time;                           // the view's time (moving Gaussians)
};

inline Cam make_cam(const gs_camera &c)
{
    Cam k;
    k.width = c.width;
    k.height = c.height;
    k.tiles_x = (c.width + kTile - 1) / kTile;
    k.tiles_y = (c.height + kTile - 1) / kTile;
    k.fx = c.fx; k.fy = c.fy; k.cx = c.cx; k.cy = c.cy;
    for (int i = 0; i < 3; i++) {
        for (int j = 0; j < 3; j++) k.R[i * 3 + j] = c.viewmat[i * 4 + j];
        k.t[i] = c.viewmat[i * 4 + 3];
    }
    k.znear = c.znear;
    k.guard = c.guard;
    k.lod = c.lod_min_radius_px;
    k.time = c.time;
    return k;
}

// Splat record as the kernels see it: three 16-byte words.
struct __align__(16) Splat {
    float4 a;   // u, v, depth, radius (int bits)
    float4 b;   // conic a, b, c, opacity
    float4 c;   // r, g, b, tiles_touched (uint bits)
};
static_assert(sizeof(Splat) == sizeof(gs_splat), "splat layout");

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- launch helpers (host) -------------------------------------------------
// Views one projection launch writes records for (parameters read once).
constexpr int kMaxProjViews = 16;
struct ProjBatch {
    int count;
    Cam cam[kMaxProjViews];
    Splat *out[kMaxProjViews];
    // optional per view (both or neither): the sort's depth keys and packed
    // tile rects, written beside the records
    uint32_t *dkeys[kMaxProjViews];
    uint2 *grect[kMaxProjViews];
};
hipError_t launch_project(const gs_gaussians &g, const ProjBatch &views, hipStream_t s);
hipError_t launch_sh_quantize8(const float *sh, int64_t n, int rows, uint8_t *codes, float *bounds, hipStream_t s);
// Per-Gaussian screen-space gradients, g2[n][9], of up to kMaxSumViews views
// in one launch, from the blend backward's per-slot partial sums.
constexpr int kMaxSumViews = 8;
struct SumView {
    int n;
    const float *partial;         // [k_capacity][9]
    const uint32_t *order;        // the visible Gaussians in depth order
    const uint32_t *off;          // their first duplication slots (+ K at the end)
    const uint32_t *count;        // the number of visible Gaussians
    uint64_t k_capacity;
    float *g2;                    // [n][9]
};
struct SumBatch {
    int count;
    SumView v[kMaxSumViews];
};
hipError_t launch_sum_partials(const SumBatch &batch, hipStream_t s);

// Views whose screen-space gradients one projection-backward launch takes.
constexpr int kMaxViews = 16;
struct ViewBatch {
    int count;
    Cam cam[kMaxViews];
    const Splat *splats[kMaxViews];
    const float *g2[kMaxViews];
    const uint32_t *dkeys[kMaxViews];   // optional: the projection's depth keys (visibility)
};
hipError_t launch_project_bwd(const gs_gaussians &g, const ViewBatch &views, const gs_grads &out,
                              hipStream_t s);

size_t bin_sort_workspace(int64_t n, int64_t k_capacity, int n_tiles);
size_t schedule_words(int n_tiles);
// Views one binning launch sequence sorts together.
constexpr int kMaxSortViews = 8;
struct SortJob {
    const Splat *splats;
    int64_t n;
    Cam cam;
    int64_t cap;                  // key capacity
    uint32_t *vals, *ranges, *schedule;
    uint32_t *bwd_index;          // optional
    uint64_t *keys;               // optional
    uint64_t *k_total;
    void *ws;                     // bin_sort_workspace(n, cap) bytes
    const uint32_t *dkeys;        // optional (both or neither): depth keys and
    const uint2 *grect;           // tile rects from the projection
    bool reach;                   // list only the tiles each Gaussian reaches
};
hipError_t launch_bin_sort_views(int count, const SortJob *jobs, hipStream_t s);
size_t active_mask_workspace(int64_t n);
hipError_t launch_active_mask(const float *scores, int64_t n, int64_t keep, uint8_t *mask, void *ws,
                              size_t ws_bytes, hipStream_t s);
// gs_active_mask with the library's own fixed scratch array (no workspace).
size_t static_mask_scratch_bytes();
hipError_t launch_active_mask_static(const float *scores, int64_t n, int64_t keep, uint8_t *mask, hipStream_t s);

// Views blended by one launch: their tiles form one work queue.
constexpr int kMaxBlendViews = 8;
struct FwdView {
    Cam cam;
    const Splat *splats;
    const uint32_t *vals;
    const uint32_t *ranges;
    const uint32_t *order;        // the view's schedule (tiles, longest list first)
    float *image;
    float *final_T;
    uint32_t *n_contrib;
    float *weight;                // optional: += per-Gaussian blending weights
    int tile_test;                // apply the per-entry tile test while staging
};
struct FwdBatch {
    int count;
    int max_tiles;                // items = count * max_tiles, view = item % count
    float bg[3];
    uint32_t *queue;              // head, done: the first view's forward counters
    FwdView v[kMaxBlendViews];
};
hipError_t launch_render_fwd(const FwdBatch &batch, hipStream_t s);
// Views whose blend backward one launch runs over one work queue.
struct BwdView {
    Cam cam;
    const Splat *splats;
    const uint32_t *vals;
    const uint32_t *ranges;
    const uint32_t *order;        // the view's schedule
    const uint32_t *entry_slots;  // duplication slot of each sorted entry
    const float *final_T;
    const uint32_t *n_contrib;
    const float *dL_dimage;
    float *partial;               // [k_capacity][9]
    int tile_test;                // apply the per-entry tile test while staging
};
struct BwdBatch {
    int count;
    int max_tiles;
    int view_major;               // items = views one after another (set by the launcher)
    float bg[3];
    uint32_t *queue;              // head, done: the first view's backward counters
    BwdView v[kMaxBlendViews];
};
hipError_t launch_render_bwd(const BwdBatch &batch, hipStream_t s);
static_assert(kMaxSumViews >= kMaxBlendViews, "a blend-backward batch is summed in one launch");

}  // namespace gsi
