// C ABI of the rasterizer (declared in include/gs.h): argument checks,
// workspace sizing and the launch sequence of each call.  No allocation, no
// synchronisation, no host round trip.
#include <math.h>
#include <string.h>

#include "gs_adam.h"
#include "gs_internal.h"

using namespace gsi;

namespace {

constexpr int32_t kVersion = 1;

bool finite_pos(float x) { return isfinite(x) && x > 0.0f; }

// Splat records and workspaces are read with 16-byte vector accesses.
bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool camera_ok(const gs_camera *c)
{
    if (!c) return false;
    if (c->width < 1 || c->height < 1 || c->width > 32768 || c->height > 32768) return false;
    if (!finite_pos(c->fx) || !finite_pos(c->fy) || !isfinite(c->cx) || !isfinite(c->cy)) return false;
    for (int i = 0; i < 12; i++)
        if (!isfinite(c->viewmat[i])) return false;
    // znear >= 0: every kept depth is then positive, the range on which the
    // depth key (the fp32 bit pattern of z) orders like z itself
    if (!isfinite(c->znear) || !(c->znear >= 0.0f) || !finite_pos(c->guard)) return false;
    if (!isfinite(c->lod_min_radius_px) || c->lod_min_radius_px < 0.0f) return false;
    if (!isfinite(c->time)) return false;
    return true;
}

gs_status gaussians_ok(const gs_gaussians *g)
{
    if (!g || g->n < 0 || g->n > INT32_MAX) return GS_ERR_INVALID_ARG;
    if (g->sh_degree < 0 || g->sh_degree > 3) return GS_ERR_UNSUPPORTED;
    if (g->sh_dtype != GS_SH_F32 && g->sh_dtype != GS_SH_F16 && g->sh_dtype != GS_SH_Q8)
        return GS_ERR_UNSUPPORTED;
    if (g->n > 0 && (!g->means || !g->scales || !g->quats || !g->opacities || !g->sh))
        return GS_ERR_INVALID_ARG;
    if (g->n > 0 && g->sh_dtype == GS_SH_Q8 && !g->sh_bounds) return GS_ERR_INVALID_ARG;
    if (g->n > 0 && (g->velocity != nullptr) != (g->t_offset != nullptr)) return GS_ERR_INVALID_ARG;
    return GS_OK;
}

gs_status from_hip(hipError_t e) { return e == hipSuccess ? GS_OK : GS_ERR_HIP; }

}  // namespace

extern "C" {

int32_t gs_version(void) { return kVersion; }

const char *gs_status_string(gs_status s)
{
    // a C caller may pass any int: take the value's bytes as an int first (a
    // load of an out-of-range value as the enum type is undefined in C++)
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
    case GS_OK: return "ok";
    case GS_ERR_INVALID_ARG: return "invalid argument";
    case GS_ERR_UNSUPPORTED: return "unsupported argument value";
    case GS_ERR_WORKSPACE: return "workspace too small";
    case GS_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

gs_status gs_project(const gs_gaussians *gaussians, const gs_camera *camera, gs_splat *splats,
                     void *stream)
{
    gs_status st = gaussians_ok(gaussians);
    if (st != GS_OK) return st;
    if (!camera_ok(camera)) return GS_ERR_INVALID_ARG;
    if ((gaussians->n > 0 && !splats) || !al16(splats)) return GS_ERR_INVALID_ARG;
    ProjBatch b;
    b.count = 1;
    b.cam[0] = make_cam(*camera);
    b.out[0] = (Splat *)splats;
    b.dkeys[0] = nullptr;
    b.grect[0] = nullptr;
    return from_hip(launch_project(*gaussians, b, (hipStream_t)stream));
}

// The sort inputs of one view: both pointers or neither, depth keys 4-byte
// and rects 8-byte aligned, and tile coordinates that fit the 16-bit fields.
// (The rects may be left out where only reached tiles are listed: that
// sort takes each rect from the record.)
static bool bin_keys_ok(const uint32_t *dk, const uint32_t *gr, const gs_camera &cam, bool rects_optional)
{
    if (dk == nullptr) return gr == nullptr;
    if (gr == nullptr && !rects_optional) return false;
    if (((uintptr_t)dk & 3u) != 0 || ((uintptr_t)gr & 7u) != 0) return false;
    const Cam c = make_cam(cam);
    return c.tiles_x <= 65535 && c.tiles_y <= 65535;
}

static gs_status project_views(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                               gs_splat *const *splats, const gs_bin_keys *bin_keys, void *stream)
{
    gs_status st = gaussians_ok(gaussians);
    if (st != GS_OK) return st;
    if (n_views < 0 || (n_views > 0 && (!cameras || !splats))) return GS_ERR_INVALID_ARG;
    for (int v = 0; v < n_views; v++) {
        if (!camera_ok(&cameras[v])) return GS_ERR_INVALID_ARG;
        if ((gaussians->n > 0 && !splats[v]) || !al16(splats[v])) return GS_ERR_INVALID_ARG;
        if (bin_keys && !bin_keys_ok(bin_keys[v].depth_keys, bin_keys[v].tile_rects, cameras[v], true))
            return GS_ERR_INVALID_ARG;
    }
    for (int v0 = 0; v0 < n_views; v0 += kMaxProjViews) {
        ProjBatch b;
        b.count = n_views - v0 < kMaxProjViews ? n_views - v0 : kMaxProjViews;
        for (int i = 0; i < kMaxProjViews; i++) {
            b.dkeys[i] = nullptr;
            b.grect[i] = nullptr;
        }
        for (int i = 0; i < b.count; i++) {
            b.cam[i] = make_cam(cameras[v0 + i]);
            b.out[i] = (Splat *)splats[v0 + i];
            if (bin_keys) {
                b.dkeys[i] = bin_keys[v0 + i].depth_keys;
                b.grect[i] = (uint2 *)bin_keys[v0 + i].tile_rects;
            }
        }
        hipError_t e = launch_project(*gaussians, b, (hipStream_t)stream);
        if (e != hipSuccess) return GS_ERR_HIP;
    }
    return GS_OK;
}

gs_status gs_project_views(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                           gs_splat *const *splats, void *stream)
{
    return project_views(gaussians, n_views, cameras, splats, nullptr, stream);
}

gs_status gs_project_views_binned(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                                  gs_splat *const *splats, const gs_bin_keys *bin_keys, void *stream)
{
    if (n_views > 0 && !bin_keys) return GS_ERR_INVALID_ARG;
    return project_views(gaussians, n_views, cameras, splats, bin_keys, stream);
}

size_t gs_bin_sort_workspace_bytes(int64_t n, int64_t k_capacity, int32_t n_tiles)
{
    if (n < 0 || k_capacity < 0) return 0;
    return bin_sort_workspace(n, k_capacity, n_tiles);
}

static int tiles_of(int32_t width, int32_t height)
{
    return ((width + kTile - 1) / kTile) * ((height + kTile - 1) / kTile);
}

size_t gs_schedule_words(int32_t width, int32_t height)
{
    if (width < 1 || height < 1 || width > 32768 || height > 32768) return 0;
    return schedule_words(tiles_of(width, height));
}

size_t gs_bwd_index_words(int64_t n, int64_t k_capacity)
{
    if (n < 0 || k_capacity < 0) return 0;
    return (size_t)k_capacity + 2 * (size_t)n + 2;
}

static gs_status check_sort_view(const gs_sort_view &v)
{
    if (v.n < 0 || v.n > INT32_MAX || v.k_capacity < 0 || v.k_capacity >= (int64_t)UINT32_MAX)
        return GS_ERR_INVALID_ARG;
    if (!camera_ok(&v.camera) || !v.tile_ranges || !v.schedule || !v.k_total) return GS_ERR_INVALID_ARG;
    if ((v.n > 0 && !v.splats) || !al16(v.splats) || !al16(v.workspace)) return GS_ERR_INVALID_ARG;
    if (v.k_capacity > 0 && !v.vals) return GS_ERR_INVALID_ARG;
    if (!bin_keys_ok(v.depth_keys, v.tile_rects, v.camera, v.reach_tiles != 0)) return GS_ERR_INVALID_ARG;
    const Cam cam = make_cam(v.camera);
    const size_t need = bin_sort_workspace(v.n, v.k_capacity, cam.tiles_x * cam.tiles_y);
    if (v.workspace_bytes < need || !v.workspace) return GS_ERR_WORKSPACE;
    return GS_OK;
}

static SortJob sort_job(const gs_sort_view &v)
{
    SortJob j;
    j.splats = (const Splat *)v.splats;
    j.n = v.n;
    j.cam = make_cam(v.camera);
    j.cap = v.k_capacity;
    j.vals = v.vals;
    j.ranges = v.tile_ranges;
    j.schedule = v.schedule;
    j.bwd_index = v.bwd_index;
    j.keys = v.keys;
    j.k_total = v.k_total;
    j.ws = v.workspace;
    j.dkeys = v.depth_keys;
    j.grect = (const uint2 *)v.tile_rects;
    j.reach = v.reach_tiles != 0;
    return j;
}

gs_status gs_bin_sort(const gs_splat *splats, int64_t n, const gs_camera *camera, int64_t k_capacity,
                      uint32_t *vals, uint32_t *tile_ranges, uint32_t *schedule, uint32_t *bwd_index,
                      uint64_t *keys, uint64_t *k_total, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    if (!camera) return GS_ERR_INVALID_ARG;
    gs_sort_view v;
    v.camera = *camera;
    v.splats = splats;
    v.n = n;
    v.k_capacity = k_capacity;
    v.vals = vals;
    v.tile_ranges = tile_ranges;
    v.schedule = schedule;
    v.bwd_index = bwd_index;
    v.keys = keys;
    v.k_total = k_total;
    v.workspace = workspace;
    v.workspace_bytes = workspace_bytes;
    v.depth_keys = nullptr;
    v.tile_rects = nullptr;
    v.reach_tiles = 0;
    return gs_bin_sort_views(1, &v, stream);
}

gs_status gs_bin_sort_views(int32_t n_views, const gs_sort_view *views, void *stream)
{
    if (n_views < 0 || (n_views > 0 && !views)) return GS_ERR_INVALID_ARG;
    for (int v = 0; v < n_views; v++) {
        const gs_status st = check_sort_view(views[v]);
        if (st != GS_OK) return st;
    }
    for (int v0 = 0; v0 < n_views; v0 += kMaxSortViews) {
        const int count = n_views - v0 < kMaxSortViews ? n_views - v0 : kMaxSortViews;
        SortJob jobs[kMaxSortViews];
        for (int i = 0; i < count; i++) jobs[i] = sort_job(views[v0 + i]);
        const gs_status st = from_hip(launch_bin_sort_views(count, jobs, (hipStream_t)stream));
        if (st != GS_OK) return st;
    }
    return GS_OK;
}

gs_status gs_render_fwd(const gs_splat *splats, const uint32_t *vals, const uint32_t *tile_ranges,
                        uint32_t *schedule, const gs_camera *camera, const float *bg, float *image,
                        float *final_T, uint32_t *n_contrib, void *stream)
{
    if (!camera_ok(camera) || !splats || !vals || !tile_ranges || !schedule || !bg || !image || !final_T ||
        !n_contrib || !al16(splats))
        return GS_ERR_INVALID_ARG;
    for (int c = 0; c < 3; c++)
        if (!isfinite(bg[c])) return GS_ERR_INVALID_ARG;
    FwdBatch b;
    b.count = 1;
    b.bg[0] = bg[0];
    b.bg[1] = bg[1];
    b.bg[2] = bg[2];
    b.v[0].cam = make_cam(*camera);
    b.max_tiles = b.v[0].cam.tiles_x * b.v[0].cam.tiles_y;
    b.queue = schedule + b.max_tiles;
    b.v[0].splats = (const Splat *)splats;
    b.v[0].vals = vals;
    b.v[0].ranges = tile_ranges;
    b.v[0].order = schedule;
    b.v[0].image = image;
    b.v[0].final_T = final_T;
    b.v[0].n_contrib = n_contrib;
    b.v[0].weight = nullptr;
    b.v[0].tile_test = 1;
    return from_hip(launch_render_fwd(b, (hipStream_t)stream));
}

gs_status gs_render_fwd_views(int32_t n_views, const gs_fwd_view *views, const float *bg, void *stream)
{
    if (n_views < 0 || (n_views > 0 && !views) || !bg) return GS_ERR_INVALID_ARG;
    for (int c = 0; c < 3; c++)
        if (!isfinite(bg[c])) return GS_ERR_INVALID_ARG;
    for (int v = 0; v < n_views; v++) {
        const gs_fwd_view &w = views[v];
        if (!camera_ok(&w.camera) || !w.splats || !w.vals || !w.tile_ranges || !w.schedule || !w.image ||
            !w.final_T || !w.n_contrib || !al16(w.splats))
            return GS_ERR_INVALID_ARG;
    }
    for (int v0 = 0; v0 < n_views; v0 += kMaxBlendViews) {
        FwdBatch b;
        b.count = n_views - v0 < kMaxBlendViews ? n_views - v0 : kMaxBlendViews;
        b.bg[0] = bg[0];
        b.bg[1] = bg[1];
        b.bg[2] = bg[2];
        b.max_tiles = 0;
        for (int i = 0; i < b.count; i++) {
            const gs_fwd_view &w = views[v0 + i];
            FwdView &d = b.v[i];
            d.cam = make_cam(w.camera);
            d.splats = (const Splat *)w.splats;
            d.vals = w.vals;
            d.ranges = w.tile_ranges;
            d.order = w.schedule;
            d.image = w.image;
            d.final_T = w.final_T;
            d.n_contrib = w.n_contrib;
            d.weight = w.weight;
            d.tile_test = w.reached_lists ? 0 : 1;
            const int nt = d.cam.tiles_x * d.cam.tiles_y;
            if (nt > b.max_tiles) b.max_tiles = nt;
        }
        // the queue counters of the batch's first view
        b.queue = views[v0].schedule + b.v[0].cam.tiles_x * b.v[0].cam.tiles_y;
        hipError_t e = launch_render_fwd(b, (hipStream_t)stream);
        if (e != hipSuccess) return GS_ERR_HIP;
    }
    return GS_OK;
}

static size_t partial_bytes(int64_t k_capacity) { return align_up((size_t)k_capacity * 9 * sizeof(float), 256); }

size_t gs_render_bwd_workspace_bytes(int64_t n, int64_t k_capacity)
{
    if (n < 0 || k_capacity < 0) return 0;
    return partial_bytes(k_capacity) + align_up((size_t)n * 9 * sizeof(float), 256) + 256;
}

size_t gs_render_bwd_screen_workspace_bytes(int64_t k_capacity)
{
    if (k_capacity < 0) return 0;
    return partial_bytes(k_capacity) + 256;
}

// Checks shared by the two backward entry points that take a view's forward outputs.
static gs_status screen_args_ok(const gs_camera *camera, int64_t n, const gs_splat *splats, const uint32_t *vals,
                                const uint32_t *tile_ranges, const uint32_t *schedule, const uint32_t *bwd_index,
                                int64_t k_capacity, const float *bg, const float *final_T,
                                const uint32_t *n_contrib, const float *dL_dimage)
{
    if (!camera_ok(camera) || !tile_ranges || !schedule || !bg || !final_T || !n_contrib || !dL_dimage ||
        n < 0 || n > INT32_MAX || k_capacity < 0 || k_capacity >= (int64_t)UINT32_MAX)
        return GS_ERR_INVALID_ARG;
    for (int c = 0; c < 3; c++)
        if (!isfinite(bg[c])) return GS_ERR_INVALID_ARG;
    if ((n > 0 && (!splats || !bwd_index)) || !al16(splats)) return GS_ERR_INVALID_ARG;
    if (k_capacity > 0 && !vals) return GS_ERR_INVALID_ARG;
    return GS_OK;
}

static bool grads_ok(const gs_grads *grads, int64_t n, bool motion)
{
    return grads && (n == 0 || (grads->means && grads->log_scales && grads->quats && grads->opacity_logits &&
                                grads->sh && (!motion || (grads->velocity && grads->t_offset))));
}

// The blend backward and the per-Gaussian sums of up to kMaxBlendViews views
// (g2[n][9] each).  Every entry's nine partial sums are written by the blend
// backward, so the partial buffers need no clearing.
static hipError_t screen_backward(int count, const gs_bwd_view *views, const float *bg, hipStream_t s)
{
    BwdBatch b;
    b.count = count;
    b.bg[0] = bg[0];
    b.bg[1] = bg[1];
    b.bg[2] = bg[2];
    b.max_tiles = 0;
    for (int i = 0; i < count; i++) {
        const gs_bwd_view &w = views[i];
        BwdView &d = b.v[i];
        d.cam = make_cam(w.camera);
        d.splats = (const Splat *)w.splats;
        d.vals = w.vals;
        d.ranges = w.tile_ranges;
        d.order = w.schedule;
        d.entry_slots = w.bwd_index;
        d.final_T = w.final_T;
        d.n_contrib = w.n_contrib;
        d.dL_dimage = w.dL_dimage;
        d.partial = (float *)w.workspace;
        d.tile_test = w.reached_lists ? 0 : 1;
        const int nt = d.cam.tiles_x * d.cam.tiles_y;
        if (nt > b.max_tiles) b.max_tiles = nt;
    }
    b.queue = views[0].schedule + b.v[0].cam.tiles_x * b.v[0].cam.tiles_y + 2;
    hipError_t e = launch_render_bwd(b, s);
    if (e != hipSuccess) return e;
    SumBatch sb;
    sb.count = count;
    for (int i = 0; i < count; i++) {
        const gs_bwd_view &w = views[i];
        sb.v[i].n = (int)w.n;
        sb.v[i].partial = (const float *)w.workspace;
        sb.v[i].order = w.bwd_index + w.k_capacity;
        sb.v[i].off = w.bwd_index + w.k_capacity + w.n;
        sb.v[i].count = w.bwd_index + w.k_capacity + 2 * w.n + 1;
        sb.v[i].k_capacity = (uint64_t)w.k_capacity;
        sb.v[i].g2 = w.g2;
    }
    return launch_sum_partials(sb, s);
}

gs_status gs_render_bwd(const gs_gaussians *gaussians, const gs_camera *camera, const gs_splat *splats,
                        const uint32_t *vals, const uint32_t *tile_ranges, uint32_t *schedule,
                        const uint32_t *bwd_index, int64_t k_capacity, const float *bg, const float *final_T,
                        const uint32_t *n_contrib, const float *dL_dimage, const gs_grads *grads,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    gs_status st = gaussians_ok(gaussians);
    if (st != GS_OK) return st;
    const int64_t n = gaussians->n;
    st = screen_args_ok(camera, n, splats, vals, tile_ranges, schedule, bwd_index, k_capacity, bg, final_T,
                        n_contrib, dL_dimage);
    if (st != GS_OK) return st;
    if (!grads_ok(grads, n, gaussians->velocity != nullptr)) return GS_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < gs_render_bwd_workspace_bytes(n, k_capacity)) return GS_ERR_WORKSPACE;
    if (!al16(workspace)) return GS_ERR_INVALID_ARG;
    if (n == 0) return GS_OK;
    hipStream_t s = (hipStream_t)stream;
    float *g2 = (float *)((char *)workspace + partial_bytes(k_capacity));
    gs_bwd_view w;
    w.camera = *camera;
    w.n = n;
    w.splats = splats;
    w.vals = vals;
    w.tile_ranges = tile_ranges;
    w.schedule = schedule;
    w.bwd_index = bwd_index;
    w.k_capacity = k_capacity;
    w.final_T = final_T;
    w.n_contrib = n_contrib;
    w.dL_dimage = dL_dimage;
    w.g2 = g2;
    w.workspace = workspace;
    w.workspace_bytes = workspace_bytes;
    w.reached_lists = 0;
    hipError_t e = screen_backward(1, &w, bg, s);
    if (e != hipSuccess) return GS_ERR_HIP;
    ViewBatch vb;
    vb.count = 1;
    vb.cam[0] = make_cam(*camera);
    vb.splats[0] = (const Splat *)splats;
    vb.g2[0] = g2;
    vb.dkeys[0] = nullptr;
    return from_hip(launch_project_bwd(*gaussians, vb, *grads, s));
}

gs_status gs_render_bwd_screen(const gs_camera *camera, int64_t n, const gs_splat *splats, const uint32_t *vals,
                               const uint32_t *tile_ranges, uint32_t *schedule, const uint32_t *bwd_index,
                               int64_t k_capacity, const float *bg, const float *final_T,
                               const uint32_t *n_contrib, const float *dL_dimage, float *g2, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    gs_status st = screen_args_ok(camera, n, splats, vals, tile_ranges, schedule, bwd_index, k_capacity, bg,
                                  final_T, n_contrib, dL_dimage);
    if (st != GS_OK) return st;
    if (n > 0 && !g2) return GS_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < gs_render_bwd_screen_workspace_bytes(k_capacity)) return GS_ERR_WORKSPACE;
    if (!al16(workspace)) return GS_ERR_INVALID_ARG;
    if (n == 0) return GS_OK;
    gs_bwd_view w;
    w.camera = *camera;
    w.n = n;
    w.splats = splats;
    w.vals = vals;
    w.tile_ranges = tile_ranges;
    w.schedule = schedule;
    w.bwd_index = bwd_index;
    w.k_capacity = k_capacity;
    w.final_T = final_T;
    w.n_contrib = n_contrib;
    w.dL_dimage = dL_dimage;
    w.g2 = g2;
    w.workspace = workspace;
    w.workspace_bytes = workspace_bytes;
    w.reached_lists = 0;
    return from_hip(screen_backward(1, &w, bg, (hipStream_t)stream));
}

gs_status gs_render_bwd_screen_views(int32_t n_views, const gs_bwd_view *views, const float *bg, void *stream)
{
    if (n_views < 0 || (n_views > 0 && !views) || !bg) return GS_ERR_INVALID_ARG;
    for (int v = 0; v < n_views; v++) {
        const gs_bwd_view &w = views[v];
        gs_status st = screen_args_ok(&w.camera, w.n, w.splats, w.vals, w.tile_ranges, w.schedule, w.bwd_index,
                                      w.k_capacity, bg, w.final_T, w.n_contrib, w.dL_dimage);
        if (st != GS_OK) return st;
        if (w.n > 0 && !w.g2) return GS_ERR_INVALID_ARG;
        if (!w.workspace || w.workspace_bytes < gs_render_bwd_screen_workspace_bytes(w.k_capacity))
            return GS_ERR_WORKSPACE;
        if (!al16(w.workspace)) return GS_ERR_INVALID_ARG;
    }
    // views without Gaussians have nothing to do; the rest go in batches
    gs_bwd_view batch[kMaxBlendViews];
    int count = 0;
    for (int v = 0; v <= n_views; v++) {
        if (v < n_views && views[v].n > 0) batch[count++] = views[v];
        if (count == kMaxBlendViews || (v == n_views && count > 0)) {
            hipError_t e = screen_backward(count, batch, bg, (hipStream_t)stream);
            if (e != hipSuccess) return GS_ERR_HIP;
            count = 0;
        }
    }
    return GS_OK;
}

namespace {
gs_status project_bwd(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                      const gs_splat *const *splats, const float *const *g2, const uint32_t *const *depth_keys,
                      const gs_grads *grads, void *stream)
{
    gs_status st = gaussians_ok(gaussians);
    if (st != GS_OK) return st;
    const int64_t n = gaussians->n;
    if (n_views < 0 || (n_views > 0 && (!cameras || !splats || !g2))) return GS_ERR_INVALID_ARG;
    if (!grads_ok(grads, n, gaussians->velocity != nullptr)) return GS_ERR_INVALID_ARG;
    for (int v = 0; v < n_views; v++) {
        if (!camera_ok(&cameras[v])) return GS_ERR_INVALID_ARG;
        if ((n > 0 && (!splats[v] || !g2[v])) || !al16(splats[v])) return GS_ERR_INVALID_ARG;
        if (depth_keys && ((uintptr_t)depth_keys[v] & 3u) != 0) return GS_ERR_INVALID_ARG;
    }
    if (n == 0) return GS_OK;
    hipStream_t s = (hipStream_t)stream;
    // batches of up to kMaxViews views per launch, in view order
    for (int v0 = 0; v0 < n_views; v0 += kMaxViews) {
        ViewBatch vb;
        vb.count = n_views - v0 < kMaxViews ? n_views - v0 : kMaxViews;
        for (int i = 0; i < vb.count; i++) {
            vb.cam[i] = make_cam(cameras[v0 + i]);
            vb.splats[i] = (const Splat *)splats[v0 + i];
            vb.g2[i] = g2[v0 + i];
            vb.dkeys[i] = depth_keys ? depth_keys[v0 + i] : nullptr;
        }
        hipError_t e = launch_project_bwd(*gaussians, vb, *grads, s);
        if (e != hipSuccess) return GS_ERR_HIP;
    }
    return GS_OK;
}
}  // namespace

gs_status gs_project_bwd(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                         const gs_splat *const *splats, const float *const *g2, const gs_grads *grads, void *stream)
{
    return project_bwd(gaussians, n_views, cameras, splats, g2, nullptr, grads, stream);
}

gs_status gs_project_bwd_binned(const gs_gaussians *gaussians, int32_t n_views, const gs_camera *cameras,
                                const gs_splat *const *splats, const float *const *g2,
                                const uint32_t *const *depth_keys, const gs_grads *grads, void *stream)
{
    if (n_views > 0 && !depth_keys) return GS_ERR_INVALID_ARG;
    return project_bwd(gaussians, n_views, cameras, splats, g2, depth_keys, grads, stream);
}

size_t gs_active_mask_workspace_bytes(int64_t n)
{
    if (n < 0) return 0;
    return active_mask_workspace(n);
}

gs_status gs_active_mask(const float *scores, int64_t n, int64_t keep, uint8_t *mask, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (n < 0 || n > INT32_MAX || keep < 0 || keep > n) return GS_ERR_INVALID_ARG;
    if (n > 0 && (!scores || !mask)) return GS_ERR_INVALID_ARG;
    if (workspace_bytes < active_mask_workspace(n) || (!workspace && active_mask_workspace(n) > 0))
        return GS_ERR_WORKSPACE;
    if (!al16(workspace)) return GS_ERR_INVALID_ARG;
    hipError_t e = launch_active_mask(scores, n, keep, mask, workspace, workspace_bytes,
                                      (hipStream_t)stream);
    if (e == hipErrorNotSupported) return GS_ERR_UNSUPPORTED;
    return from_hip(e);
}

gs_status gs_active_mask_static(const float *scores, int64_t n, int64_t keep, uint8_t *mask, void *stream)
{
    if (n < 0 || n > INT32_MAX || keep < 0 || keep > n) return GS_ERR_INVALID_ARG;
    if (n > 0 && (!scores || !mask)) return GS_ERR_INVALID_ARG;
    if (n > GS_ACTIVE_MASK_STATIC_MAX_N) return GS_ERR_WORKSPACE;
    return from_hip(launch_active_mask_static(scores, n, keep, mask, (hipStream_t)stream));
}

size_t gs_active_mask_static_scratch_bytes(void) { return static_mask_scratch_bytes(); }

size_t gs_sh_q8_bounds_floats(int64_t n, int32_t rows)
{
    if (n < 0 || rows < 1) return 0;
    return (size_t)rows * (size_t)((n + 255) / 256) * 2;
}

gs_status gs_sh_quantize8(const float *sh, int64_t n, int32_t rows, uint8_t *codes, float *bounds, void *stream)
{
    if (n < 0 || n > INT32_MAX || rows < 1 || rows > 65535) return GS_ERR_INVALID_ARG;
    if (n > 0 && (!sh || !codes || !bounds)) return GS_ERR_INVALID_ARG;
    if (n == 0) return GS_OK;
    return from_hip(launch_sh_quantize8(sh, n, rows, codes, bounds, (hipStream_t)stream));
}

gs_status gs_sh_adam_step(const gs_sh_adam *a, void *stream)
{
    if (!a) return GS_ERR_INVALID_ARG;
    if (a->n < 0 || a->n > INT32_MAX || a->rows < 1 || a->rows > 65535) return GS_ERR_INVALID_ARG;
    if (a->value_dtype != GS_SH_F32 && a->value_dtype != GS_SH_F16) return GS_ERR_INVALID_ARG;
    if (a->state_dtype != GS_ADAM_F32 && a->state_dtype != GS_ADAM_Q8LOG) return GS_ERR_INVALID_ARG;
    if (a->update != GS_ADAM_DENSE && a->update != GS_ADAM_LAZY) return GS_ERR_INVALID_ARG;
    if (a->step < 1) return GS_ERR_INVALID_ARG;
    if (!std::isfinite(a->lr) || !(a->lr >= 0.0f)) return GS_ERR_INVALID_ARG;
    if (!(a->beta1 >= 0.0f && a->beta1 < 1.0f) || !(a->beta2 >= 0.0f && a->beta2 < 1.0f)) return GS_ERR_INVALID_ARG;
    if (!std::isfinite(a->eps) || !(a->eps > 0.0f)) return GS_ERR_INVALID_ARG;
    if (a->n > 0) {
        if (!a->grad || !a->value || !a->m || !a->v) return GS_ERR_INVALID_ARG;
        if (a->state_dtype == GS_ADAM_Q8LOG && (!a->m_bounds || !a->v_bounds)) return GS_ERR_INVALID_ARG;
    }
    if (a->n == 0) return GS_OK;
    return from_hip(launch_sh_adam(*a, (hipStream_t)stream));
}

}  // extern "C"
