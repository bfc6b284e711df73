/*
 * gs.h -- C ABI of the MI355X (gfx950) tiled 3D Gaussian-splatting rasterizer.
 *
 * One view is rendered by four calls on one stream:
 *   gs_project     per Gaussian: cull, EWA projection to a 2D conic, 3-sigma
 *                  tile rect, SH colour, depth -> one 48-byte splat record;
 *   gs_bin_sort    per (Gaussian, tile) pair: keys (tile << 32 | depth bits)
 *                  sorted with an LSB radix sort, index order among equal
 *                  keys; per-tile [start, end) ranges of the sorted list;
 *   gs_render_fwd  per pixel: front-to-back alpha compositing of its tile's
 *                  list;
 *   gs_render_bwd  reverse pass through the compositing and the projection:
 *                  gradients with respect to means, log-scales, quaternions,
 *                  opacity logits and SH coefficients (accumulated); also
 *                  available split as gs_render_bwd_screen per view and
 *                  gs_project_bwd over a batch of views.
 * gs_active_mask builds the optional importance mask that gs_project honours.
 *
 * Where the pages touch this path (they give no formulas):
 *   - Gaussians are projected onto the image plane over screen tiles and
 *     blended per pixel by alpha compositing -- VisionTech 4DGS page, section
 *     on its technical architecture and key mechanisms;
 *   - each Gaussian carries position, scale, rotation, opacity and SH colour
 *     -- GlobalSplat page, step (4) of its pipeline;
 *   - Gaussians are projected to screen tiles before anything is exchanged --
 *     BlitzGS page, section 2.1; the distance-LOD gate and importance mask
 *     that shrink the per-view active set -- BlitzGS page, section 2.3;
 *   - intermediate results cached in on-chip shared memory to cut global
 *     memory traffic; stages of the raster pipeline run as separate thread
 *     blocks -- "Gsplat" section of the pixel-diffusion page (sections 2.2
 *     and 3.2);
 *   - SH coefficients dominate the memory of a splat scene and may be stored
 *     in 16 bits while gradients stay fp32 -- Spirula Studio page, sections
 *     on the memory budget and the quantization switch.
 * The rules the pages leave open are fixed as follows: pinhole camera with
 * OpenCV axes; 0.3 px^2 low-pass dilation; radius ceil(3 sqrt(lambda_max));
 * 16x16 tiles; alpha = min(0.99, o exp(power)); entries with alpha < 1/255
 * are skipped; a pixel stops once its transmittance T < 1e-4 (tested before
 * each entry); image = sum alpha_i T_i rgb_i + T_final bg.
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned device memory on the current device;
 *     host pointers are named as such.  The library never allocates device
 *     memory: temporaries live in a caller workspace sized by the matching
 *     *_workspace_bytes query (gs_active_mask_static uses a fixed array of
 *     the library instead).
 *   - Splat arrays and workspaces must be 16-byte aligned (they are read with
 *     16-byte vector accesses); a misaligned one is GS_ERR_INVALID_ARG.  Every
 *     other array needs only the natural alignment of its element type.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; results are ready once the stream
 *     is synchronised.  Nothing is read back to the host, so a view's four
 *     calls can be enqueued back to back (and captured in a graph).
 *   - Argument errors are returned synchronously and nothing is enqueued.
 *     A failed kernel launch returns GS_ERR_HIP.
 *   - Calls on different streams may run concurrently if they use disjoint
 *     outputs and workspaces.  The library keeps no global mutable state
 *     apart from the fixed scratch array of gs_active_mask_static.
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gs_status {
    GS_OK = 0,
    GS_ERR_INVALID_ARG = 1,     /* a pointer, size or camera field is invalid */
    GS_ERR_UNSUPPORTED = 2,     /* e.g. SH degree above 3                      */
    GS_ERR_WORKSPACE = 3,       /* workspace smaller than the query returned   */
    GS_ERR_HIP = 4              /* a kernel launch failed                      */
} gs_status;

/* SH storage: fp32, fp16, or 8-bit codes with per-block bounds (see
 * gs_sh_quantize8); the kernels compute in fp32 whatever the storage. */
typedef enum gs_sh_dtype { GS_SH_F32 = 0, GS_SH_F16 = 1, GS_SH_Q8 = 2 } gs_sh_dtype;

/* Pinhole camera (host memory). */
typedef struct gs_camera {
    int32_t width, height;      /* image size in pixels, 1..32768 each        */
    float fx, fy, cx, cy;       /* focal lengths and principal point (px)      */
    float viewmat[12];          /* row-major 3x4 world->camera [R | t];
                                   camera axes x right, y down, z forward     */
    float znear;                /* Gaussians with camera z <= znear are culled
                                   (0.2 in every workload); must be >= 0, so
                                   that every kept depth is positive (the sort
                                   key is the bit pattern of the fp32 depth)   */
    float guard;                /* Jacobian taken at x/z, y/z clamped to guard
                                   x the half field of view (1.3)              */
    float lod_min_radius_px;    /* distance-LOD gate: cull when the undilated
                                   3-sigma radius 3 max(fx,fy) max(s) / |mu-c|
                                   is below this many pixels; 0 = off          */
    float time;                 /* the view's time tau: Gaussians with motion
                                   are drawn at mu + (tau - t_g) v (ignored
                                   when gs_gaussians.velocity is NULL)         */
} gs_camera;

/* The Gaussians (device memory, structure of arrays). */
typedef struct gs_gaussians {
    int64_t n;                  /* number of Gaussians, 0 .. 2^31-1            */
    int32_t sh_degree;          /* 0..3; K = (sh_degree+1)^2 coefficients      */
    int32_t sh_dtype;           /* gs_sh_dtype of `sh`                          */
    const float *means;         /* [3][n] world positions                      */
    const float *scales;        /* [3][n] activated scales (exp of log-scale)  */
    const float *quats;         /* [4][n] rotations (w, x, y, z), any norm > 0 */
    const float *opacities;     /* [n] activated opacities (sigmoid of logit)  */
    const void *sh;             /* [K][3][n] SH coefficients, band order
                                   l = 0..3, m = -l..l: float, half or uint8
                                   codes                                        */
    const uint8_t *active;      /* [n] per-Gaussian keep mask, or NULL = all   */
    const float *sh_bounds;     /* GS_SH_Q8 only: [K*3][ceil(n/256)][2] (lo, hi)
                                   of every 256-Gaussian block of an SH row     */
    const float *velocity;      /* [3][n] motion vectors v, or NULL: static     */
    const float *t_offset;      /* [n] time offsets t_g (required with velocity)*/
} gs_gaussians;

/* Motion (the VisionTech page's 4D Gaussian record: a time offset and a
 * motion vector per Gaussian).  With velocity set, every step of the path
 * sees Gaussian g in view c at the displaced mean
 *     dt = c.time - t_g,   mu'_i = mu_i + dt * v_i,
 * each an fp32 operation in that order (part of the op-order contract), and
 * a Gaussian whose displaced mean is not finite is culled in that view.  The
 * backward adds dL/dv = sum over views of dt dL/dmu' and dL/dt_g = -v . sum
 * over views of dL/dmu' to gs_grads.velocity and gs_grads.t_offset; dL/dmu
 * is dL/dmu'. */

/* 8-bit linear block quantization of SH storage (the Spirula Studio page's
 * description of its block-quantized tensors: 256 consecutive units share a
 * min/max pair and decode as min + (max - min) q / 255).
 * Input sh: float [rows][n] (rows = K * 3, the gs_gaussians layout); output
 * codes: uint8 [rows][n] and bounds: float [rows][ceil(n/256)][2], the
 * minimum and maximum of each block of 256 Gaussians of a row.  A value x
 * becomes q = min(255, floor(((x - lo) * 255) / (hi - lo) + 1/2)) (0 when
 * hi == lo) and is read back as lo + q * step with step = (hi - lo) *
 * fp32(1/255), each step one fp32 operation in that order.  Inputs must be
 * finite.
 * Errors: GS_ERR_INVALID_ARG (NULL pointers with n > 0, n < 0, rows < 1). */
size_t gs_sh_q8_bounds_floats(int64_t n, int32_t rows);
gs_status gs_sh_quantize8(const float *sh, int64_t n, int32_t rows, uint8_t *codes, float *bounds,
                          void *stream);

/* Fused SH Adam step (the Spirula Studio page's fused SH optimizer, with its
 * 16-bit SH values and 8-bit log-domain Adam state).  One launch updates the
 * SH values and both Adam moments of every unit (one SH coefficient of one
 * channel of one Gaussian) in place, from the fp32 SH gradients:
 *     m' = b1 m + (1 - b1) g,   v' = b2 v + (1 - b2) g^2,
 *     value' = value - lr (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps),
 * computed in fp32 from the fp32 hyper-parameters given (1 - b and the bias
 * corrections are formed from them in double precision), the new value
 * rounded to nearest into its storage type.  `update` picks which units
 * move: GS_ADAM_DENSE updates every unit (torch.optim.Adam's rule: a unit
 * with a zero gradient still decays its moments and moves by its first
 * moment); GS_ADAM_LAZY updates only units whose gradient is not exactly
 * zero, the others keeping their value and both moments (torch.optim.
 * SparseAdam's rule; t still counts every step).  The page names neither;
 * lazy is the usual choice with the 8-bit state: a first moment seldom
 * decodes to exactly 0, so a dense step moves every Gaussian no view saw,
 * by about lr x (code residue) / eps where its second moment decodes to 0
 * (far past fp16 range with eps = 1e-15).
 * State GS_ADAM_F32: m and v are float [rows][n].
 * State GS_ADAM_Q8LOG: m holds uint8 codes of the first moment and v uint8
 * codes of s = log1p(sqrt(v) / eps), each with bounds [rows][ceil(n/256)][2]
 * (lo, hi) per block of 256 Gaussians of a row, decoded lo + q * step with
 * step = (hi - lo) * fp32(1/255) as for GS_SH_Q8.  After the update each
 * block's bounds become the min and max of its new values and each code
 * min(255, floor((x - lo) * 255 / (hi - lo) + 1/2)) (0 when hi == lo).  A
 * fresh state is all codes 0 with bounds (0, 0).  The last block of a row
 * covers only the row's remaining n mod 256 Gaussians.
 * All arrays are device memory owned by the caller; value, m, v and the
 * bounds are read and overwritten, grad is only read and must not overlap
 * them.  Concurrent calls on overlapping arrays race. */
typedef enum gs_adam_state_dtype { GS_ADAM_F32 = 0, GS_ADAM_Q8LOG = 1 } gs_adam_state_dtype;
typedef enum gs_adam_update { GS_ADAM_DENSE = 0, GS_ADAM_LAZY = 1 } gs_adam_update;

typedef struct gs_sh_adam {
    int64_t n;                  /* Gaussians, 0 .. 2^31-1                      */
    int32_t rows;               /* SH rows, K * 3 for K coefficients, 1..65535 */
    int32_t value_dtype;        /* GS_SH_F32 or GS_SH_F16 of `value`           */
    int32_t state_dtype;        /* gs_adam_state_dtype of m and v              */
    int32_t step;               /* t >= 1: the number of this update           */
    float lr;                   /* learning rate >= 0                          */
    float beta1, beta2;         /* moment decays in [0, 1)                     */
    float eps;                  /* > 0: Adam's epsilon and the log scale       */
    int32_t update;             /* gs_adam_update: GS_ADAM_DENSE or _LAZY      */
    const float *grad;          /* [rows][n] fp32 SH gradients                 */
    void *value;                /* [rows][n] SH values, float or half          */
    void *m;                    /* [rows][n] float, or uint8 codes             */
    void *v;                    /* [rows][n] float, or uint8 codes of s        */
    float *m_bounds;            /* GS_ADAM_Q8LOG: [rows][ceil(n/256)][2]       */
    float *v_bounds;            /* GS_ADAM_Q8LOG: [rows][ceil(n/256)][2]       */
} gs_sh_adam;

/* Errors: GS_ERR_INVALID_ARG (NULL descriptor, NULL arrays with n > 0, n or
 * rows out of range, an unknown dtype or update mode, step < 1, lr < 0, a
 * decay outside [0, 1), eps <= 0, a non-finite hyper-parameter). */
gs_status gs_sh_adam_step(const gs_sh_adam *adam, void *stream);

/* One projected Gaussian (device memory, 48 bytes, 16-byte aligned).
 * A culled Gaussian has every field 0. */
typedef struct gs_splat {
    float u, v;                 /* image-plane mean (px); pixel (i, j) covers
                                   [i, i+1) x [j, j+1)                          */
    float depth;                /* camera-space z (> znear)                     */
    int32_t radius;             /* ceil(3 sqrt(lambda_max)) px, 0 = culled      */
    float conic_a, conic_b, conic_c;  /* inverse of the dilated 2D covariance:
                                   [[a, b], [b, c]]                            */
    float opacity;
    float r, g, b;              /* max(0, 0.5 + sum_j k_j Y_j(view direction)) */
    uint32_t tiles_touched;     /* tiles in the rect (0 = culled)               */
} gs_splat;

/* Gradients (device memory, fp32, structure of arrays, accumulated with +=
 * so a batch of views sums; the caller zeroes them once per batch). */
typedef struct gs_grads {
    float *means;               /* [3][n]                                       */
    float *log_scales;          /* [3][n]  d/d log-scale = s * d/ds             */
    float *quats;               /* [4][n]  through the normalisation            */
    float *opacity_logits;      /* [n]     d/d logit = o (1 - o) d/do           */
    float *sh;                  /* [K][3][n] always fp32, also for half SH      */
    float *velocity;            /* [3][n] with motion (required then), else
                                   unused                                       */
    float *t_offset;            /* [n]    with motion (required then)           */
} gs_grads;

/* ---------------------------------------------------------------------- */

/* Projection + SH colour of every Gaussian for one camera.
 * Writes splats[n].  Every value that decides a tile (u, v, depth, radius,
 * the rect) and the conic are computed in fp32 one correctly rounded
 * operation at a time in a fixed order, so they are reproducible bit for
 * bit by any IEEE fp32 implementation of the same sequence.
 * Errors: GS_ERR_INVALID_ARG for NULL pointers with n > 0, n < 0, a camera
 * with non-positive size or focal length; GS_ERR_UNSUPPORTED for
 * sh_degree outside 0..3 or an unknown sh_dtype. */
gs_status gs_project(const gs_gaussians *gaussians /* host struct */,
                     const gs_camera *camera /* host */, gs_splat *splats,
                     void *stream);

/* gs_project for n_views cameras (host array) in one pass over the
 * Gaussians: each Gaussian's parameters are read once for the batch (up to
 * 16 views per launch) and one record array is written per view (splats:
 * host array of n_views device pointers).  Same records as n_views
 * gs_project calls.
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_UNSUPPORTED. */
gs_status gs_project_views(const gs_gaussians *gaussians /* host struct */, int32_t n_views,
                           const gs_camera *cameras, gs_splat *const *splats, void *stream);

/* The sort's per-Gaussian inputs of one view, written by the projection
 * (gs_project_views_binned) so that gs_bin_sort_views need not read the
 * records back for them.  Device arrays of n entries each (depth_keys
 * 4-byte, tile_rects 8-byte aligned):
 *   depth_keys[n]   bits of the record's fp32 depth, 0xFFFFFFFF for a
 *                   Gaussian that touches no tile
 *   tile_rects[2n]  per Gaussian (x0 | y0 << 16, width | height << 16): its
 *                   tile rect, first tile and extent in tiles; (0, 0) for a
 *                   Gaussian that touches no tile
 * Owned by the caller.  Both describe the records of the same call and stay
 * valid only as long as those records are unchanged.  tile_rects may be NULL
 * for a view that is sorted with reach_tiles (that sort takes each rect from
 * the record it reads for the reach test). */
typedef struct gs_bin_keys {
    uint32_t *depth_keys;
    uint32_t *tile_rects;
} gs_bin_keys;

/* gs_project_views that also writes, for every view i whose bin_keys[i]
 * has depth_keys set, the sort inputs above (bin_keys: host array of
 * n_views entries; an entry with NULL pointers writes records only).  The
 * records are those of gs_project_views, except that in a view with
 * depth_keys the records of Gaussians outside the importance mask
 * (gs_gaussians.active) are left unwritten: gs_bin_sort_views given the
 * depth keys reads no record of an unlisted Gaussian, the blend reads listed
 * Gaussians only and gs_project_bwd skips Gaussians outside the mask (such
 * records must not be handed to gs_bin_sort without the depth keys).  Passing the arrays to
 * gs_bin_sort_views (gs_sort_view.depth_keys / tile_rects) spares the sort
 * its read of every record: one pass over the Gaussians produces both (the
 * projection of the VisionTech 4DGS page, section on technical architecture
 * and key mechanisms, ahead of the tile binning of the BlitzGS page,
 * section 2.1).
 * Errors: as gs_project_views; GS_ERR_INVALID_ARG for tile_rects without
 * depth_keys, a misaligned pointer, or a view whose tile grid has more than
 * 65535 tiles across or down. */
gs_status gs_project_views_binned(const gs_gaussians *gaussians /* host struct */, int32_t n_views,
                                  const gs_camera *cameras, gs_splat *const *splats,
                                  const gs_bin_keys *bin_keys /* host */, void *stream);

/* Workspace for gs_bin_sort, in bytes, for n Gaussians, a key capacity
 * k_capacity and the camera's tile count. */
size_t gs_bin_sort_workspace_bytes(int64_t n, int64_t k_capacity, int32_t n_tiles);

/* Number of 32-bit words of the tile schedule for a width x height image:
 * one per 16x16 tile plus four queue counters. */
size_t gs_schedule_words(int32_t width, int32_t height);

/* Number of 32-bit words of the backward index for n Gaussians and a key
 * capacity k_capacity (see gs_bin_sort). */
size_t gs_bwd_index_words(int64_t n, int64_t k_capacity);

/* Tile binning and depth sort of one view.
 * Input: splats[n] from gs_project with the same camera.
 * Output:
 *   vals[k_capacity]        Gaussian index of each sorted (tile, depth) entry
 *   tile_ranges[2*n_tiles]  [start, end) of each tile's entries in vals,
 *                           (0, 0) for an empty tile; tiles are row-major,
 *                           n_tiles = ceil(W/16) * ceil(H/16)
 *   schedule[gs_schedule_words(W, H)]  the tiles ordered longest list first
 *                           (the order in which the blend kernels take
 *                           them) and zeroed queue counters; pass it to
 *                           gs_render_fwd / gs_render_bwd
 *   bwd_index[gs_bwd_index_words(n, k_capacity)]  (optional, NULL to
 *                           skip; needed by gs_render_bwd) the duplication
 *                           slot of every sorted entry (k_capacity words),
 *                           the visible Gaussians in depth order (n words),
 *                           their first slots and K (n + 1 words), the number
 *                           of visible Gaussians (1 word); a Gaussian's
 *                           tiles_touched slots are contiguous
 *   keys[k_capacity]        (optional, NULL to skip) the 64-bit sort keys
 *                           tile << 32 | bits of the fp32 depth
 *   k_total                 device uint64: K, the number of entries
 * The order is that of a stable sort of the keys in emission order (Gaussian
 * index, then tile row-major), i.e. by (tile, depth, Gaussian index).
 * If K > k_capacity nothing is written past k_capacity, k_total still holds
 * the true K and vals / tile_ranges are undefined: the caller reads k_total
 * after synchronising and retries with a larger buffer.  k_capacity must be
 * below 2^32.
 * Errors: GS_ERR_INVALID_ARG (NULL pointers, bad sizes), GS_ERR_WORKSPACE. */
gs_status gs_bin_sort(const gs_splat *splats, int64_t n,
                      const gs_camera *camera /* host */, int64_t k_capacity,
                      uint32_t *vals, uint32_t *tile_ranges, uint32_t *schedule,
                      uint32_t *bwd_index, uint64_t *keys, uint64_t *k_total,
                      void *workspace, size_t workspace_bytes, void *stream);

/* One view's arguments of gs_bin_sort, for gs_bin_sort_views. */
typedef struct gs_sort_view {
    gs_camera camera;
    const gs_splat *splats;
    int64_t n;
    int64_t k_capacity;
    uint32_t *vals;
    uint32_t *tile_ranges;
    uint32_t *schedule;
    uint32_t *bwd_index;        /* optional */
    uint64_t *keys;             /* optional */
    uint64_t *k_total;
    void *workspace;            /* its own, gs_bin_sort_workspace_bytes */
    size_t workspace_bytes;
    /* optional: the view's gs_bin_keys from gs_project_views_binned for
     * these splats; the sort then takes each Gaussian's depth key and tile
     * rect from them instead of its record (same results).  tile_rects may
     * be NULL with depth_keys set when reach_tiles is nonzero. */
    const uint32_t *depth_keys;
    const uint32_t *tile_rects;
    /* nonzero: list a Gaussian only in the tiles of its rect that it reaches,
     * i.e. where o exp(-Q/2) >= (1/255)(1 - 1e-3) somewhere on the box of
     * the tile's pixel centres (Q the minimum over that box of the conic's
     * quadratic form: closed form, evaluated in fp64).  The pairs it leaves
     * out have alpha below 1/255 at every pixel of their tile, so the blend
     * skips them anyway: images, final_T and gradients equal those of the
     * full lists; K, vals, the ranges and n_contrib refer to the shorter
     * lists.  0: every tile of the rect. */
    int32_t reach_tiles;
} gs_sort_view;

/* gs_bin_sort for n_views views (host array) at once: the views go through
 * each step of the sort together, one launch per step for up to 8 views, so
 * views of a few million keys still fill the device.  Every view has its
 * own buffers and workspace; the results are those of n_views gs_bin_sort
 * calls.  Views may differ in size and resolution, and in whether they
 * bring gs_bin_keys.
 * Errors: as gs_bin_sort, checked for every view before anything runs;
 * GS_ERR_INVALID_ARG also for tile_rects without depth_keys, depth_keys
 * without tile_rects in a view without reach_tiles, or either misaligned. */
gs_status gs_bin_sort_views(int32_t n_views, const gs_sort_view *views /* host */,
                            void *stream);

/* Forward compositing of every pixel.
 * Inputs: splats (gs_project), vals, tile_ranges and schedule (gs_bin_sort),
 * bg: host float[3] background colour.
 * Outputs: image[3][H][W] (fp32, channel planes), final_T[H][W] (the
 * transmittance left after the pixel's last entry), n_contrib[H][W]
 * (1 + position in the tile's list of the last composited entry, 0 if
 * none).  final_T and n_contrib are what gs_render_bwd needs.
 * Tiles are processed by persistent waves in the schedule's order; the
 * result does not depend on it.  The call uses the schedule's forward queue
 * counters and leaves them reset, so calls sharing a schedule must be
 * ordered on one stream.  splats and vals must not be NULL, even for a view
 * with no visible Gaussian (pass buffers of at least one element).
 * Errors: GS_ERR_INVALID_ARG. */
gs_status gs_render_fwd(const gs_splat *splats, const uint32_t *vals,
                        const uint32_t *tile_ranges, uint32_t *schedule,
                        const gs_camera *camera, const float *bg /* host [3] */,
                        float *image, float *final_T, uint32_t *n_contrib,
                        void *stream);

/* One view's arguments of gs_render_fwd, for gs_render_fwd_views.
 * weight (optional, NULL to skip): float[n] indexed by Gaussian, to which
 * the call adds, for every Gaussian the view composites, the sum over the
 * view's pixels of its blending weight alpha_i T_i (the share of the pixel's
 * colour it supplies; summed over views, the per-Gaussian visibility weight
 * of the BlitzGS page's section 2.2).  Several views may share one array.
 * The additions are fp32 atomics in an unspecified order, so results agree
 * with a sequential sum to fp32 rounding. */
typedef struct gs_fwd_view {
    gs_camera camera;
    const gs_splat *splats;
    const uint32_t *vals;
    const uint32_t *tile_ranges;
    uint32_t *schedule;
    float *image;
    float *final_T;
    uint32_t *n_contrib;
    float *weight;
    /* nonzero when the lists come from gs_bin_sort_views with reach_tiles:
     * every entry passed the reach test there, so the blend skips its own
     * per-entry tile test (a hint: the results are the same either way) */
    int32_t reached_lists;
} gs_fwd_view;

/* gs_render_fwd of n_views views (host array) with one background colour,
 * up to 8 views per launch: the views' tiles form one work queue (each
 * view's longest tiles first, the views interleaved), so one view's last
 * long tiles overlap the others' work instead of idling the device.  The
 * outputs are those of n_views gs_render_fwd calls, plus the optional
 * blending weights.  A launch uses the forward queue counters of its first
 * view's schedule.  As for gs_render_fwd, no view's splats or vals may be
 * NULL.
 * Errors: GS_ERR_INVALID_ARG. */
gs_status gs_render_fwd_views(int32_t n_views, const gs_fwd_view *views,
                              const float *bg /* host [3] */, void *stream);

/* Workspace for gs_render_bwd, in bytes: nine fp32 partial sums per key
 * slot for a key capacity k_capacity, and nine fp32 sums per Gaussian. */
size_t gs_render_bwd_workspace_bytes(int64_t n, int64_t k_capacity);

/* Backward of one view: given dL/dimage[3][H][W], accumulates (+=) into
 * grads the gradient of L with respect to the raw parameters.  Every
 * discrete decision of the forward (tile membership, order, the 1/255 skip,
 * the stop, the 0.99 cap, the colour clamp at 0, the guard clamp) is held as
 * the forward took it; depth gets no gradient.  The inputs must be those of
 * the matching forward call, with bwd_index and the same k_capacity from
 * its gs_bin_sort.  Per (Gaussian, tile) the 9 screen-space gradients are
 * reduced across the tile's pixels on chip and stored at the pair's slot;
 * each Gaussian then sums its own slots.  No atomics are used: the result is
 * bit-reproducible.  It uses the schedule's backward queue counters (see
 * gs_render_fwd).
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_UNSUPPORTED, GS_ERR_WORKSPACE. */
gs_status gs_render_bwd(const gs_gaussians *gaussians /* host struct */,
                        const gs_camera *camera /* host */,
                        const gs_splat *splats, const uint32_t *vals,
                        const uint32_t *tile_ranges, uint32_t *schedule,
                        const uint32_t *bwd_index, int64_t k_capacity,
                        const float *bg /* host [3] */,
                        const float *final_T, const uint32_t *n_contrib,
                        const float *dL_dimage, const gs_grads *grads /* host struct */,
                        void *workspace, size_t workspace_bytes, void *stream);

/* The same backward split in two, for batches of views: the screen-space
 * part of one view (gs_render_bwd_screen) and the projection's chain rule of
 * several views in one pass over the Gaussians (gs_project_bwd), which reads
 * each Gaussian's parameters once per batch instead of once per view.
 * gs_render_bwd(view) = gs_render_bwd_screen(view) + gs_project_bwd({view}). */

/* Workspace for gs_render_bwd_screen, in bytes: nine fp32 partial sums per
 * key slot, for a key capacity k_capacity. */
size_t gs_render_bwd_screen_workspace_bytes(int64_t k_capacity);

/* Screen-space backward of one view (the reverse compositing pass of
 * gs_render_bwd and its per-Gaussian sum): writes g2[n][9] (device fp32,
 * one row of nine per Gaussian) for every Gaussian visible in the view;
 * rows of Gaussians culled in the view (radius 0) are left unwritten.  The
 * nine components are an internal representation that only gs_project_bwd
 * reads with the same view's records: the mean gradient and the 2D
 * covariance gradient in the principal frame of the record's conic, the
 * opacity gradient and the colour gradient.  Arguments as gs_render_bwd; n is
 * the number of Gaussians of the view's records.  Deterministic (no atomics).
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_WORKSPACE. */
gs_status gs_render_bwd_screen(const gs_camera *camera /* host */, int64_t n,
                               const gs_splat *splats, const uint32_t *vals,
                               const uint32_t *tile_ranges, uint32_t *schedule,
                               const uint32_t *bwd_index, int64_t k_capacity,
                               const float *bg /* host [3] */, const float *final_T,
                               const uint32_t *n_contrib, const float *dL_dimage,
                               float *g2, void *workspace, size_t workspace_bytes,
                               void *stream);

/* One view's arguments of gs_render_bwd_screen, for
 * gs_render_bwd_screen_views. */
typedef struct gs_bwd_view {
    gs_camera camera;
    int64_t n;
    const gs_splat *splats;
    const uint32_t *vals;
    const uint32_t *tile_ranges;
    uint32_t *schedule;
    const uint32_t *bwd_index;
    int64_t k_capacity;
    const float *final_T;
    const uint32_t *n_contrib;
    const float *dL_dimage;
    float *g2;
    void *workspace;
    size_t workspace_bytes;
    int32_t reached_lists;      /* as in gs_fwd_view */
} gs_bwd_view;

/* gs_render_bwd_screen of n_views views (host array) with one background
 * colour, up to 8 views per launch of the blend backward: as in
 * gs_render_fwd_views the views' tiles form one work queue.  Outputs as
 * n_views gs_render_bwd_screen calls.  A launch uses the backward queue
 * counters of its first view's schedule.
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_WORKSPACE. */
gs_status gs_render_bwd_screen_views(int32_t n_views, const gs_bwd_view *views,
                                     const float *bg /* host [3] */, void *stream);

/* Projection backward of n_views views (the chain rule of the EWA projection
 * and the SH colour, as in gs_render_bwd): grads += sum over the views of the
 * raw-parameter gradients, the views taken in order.
 *   cameras  host gs_camera[n_views]
 *   splats   host array of n_views device pointers: each view's records
 *   g2       host array of n_views device pointers: each view's g2[n][9]
 *            from gs_render_bwd_screen
 * Up to 16 views go into one launch; longer batches take several.
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_UNSUPPORTED. */
gs_status gs_project_bwd(const gs_gaussians *gaussians /* host struct */, int32_t n_views,
                         const gs_camera *cameras, const gs_splat *const *splats,
                         const float *const *g2, const gs_grads *grads /* host struct */,
                         void *stream);

/* gs_project_bwd for views projected by gs_project_views_binned: the same
 * gradients, with each view's visibility taken from the depth keys that call
 * wrote (a key other than 0xFFFFFFFF: visible) instead of from the record's
 * radius, so the colour part reads 4 bytes per Gaussian and view in place of
 * a line of records (the projection backward of the VisionTech 4DGS page,
 * section on technical architecture and key mechanisms).
 *   depth_keys  host array of n_views device pointers (4-byte aligned), each
 *               the gs_bin_keys.depth_keys of the same view and records, or
 *               NULL for a view whose visibility is read from its records
 * Errors: as gs_project_bwd; GS_ERR_INVALID_ARG for a NULL depth_keys array
 * (with n_views > 0) or a misaligned key pointer.  Keys that do not belong to
 * the records give unspecified gradients. */
gs_status gs_project_bwd_binned(const gs_gaussians *gaussians /* host struct */, int32_t n_views,
                                const gs_camera *cameras, const gs_splat *const *splats,
                                const float *const *g2, const uint32_t *const *depth_keys,
                                const gs_grads *grads /* host struct */, void *stream);

/* Workspace for gs_active_mask, in bytes. */
size_t gs_active_mask_workspace_bytes(int64_t n);

/* Importance mask of the BlitzGS page (section 2.3): mask[g] = 1 for the
 * `keep` Gaussians with the highest scores (ties, -0 and +0 included, to the
 * lower index), else 0; the result feeds gs_gaussians.active.
 *   scores  device float[n], finite (any sign; a NaN score gives a mask that
 *           is well defined but unspecified); any alignment
 *   n       0 .. INT32_MAX;  keep 0 .. n
 *   mask    device uint8[n], written in full; any alignment
 * Radix select on the device: four 8-bit histogram passes, then one pass
 * that writes the mask; no host synchronisation.
 * Errors: GS_ERR_INVALID_ARG, GS_ERR_WORKSPACE. */
gs_status gs_active_mask(const float *scores, int64_t n, int64_t keep,
                         uint8_t *mask, void *workspace, size_t workspace_bytes,
                         void *stream);

/* gs_active_mask for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same mask, bit for bit, computed with the library's own
 * fixed scratch array instead of a caller workspace.  The call allocates
 * nothing and needs no workspace; the caller still passes scores and mask.
 *   n  0 .. GS_ACTIVE_MASK_STATIC_MAX_N; larger n returns GS_ERR_WORKSPACE
 *      (the fixed array is too small) before anything is enqueued
 * The array (gs_active_mask_static_scratch_bytes() bytes, about 1 MiB) is a
 * static device variable: every GPU the library runs on holds its own copy
 * until the process ends, and its device address is looked up once per
 * device, on the first call made with that device current.  All calls on
 * one GPU share that GPU's copy, so calls that may overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give undefined masks; calls ordered on one stream are safe.  Each call
 * re-initialises whatever it reads, so nothing carries over between calls.
 * Errors: GS_ERR_INVALID_ARG (as gs_active_mask), GS_ERR_WORKSPACE (n above
 * the maximum), GS_ERR_HIP (no current device, the array's address could
 * not be found, or a launch failed). */
#define GS_ACTIVE_MASK_STATIC_MAX_N ((int64_t)1 << 30)
gs_status gs_active_mask_static(const float *scores, int64_t n, int64_t keep,
                                uint8_t *mask, void *stream);
size_t gs_active_mask_static_scratch_bytes(void);

/* Static description of a status code. */
const char *gs_status_string(gs_status status);

/* Library version, for the binding's load check. */
int32_t gs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
