/*
 * CPU oracle for the tiled 3D Gaussian-splatting rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists to check the GPU library; only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, table or constant with the HIP path.
 *
 * What it computes, and where the pages touch it (they give no formulas):
 *   - Gaussians are projected to the image plane and blended per pixel by
 *     alpha compositing over screen tiles -- VisionTech 4DGS page, section on
 *     its technical architecture and key mechanisms;
 *   - each Gaussian carries a position, scale, rotation, opacity and SH
 *     colour -- GlobalSplat page, step (4) of its pipeline;
 *   - Gaussians are projected onto screen tiles before being routed to the
 *     tiles that use them -- BlitzGS page, section 2.1;
 *   - a per-view distance-LOD gate and an importance mask shrink the active
 *     set -- BlitzGS page, section 2.3.
 * The pages give no formulas, so the exact rules are readings: EWA projection
 * with a 0.3 px^2 dilation, 3-sigma radius, 16x16 tiles, key = tile<<32 |
 * depth bits with index tiebreak, alpha = min(0.99, o exp(power)), skip
 * alpha < 1/255, stop once T < 1e-4.  Each reading is restated beside the
 * code that takes it.
 *
 * Precision: every quantity that decides an integer (camera-space position,
 * image mean, covariance, conic, radius, tile rectangle, depth key, LOD gate)
 * is computed in IEEE fp32, one correctly rounded operation at a time, in the
 * written order (the op-order contract), so that tile lists can be compared
 * bit for bit.  Colour, compositing and all gradients are fp64.  A second
 * build of the projection in fp64 serves the finite-difference checks.
 */
#ifndef GS_ORACLE_H
#define GS_ORACLE_H

#include <stdint.h>

typedef struct orc_cam {
    int32_t width, height;
    double fx, fy, cx, cy;
    double viewmat[12];      /* row-major [R | t], world -> camera, OpenCV axes */
    double znear;            /* cull z <= znear */
    double guard;            /* Jacobian evaluated inside guard x half-FOV */
    double lod_px;           /* distance-LOD gate threshold in px; 0 = off */
} orc_cam;

/* Per-Gaussian projection outputs (arrays of length n, or [k][n]). */
typedef struct orc_proj_out {
    double *u, *v, *z;       /* image mean (px) and camera-space depth */
    int32_t *radius;         /* 0 when culled */
    int32_t *rect;           /* [4][n]: x0, x1, y0, y1 (half-open tile rect) */
    double *conic;           /* [3][n]: a, b, c of the inverse 2D covariance */
    double *opacity;         /* [n] */
    double *rgb;             /* [3][n] */
    int32_t *tiles;          /* tiles touched */
    uint8_t *clamped;        /* bit ch set when rgb channel ch was clamped at 0 */
    double *rgb_raw;         /* [3][n]: 0.5 + sum k_j Y_j before the clamp */
} orc_proj_out;

/* Projection + SH colour.  The _f32 variant takes float inputs and follows the
 * fp32 op-order contract; the _f64 variant takes double inputs and is the
 * smooth function the gradients are checked against. */
void orc_project_f32(int64_t n, const float *means, const float *scales,
                     const float *quats, const float *opac, int sh_degree,
                     const float *sh, const uint8_t *active, const orc_cam *cam,
                     orc_proj_out *out);
void orc_project_f64(int64_t n, const double *means, const double *scales,
                     const double *quats, const double *opac, int sh_degree,
                     const double *sh, const uint8_t *active, const orc_cam *cam,
                     orc_proj_out *out);

/* Binning: every (Gaussian, tile) pair of each rectangle, sorted by
 * (tile, depth, index).  Returns K.  vals[K] receives Gaussian indices,
 * tile_of[K] the tile ids, ranges[2*T] the [start, end) of each tile. */
int64_t orc_bin(int64_t n, const int32_t *rect, const double *z, int tiles_x,
                int tiles_y, uint32_t *vals, uint32_t *tile_of, uint32_t *ranges);

/* The largest opacity-scaled Gaussian value o exp(-Q_min / 2) over the box
 * spanned by the pixel centres of tile (tx, ty), Q_min the minimum there of
 * Q(d) = a dx^2 + 2 b dx dy + c dy^2, d = pixel centre - (u, v). */
double orc_tile_reach(double u, double v, double a, double b, double c, double o, int tx, int ty);

/* Binning restricted to reached tiles: as orc_bin, keeping the pair
 * (Gaussian, tile) of a rectangle only when orc_tile_reach of that tile is at
 * least (1/255)(1 - 1e-3).  u, v, opac[n], conic[3][n] as orc_proj_out.
 * vals / tile_of need room for every pair of the rectangles. */
int64_t orc_bin_reach(int64_t n, const int32_t *rect, const double *z, const double *u, const double *v,
                      const double *conic, const double *opac, int tiles_x, int tiles_y, uint32_t *vals,
                      uint32_t *tile_of, uint32_t *ranges);

/* Near-threshold bands (relative) used to flag decisions that fp32 arithmetic
 * may legitimately take the other way. */
typedef struct orc_bands { double alpha, trans, cap, clamp; } orc_bands;

/* Forward compositing of every pixel of the sampled tiles (tile_mask NULL =
 * all).  Outputs are [3][H][W], [H][W], [H][W]; events[H][W] counts the
 * near-threshold alpha-skip and stop decisions; capflag[H][W] marks pixels
 * whose composited set holds an alpha within the band of the 0.99 cap.
 * weight[n] (NULL to skip) receives += for every composited entry its
 * blending weight alpha_i T_i: the share of the pixel's colour that the
 * Gaussian supplies.  Summed over a view's pixels (and by the caller over
 * views) this is the per-Gaussian visibility weight that the BlitzGS page's
 * section 2.2 scores Gaussians by (reading: the page names a cross-view
 * visibility weight and gives no formula; the sum of blending weights is
 * the plainest one).
 * Returns the number of list entries examined (P_eval). */
int64_t orc_render(const orc_cam *cam, const double *u, const double *v,
                   const double *conic, const double *opac, const double *rgb,
                   int64_t n, const uint32_t *vals, const uint32_t *ranges,
                   const double *bg, const uint8_t *tile_mask,
                   const orc_bands *bands, double *image, double *final_T,
                   int32_t *n_contrib, int32_t *events, uint8_t *capflag,
                   double *weight);

/* One pixel with the k-th near-threshold decision (in encounter order) taken
 * the other way when bit k of flips is set. */
int orc_render_pixel(const orc_cam *cam, const double *u, const double *v,
                     const double *conic, const double *opac, const double *rgb,
                     int64_t n, const uint32_t *vals, const uint32_t *ranges,
                     const double *bg, const orc_bands *bands, int px, int py,
                     uint32_t flips, double *out_rgb, double *out_T,
                     int32_t *out_n);

/* Reverse pass through the compositing of the sampled tiles: per-Gaussian
 * gradients of L = sum(dL_dimage * image) with respect to the 2D record
 * quantities, grad2d[9][n] = du, dv, da, db, dc, dopacity, dr, dg, db
 * (accumulated with +=). */
void orc_render_bwd(const orc_cam *cam, const double *u, const double *v,
                    const double *conic, const double *opac, const double *rgb,
                    int64_t n, const uint32_t *vals, const uint32_t *ranges,
                    const double *bg, const uint8_t *tile_mask,
                    const orc_bands *bands, const double *dL_dimage,
                    double *grad2d);

/* Chain rule from grad2d to the raw parameters (fp64, += accumulation):
 * d means[3][n], d log-scales[3][n], d quats[4][n], d opacity logits[n],
 * d SH[K][3][n].  Inputs are the activated parameters. */
void orc_project_bwd(int64_t n, const double *means, const double *scales,
                     const double *quats, const double *opac, int sh_degree,
                     const double *sh, const orc_cam *cam,
                     const int32_t *radius, const uint8_t *clamped,
                     const double *grad2d, double *d_means,
                     double *d_log_scales, double *d_quats,
                     double *d_logits, double *d_sh);

/* Importance mask: keep the k highest scores, ties to the lower index. */
void orc_topk_mask(int64_t n, const float *scores, int64_t k, uint8_t *mask);

/* 8-bit linear block quantization of SH storage (the Spirula Studio page,
 * its section on what each bit width holds and its description of the
 * block-wise min/max bounds): the coefficients are rows [rows][n] (row =
 * coefficient x channel, n Gaussians); every block of 256 consecutive
 * Gaussians of a row shares one (lo, hi) pair, the block's minimum and
 * maximum, bounds[rows][ceil(n / 256)][2].  Readings (the page gives the
 * decode formula and the block size, not the rounding): a value x becomes
 *   q = min(255, floor(((x - lo) * 255) / (hi - lo) + 1/2)),  q = 0 if hi == lo,
 * and decodes to  lo + q * step,  step = (hi - lo) * fp32(1/255) (the page's
 * decode is one multiplication per value once the block's step is known),
 * every step one fp32 IEEE operation in that order. */
void orc_sh_quantize8(int64_t n, int rows, const float *x, uint8_t *q, float *bounds);
void orc_sh_dequantize8(int64_t n, int rows, const uint8_t *q, const float *bounds, float *x);

/* The number of OpenMP threads the oracle's parallel loops use. */
int orc_num_threads(void);
void orc_set_num_threads(int n);

/* Real spherical-harmonic basis (degree <= 3) at unit direction d, and its
 * gradient with respect to the three components of d. */
void orc_sh_basis(const double *d, double *Y /*[16]*/, double *dY /*[16][3]*/);

#endif
