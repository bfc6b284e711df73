/*
 * CPU oracle for the tiled 3D Gaussian-splatting rasterizer -- plain, slow,
 * obviously correct.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark are its only users.  It shares no code
 * with the HIP library.  The interface and the readings are described in
 * gs_oracle.h; build with  gcc -O2 -ffp-contract=off -fopenmp  (no fast-math,
 * no -march flags: every float operation must be one IEEE operation).
 */
#include "gs_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Camera centre c = -R^T t in fp64 (used for the colour's view direction).  */
static void camera_centre(const orc_cam *cam, double c[3])
{
    const double *m = cam->viewmat;
    for (int i = 0; i < 3; i++)
        c[i] = -(m[0 * 4 + i] * m[3] + m[1 * 4 + i] * m[7] + m[2 * 4 + i] * m[11]);
}

/* ------------------------------------------------------------------------ */
/* Real spherical harmonics up to degree 3 (SH colour as on the GlobalSplat
 * page's appearance head and the Spirula Studio page's SH3 colour).  Reading:
 * the real basis ordered l = 0..3, m = -l..l, with sign (-1)^|m| relative to
 * the textbook real basis (the convention common 3DGS coefficient files use).
 * Constants are the closed forms sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) times
 * the Legendre polynomial factors, written out below. */
void orc_sh_basis(const double *d, double *Y, double *dY)
{
    const double x = d[0], y = d[1], z = d[2];
    const double PI = 3.14159265358979323846;
    const double c0 = 0.5 * sqrt(1.0 / PI);
    const double c1 = sqrt(3.0 / (4.0 * PI));
    const double c2a = 0.5 * sqrt(15.0 / PI);      /* xy, yz, xz */
    const double c2b = 0.25 * sqrt(5.0 / PI);      /* 2z^2 - x^2 - y^2 */
    const double c2c = 0.25 * sqrt(15.0 / PI);     /* x^2 - y^2 */
    const double c3a = 0.25 * sqrt(35.0 / (2.0 * PI));   /* |m| = 3 */
    const double c3b = 0.5 * sqrt(105.0 / PI);           /* xyz */
    const double c3c = 0.25 * sqrt(21.0 / (2.0 * PI));   /* |m| = 1 */
    const double c3d = 0.25 * sqrt(7.0 / PI);            /* m = 0 */
    const double c3e = 0.25 * sqrt(105.0 / PI);          /* z (x^2 - y^2) */
    double g[16][3];
    memset(g, 0, sizeof g);

    Y[0] = c0;
    /* l = 1: m = -1, 0, 1 */
    Y[1] = -c1 * y;  g[1][1] = -c1;
    Y[2] = c1 * z;   g[2][2] = c1;
    Y[3] = -c1 * x;  g[3][0] = -c1;
    /* l = 2 */
    Y[4] = c2a * x * y;                       g[4][0] = c2a * y; g[4][1] = c2a * x;
    Y[5] = -c2a * y * z;                      g[5][1] = -c2a * z; g[5][2] = -c2a * y;
    Y[6] = c2b * (2.0 * z * z - x * x - y * y);
    g[6][0] = -2.0 * c2b * x; g[6][1] = -2.0 * c2b * y; g[6][2] = 4.0 * c2b * z;
    Y[7] = -c2a * x * z;                      g[7][0] = -c2a * z; g[7][2] = -c2a * x;
    Y[8] = c2c * (x * x - y * y);             g[8][0] = 2.0 * c2c * x; g[8][1] = -2.0 * c2c * y;
    /* l = 3 */
    Y[9] = -c3a * y * (3.0 * x * x - y * y);
    g[9][0] = -c3a * 6.0 * x * y; g[9][1] = -c3a * (3.0 * x * x - 3.0 * y * y);
    Y[10] = c3b * x * y * z;
    g[10][0] = c3b * y * z; g[10][1] = c3b * x * z; g[10][2] = c3b * x * y;
    Y[11] = -c3c * y * (4.0 * z * z - x * x - y * y);
    g[11][0] = -c3c * y * (-2.0 * x);
    g[11][1] = -c3c * (4.0 * z * z - x * x - 3.0 * y * y);
    g[11][2] = -c3c * y * (8.0 * z);
    Y[12] = c3d * z * (2.0 * z * z - 3.0 * x * x - 3.0 * y * y);
    g[12][0] = c3d * z * (-6.0 * x); g[12][1] = c3d * z * (-6.0 * y);
    g[12][2] = c3d * (6.0 * z * z - 3.0 * x * x - 3.0 * y * y);
    Y[13] = -c3c * x * (4.0 * z * z - x * x - y * y);
    g[13][0] = -c3c * (4.0 * z * z - 3.0 * x * x - y * y);
    g[13][1] = -c3c * x * (-2.0 * y);
    g[13][2] = -c3c * x * (8.0 * z);
    Y[14] = c3e * z * (x * x - y * y);
    g[14][0] = c3e * z * 2.0 * x; g[14][1] = -c3e * z * 2.0 * y; g[14][2] = c3e * (x * x - y * y);
    Y[15] = -c3a * x * (x * x - 3.0 * y * y);
    g[15][0] = -c3a * (3.0 * x * x - 3.0 * y * y); g[15][1] = -c3a * x * (-6.0 * y);
    if (dY) memcpy(dY, g, sizeof g);
}

/* ------------------------------------------------------------------------ */
/* Projection, two builds of one text.                                       */
#define REAL float
#define FN(name) name##_f32
#define SQRT sqrtf
#define CEIL ceilf
#define FLOOR floorf
#define FMIN fminf
#define FMAX fmaxf
#include "project_real.h"
#undef REAL
#undef FN
#undef SQRT
#undef CEIL
#undef FLOOR
#undef FMIN
#undef FMAX

#define REAL double
#define FN(name) name##_f64
#define SQRT sqrt
#define CEIL ceil
#define FLOOR floor
#define FMIN fmin
#define FMAX fmax
#include "project_real.h"
#undef REAL
#undef FN
#undef SQRT
#undef CEIL
#undef FLOOR
#undef FMIN
#undef FMAX

/* ------------------------------------------------------------------------ */
/* Binning.  Every Gaussian emits one entry per tile of its rectangle; the
 * per-tile lists are ordered by view depth with the lower index first among
 * equal depths (readings: camera-space z, not Euclidean distance; index
 * tiebreak).  Done by brute force: collect everything, qsort.
 * The reached-tile variant keeps an entry only when the Gaussian can reach
 * alpha >= (1/255)(1 - 1e-3) somewhere on the box of the tile's pixel
 * centres.  An entry it drops has alpha below 1/255 at every pixel of the
 * tile, where compositing skips it anyway, so images are those of the full
 * lists (a choice of this implementation: the pages do not say which tiles
 * a Gaussian is listed in). */
typedef struct { uint32_t tile; double z; uint32_t g; } bin_entry;

static int bin_cmp(const void *pa, const void *pb)
{
    const bin_entry *a = (const bin_entry *)pa, *b = (const bin_entry *)pb;
    if (a->tile != b->tile) return a->tile < b->tile ? -1 : 1;
    if (a->z != b->z) return a->z < b->z ? -1 : 1;
    if (a->g != b->g) return a->g < b->g ? -1 : 1;
    return 0;
}

/* Minimum of the convex quadratic Q(d) = a dx^2 + 2 b dx dy + c dy^2 over
 * the box [x0, x1] x [y0, y1]: 0 if the box holds d = 0, its unconstrained
 * minimiser; otherwise the minimum lies on the boundary, and along each edge
 * Q is a 1D convex quadratic whose minimum is at its vertex clamped to the
 * edge (vertex dy = -b dx / c on an edge of fixed dx, dx = -b dy / a on an
 * edge of fixed dy). */
static double box_min_q(double a, double b, double c, double x0, double x1, double y0, double y1)
{
    if (x0 <= 0.0 && 0.0 <= x1 && y0 <= 0.0 && 0.0 <= y1) return 0.0;
    double best = INFINITY;
    const double xe[2] = {x0, x1}, ye[2] = {y0, y1};
    for (int i = 0; i < 2; i++) {
        const double dx = xe[i];
        const double dy = fmin(fmax(-b * dx / c, y0), y1);
        best = fmin(best, a * dx * dx + 2.0 * b * dx * dy + c * dy * dy);
    }
    for (int i = 0; i < 2; i++) {
        const double dy = ye[i];
        const double dx = fmin(fmax(-b * dy / a, x0), x1);
        best = fmin(best, a * dx * dx + 2.0 * b * dx * dy + c * dy * dy);
    }
    return best;
}

/* Pixel centres of tile (tx, ty) are (16 tx + i + 1/2, 16 ty + j + 1/2),
 * i, j = 0..15; the box they span, relative to the mean. */
double orc_tile_reach(double u, double v, double a, double b, double c, double o, int tx, int ty)
{
    const double x0 = 16.0 * tx + 0.5 - u, y0 = 16.0 * ty + 0.5 - v;
    return o * exp(-0.5 * box_min_q(a, b, c, x0, x0 + 15.0, y0, y0 + 15.0));
}

/* Collects the pairs (every pair of each rectangle, or only those whose tile
 * the Gaussian reaches), sorts them and fills the outputs. */
static int64_t bin_pairs(int64_t n, const int32_t *rect, const double *z, const double *u, const double *v,
                         const double *conic, const double *opac, int tiles_x, int tiles_y, uint32_t *vals,
                         uint32_t *tile_of, uint32_t *ranges)
{
    int64_t K = 0;
    for (int64_t g = 0; g < n; g++)
        K += (int64_t)(rect[n + g] - rect[g]) * (rect[3 * n + g] - rect[2 * n + g]);
    bin_entry *e = (bin_entry *)malloc(sizeof(bin_entry) * (size_t)(K > 0 ? K : 1));
    const double reach_min = (1.0 / 255.0) * (1.0 - 1e-3);
    int64_t m = 0;
    for (int64_t g = 0; g < n; g++)
        for (int ty = rect[2 * n + g]; ty < rect[3 * n + g]; ty++)
            for (int tx = rect[g]; tx < rect[n + g]; tx++) {
                if (conic && !(orc_tile_reach(u[g], v[g], conic[g], conic[n + g], conic[2 * n + g], opac[g], tx,
                                              ty) >= reach_min))
                    continue;
                e[m].tile = (uint32_t)(ty * tiles_x + tx);
                e[m].z = z[g];
                e[m].g = (uint32_t)g;
                m++;
            }
    K = m;
    qsort(e, (size_t)K, sizeof(bin_entry), bin_cmp);
    const int64_t T = (int64_t)tiles_x * tiles_y;
    for (int64_t t = 0; t < 2 * T; t++) ranges[t] = 0;
    for (int64_t i = 0; i < K; i++) {
        vals[i] = e[i].g;
        tile_of[i] = e[i].tile;
        if (i == 0 || e[i - 1].tile != e[i].tile) ranges[2 * e[i].tile] = (uint32_t)i;
        if (i == K - 1 || e[i + 1].tile != e[i].tile) ranges[2 * e[i].tile + 1] = (uint32_t)(i + 1);
    }
    free(e);
    return K;
}

int64_t orc_bin(int64_t n, const int32_t *rect, const double *z, int tiles_x,
                int tiles_y, uint32_t *vals, uint32_t *tile_of, uint32_t *ranges)
{
    return bin_pairs(n, rect, z, NULL, NULL, NULL, NULL, tiles_x, tiles_y, vals, tile_of, ranges);
}

int64_t orc_bin_reach(int64_t n, const int32_t *rect, const double *z, const double *u, const double *v,
                      const double *conic, const double *opac, int tiles_x, int tiles_y, uint32_t *vals,
                      uint32_t *tile_of, uint32_t *ranges)
{
    return bin_pairs(n, rect, z, u, v, conic, opac, tiles_x, tiles_y, vals, tile_of, ranges);
}

/* ------------------------------------------------------------------------ */
/* Compositing of one pixel (fp64).  Readings:
 *   alpha = min(0.99, o exp(power)), power = -1/2 d^T conic d, d = mean - p,
 *     p = (i + 1/2, j + 1/2) the pixel centre;
 *   an entry with alpha < 1/255 is skipped (alpha == 1/255 composites);
 *   the stop test T < 1e-4 is made before each entry, so the entry that took
 *     T below 1e-4 was itself composited;
 *   image = sum alpha_i T_i rgb_i + T_final bg;
 *   n_contrib = 1 + list position of the last composited entry (0 if none).
 * A decision whose value lies within the relative band of its threshold is
 * an "event"; bit k of flips reverses the k-th event.  The stop test depends
 * on T alone, so its repeats while T is unchanged (entries skipped in
 * between) are one decision: one event, taken the same way each time. */
typedef struct {
    int n_comp;                 /* entries composited                     */
    int64_t evals;              /* entries examined before the stop       */
    int events;                 /* near-threshold alpha / stop decisions  */
    int capflag;                /* a composited alpha near the 0.99 cap   */
} pix_stats;

static void composite(const double *u, const double *v, const double *conic,
                      const double *opac, const double *rgb, int64_t n,
                      const uint32_t *vals, uint32_t start, uint32_t end,
                      const double *bg, const orc_bands *bands, double px,
                      double py, uint32_t flips, double out_c[3], double *out_T,
                      int32_t *out_n, pix_stats *st, double *weight)
{
    const double a_thr = 1.0 / 255.0, t_thr = 1e-4, cap = 0.99;
    double T = 1.0, C[3] = {0.0, 0.0, 0.0};
    int32_t last = 0;
    int ev = 0;
    int stop_held = 0, stop_value = 0;   /* the event decision for the current T */
    st->n_comp = 0; st->evals = 0; st->events = 0; st->capflag = 0;
    for (uint32_t m = start; m < end; m++) {
        int stop = T < t_thr;
        if (fabs(T - t_thr) <= bands->trans * t_thr) {
            if (!stop_held) {
                if ((flips >> ev) & 1u) stop = !stop;
                ev++;
                stop_held = 1;
                stop_value = stop;
            }
            stop = stop_value;
        }
        if (stop) break;
        st->evals++;
        const uint32_t g = vals[m];
        const double dx = u[g] - px, dy = v[g] - py;
        const double a = conic[g], b = conic[n + g], c = conic[2 * n + g];
        const double power = -0.5 * (a * dx * dx + c * dy * dy) - b * dx * dy;
        const double raw = opac[g] * exp(power);
        const double alpha = raw < cap ? raw : cap;
        int skip = alpha < a_thr;
        if (fabs(alpha - a_thr) <= bands->alpha * a_thr) {
            if ((flips >> ev) & 1u) skip = !skip;
            ev++;
        }
        if (skip) continue;
        if (fabs(raw - cap) <= bands->cap * cap) st->capflag = 1;
        for (int ch = 0; ch < 3; ch++) C[ch] += alpha * T * rgb[ch * n + g];
        if (weight) {
#pragma omp atomic
            weight[g] += alpha * T;
        }
        T = T * (1.0 - alpha);
        stop_held = 0;
        last = (int32_t)(m - start + 1);
        st->n_comp++;
    }
    for (int ch = 0; ch < 3; ch++) out_c[ch] = C[ch] + T * bg[ch];
    *out_T = T;
    *out_n = last;
    st->events = ev;
}

int64_t orc_render(const orc_cam *cam, const double *u, const double *v,
                   const double *conic, const double *opac, const double *rgb,
                   int64_t n, const uint32_t *vals, const uint32_t *ranges,
                   const double *bg, const uint8_t *tile_mask,
                   const orc_bands *bands, double *image, double *final_T,
                   int32_t *n_contrib, int32_t *events, uint8_t *capflag,
                   double *weight)
{
    const int W = cam->width, H = cam->height;
    const int TX = (W + 15) / 16, TY = (H + 15) / 16;
    const int64_t HW = (int64_t)H * W;
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : total)
    for (int t = 0; t < TX * TY; t++) {
        if (tile_mask && !tile_mask[t]) continue;
        const int tx = t % TX, ty = t / TX;
        for (int j = ty * 16; j < ty * 16 + 16 && j < H; j++)
            for (int i = tx * 16; i < tx * 16 + 16 && i < W; i++) {
                double c[3], T;
                int32_t nc;
                pix_stats st;
                composite(u, v, conic, opac, rgb, n, vals, ranges[2 * t],
                          ranges[2 * t + 1], bg, bands, i + 0.5, j + 0.5, 0u, c,
                          &T, &nc, &st, weight);
                const int64_t p = (int64_t)j * W + i;
                for (int ch = 0; ch < 3; ch++) image[ch * HW + p] = c[ch];
                final_T[p] = T;
                n_contrib[p] = nc;
                events[p] = st.events;
                capflag[p] = (uint8_t)st.capflag;
                total += st.evals;
            }
    }
    return total;
}

int orc_render_pixel(const orc_cam *cam, const double *u, const double *v,
                     const double *conic, const double *opac, const double *rgb,
                     int64_t n, const uint32_t *vals, const uint32_t *ranges,
                     const double *bg, const orc_bands *bands, int px, int py,
                     uint32_t flips, double *out_rgb, double *out_T,
                     int32_t *out_n)
{
    const int TX = (cam->width + 15) / 16;
    const int t = (py / 16) * TX + px / 16;
    pix_stats st;
    composite(u, v, conic, opac, rgb, n, vals, ranges[2 * t], ranges[2 * t + 1],
              bg, bands, px + 0.5, py + 0.5, flips, out_rgb, out_T, out_n, &st, NULL);
    return st.events;
}

/* ------------------------------------------------------------------------ */
/* Reverse pass through the compositing (fp64), every discrete decision held
 * as the forward took it.  For the composited entries i = 1..n of a pixel with
 * transmittance T_i before entry i, upstream G = dL/dC and final T_f:
 *   dL/drgb_i   = alpha_i T_i G
 *   dL/dalpha_i = T_i <rgb_i - S_i, G>,
 *       S_i = (sum_{j>i} alpha_j T_j rgb_j + T_f bg) / (T_i (1 - alpha_i))
 *   alpha = o exp(power) below the cap: dalpha/do = exp(power),
 *       dalpha/dpower = alpha; at the cap both are 0
 *   power = -1/2 (a dx^2 + c dy^2) - b dx dy, dx = u - px, dy = v - py. */
void orc_render_bwd(const orc_cam *cam, const double *u, const double *v,
                    const double *conic, const double *opac, const double *rgb,
                    int64_t n, const uint32_t *vals, const uint32_t *ranges,
                    const double *bg, const uint8_t *tile_mask,
                    const orc_bands *bands, const double *dL_dimage,
                    double *grad2d)
{
    const int W = cam->width, H = cam->height;
    const int TX = (W + 15) / 16, TY = (H + 15) / 16;
    const int64_t HW = (int64_t)H * W;
    const double a_thr = 1.0 / 255.0, t_thr = 1e-4, cap = 0.99;
    (void)bands;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < TX * TY; t++) {
        if (tile_mask && !tile_mask[t]) continue;
        const uint32_t start = ranges[2 * t], end = ranges[2 * t + 1];
        if (end <= start) continue;
        const int L = (int)(end - start);
        double *acc = (double *)calloc((size_t)L * 9, sizeof(double));
        int *idx = (int *)malloc(sizeof(int) * (size_t)L);
        double *al = (double *)malloc(sizeof(double) * (size_t)L);
        double *Ti = (double *)malloc(sizeof(double) * (size_t)L);
        double *Gv = (double *)malloc(sizeof(double) * (size_t)L);
        const int tx = t % TX, ty = t / TX;
        for (int j = ty * 16; j < ty * 16 + 16 && j < H; j++)
            for (int i = tx * 16; i < tx * 16 + 16 && i < W; i++) {
                const double px = i + 0.5, py = j + 0.5;
                const int64_t p = (int64_t)j * W + i;
                const double G[3] = {dL_dimage[p], dL_dimage[HW + p], dL_dimage[2 * HW + p]};
                /* forward again, recording the composited entries */
                double T = 1.0;
                int cnt = 0;
                for (uint32_t m = start; m < end; m++) {
                    if (T < t_thr) break;
                    const uint32_t g = vals[m];
                    const double dx = u[g] - px, dy = v[g] - py;
                    const double a = conic[g], b = conic[n + g], c = conic[2 * n + g];
                    const double power = -0.5 * (a * dx * dx + c * dy * dy) - b * dx * dy;
                    const double e = exp(power);
                    const double raw = opac[g] * e;
                    const double alpha = raw < cap ? raw : cap;
                    if (alpha < a_thr) continue;
                    idx[cnt] = (int)(m - start);
                    al[cnt] = alpha;
                    Ti[cnt] = T;
                    Gv[cnt] = e;
                    cnt++;
                    T = T * (1.0 - alpha);
                }
                const double Tf = T;
                /* suffix sums  sum_{j>i} alpha_j T_j rgb_j + T_f bg  */
                double suf[3] = {Tf * bg[0], Tf * bg[1], Tf * bg[2]};
                for (int k = cnt - 1; k >= 0; k--) {
                    const uint32_t g = vals[start + (uint32_t)idx[k]];
                    const double alpha = al[k], Tk = Ti[k];
                    const double Tnext = Tk * (1.0 - alpha);
                    double dl_dalpha = 0.0;
                    double *ac = acc + (size_t)idx[k] * 9;
                    for (int ch = 0; ch < 3; ch++) {
                        const double col = rgb[ch * n + g];
                        const double S = suf[ch] / Tnext;
                        dl_dalpha += Tk * (col - S) * G[ch];
                        ac[6 + ch] += alpha * Tk * G[ch];
                    }
                    for (int ch = 0; ch < 3; ch++) suf[ch] += alpha * Tk * rgb[ch * n + g];
                    const double raw = opac[g] * Gv[k];
                    if (raw < cap) {
                        const double dx = u[g] - px, dy = v[g] - py;
                        const double a = conic[g], b = conic[n + g], c = conic[2 * n + g];
                        const double dl_dpower = dl_dalpha * alpha;
                        ac[5] += dl_dalpha * Gv[k];                         /* opacity */
                        ac[0] += dl_dpower * (-(a * dx + b * dy));          /* u */
                        ac[1] += dl_dpower * (-(c * dy + b * dx));          /* v */
                        ac[2] += dl_dpower * (-0.5 * dx * dx);              /* conic a */
                        ac[3] += dl_dpower * (-dx * dy);                    /* conic b */
                        ac[4] += dl_dpower * (-0.5 * dy * dy);              /* conic c */
                    }
                }
            }
        for (int k = 0; k < L; k++) {
            const uint32_t g = vals[start + (uint32_t)k];
            for (int q = 0; q < 9; q++) {
                const double val = acc[(size_t)k * 9 + q];
                if (val != 0.0) {
#pragma omp atomic
                    grad2d[(int64_t)q * n + g] += val;
                }
            }
        }
        free(acc); free(idx); free(al); free(Ti); free(Gv);
    }
}

/* ------------------------------------------------------------------------ */
/* Chain rule from the 2D record gradients to the raw parameters (fp64).
 * The forward is recomputed in fp64 from the activated parameters; the
 * guard clamp and the colour clamp keep the branch the forward took.
 *   conic = Sigma'^-1:      dSigma' = -Q A Q, A = [[da, db/2], [db/2, dc]]
 *   Sigma2 = T Sigma T^T:   dSigma = T^T dSigma2 T,  dT = 2 dSigma2 T Sigma
 *   T = J W:                dJ = dT W^T
 *   Sigma = M M^T:          dM = 2 dSigma M;  ds_j = sum_i R_ij dM_ij;
 *                           dR = dM diag(s)
 *   q_hat = q / |q|:        dq = (I - q_hat q_hat^T) dq_hat / |q|
 *   colour:                 dk_j = Y_j(d) drgb (unclamped channels),
 *                           dmu += (I - d d^T) / |mu - c| sum k_j grad Y_j drgb
 *   raw outputs:            dlog s = s ds,  dlogit = o (1 - o) do. */
void orc_project_bwd(int64_t n, const double *means, const double *scales,
                     const double *quats, const double *opac, int sh_degree,
                     const double *sh, const orc_cam *cam,
                     const int32_t *radius, const uint8_t *clamped,
                     const double *grad2d, double *d_means,
                     double *d_log_scales, double *d_quats,
                     double *d_logits, double *d_sh)
{
    const int K = (sh_degree + 1) * (sh_degree + 1);
    const double *vm = cam->viewmat;
    double W[3][3], tt[3];
    for (int i = 0; i < 3; i++) {
        for (int j = 0; j < 3; j++) W[i][j] = vm[i * 4 + j];
        tt[i] = vm[i * 4 + 3];
    }
    double cc[3];
    camera_centre(cam, cc);
    const double fx = cam->fx, fy = cam->fy;
    const double lx = cam->guard * (0.5 * cam->width / fx);
    const double ly = cam->guard * (0.5 * cam->height / fy);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n; g++) {
        if (radius[g] == 0) continue;
        const double gu = grad2d[g], gv = grad2d[n + g];
        const double ga = grad2d[2 * n + g], gb = grad2d[3 * n + g], gc = grad2d[4 * n + g];
        const double go = grad2d[5 * n + g];
        const double grgb[3] = {grad2d[6 * n + g], grad2d[7 * n + g], grad2d[8 * n + g]};
        const double mu[3] = {means[g], means[n + g], means[2 * n + g]};
        const double s[3] = {scales[g], scales[n + g], scales[2 * n + g]};
        const double q[4] = {quats[g], quats[n + g], quats[2 * n + g], quats[3 * n + g]};

        /* forward, fp64 */
        double p[3];
        for (int i = 0; i < 3; i++) p[i] = W[i][0] * mu[0] + W[i][1] * mu[1] + W[i][2] * mu[2] + tt[i];
        const double x = p[0], y = p[1], z = p[2];
        const double qn = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
        const double w = q[0] / qn, a = q[1] / qn, b = q[2] / qn, c = q[3] / qn;
        double R[3][3] = {
            {1 - 2 * (b * b + c * c), 2 * (a * b - w * c), 2 * (a * c + w * b)},
            {2 * (a * b + w * c), 1 - 2 * (a * a + c * c), 2 * (b * c - w * a)},
            {2 * (a * c - w * b), 2 * (b * c + w * a), 1 - 2 * (a * a + b * b)}};
        double M[3][3], S[3][3];
        for (int i = 0; i < 3; i++)
            for (int j = 0; j < 3; j++) M[i][j] = R[i][j] * s[j];
        for (int i = 0; i < 3; i++)
            for (int j = 0; j < 3; j++)
                S[i][j] = M[i][0] * M[j][0] + M[i][1] * M[j][1] + M[i][2] * M[j][2];
        const double txr = x / z, tyr = y / z;
        const int clx = (txr < -lx) || (txr > lx);
        const int cly = (tyr < -ly) || (tyr > ly);
        const double xg = fmin(fmax(txr, -lx), lx) * z;
        const double yg = fmin(fmax(tyr, -ly), ly) * z;
        double J[2][3] = {{fx / z, 0.0, -fx * xg / (z * z)}, {0.0, fy / z, -fy * yg / (z * z)}};
        double Tm[2][3];
        for (int i = 0; i < 2; i++)
            for (int k = 0; k < 3; k++) Tm[i][k] = J[i][0] * W[0][k] + J[i][1] * W[1][k] + J[i][2] * W[2][k];
        double S2[2][2];
        for (int i = 0; i < 2; i++)
            for (int j = 0; j < 2; j++) {
                double acc = 0.0;
                for (int k = 0; k < 3; k++)
                    for (int l = 0; l < 3; l++) acc += Tm[i][k] * S[k][l] * Tm[j][l];
                S2[i][j] = acc;
            }
        const double P00 = S2[0][0] + 0.3, P01 = S2[0][1], P11 = S2[1][1] + 0.3;
        const double det = P00 * P11 - P01 * P01;
        const double Q[2][2] = {{P11 / det, -P01 / det}, {-P01 / det, P00 / det}};

        /* conic -> Sigma' -> Sigma2 */
        const double A[2][2] = {{ga, 0.5 * gb}, {0.5 * gb, gc}};
        double QA[2][2], dS2[2][2];
        for (int i = 0; i < 2; i++)
            for (int j = 0; j < 2; j++) QA[i][j] = Q[i][0] * A[0][j] + Q[i][1] * A[1][j];
        for (int i = 0; i < 2; i++)
            for (int j = 0; j < 2; j++) dS2[i][j] = -(QA[i][0] * Q[0][j] + QA[i][1] * Q[1][j]);

        /* Sigma2 = Tm Sigma Tm^T */
        double dS[3][3], dTm[2][3];
        for (int k = 0; k < 3; k++)
            for (int l = 0; l < 3; l++) {
                double acc = 0.0;
                for (int i = 0; i < 2; i++)
                    for (int j = 0; j < 2; j++) acc += Tm[i][k] * dS2[i][j] * Tm[j][l];
                dS[k][l] = acc;
            }
        for (int i = 0; i < 2; i++)
            for (int k = 0; k < 3; k++) {
                double acc = 0.0;
                for (int j = 0; j < 2; j++)
                    for (int l = 0; l < 3; l++) acc += dS2[i][j] * Tm[j][l] * S[l][k];
                dTm[i][k] = 2.0 * acc;
            }
        /* Tm = J W  ->  dJ = dTm W^T */
        double dJ[2][3];
        for (int i = 0; i < 2; i++)
            for (int j = 0; j < 3; j++) dJ[i][j] = dTm[i][0] * W[j][0] + dTm[i][1] * W[j][1] + dTm[i][2] * W[j][2];

        /* J(x, y, z) and (u, v)(x, y, z) */
        double dp[3] = {0.0, 0.0, 0.0};
        dp[0] += gu * fx / z;
        dp[1] += gv * fy / z;
        dp[2] += gu * (-fx * x / (z * z)) + gv * (-fy * y / (z * z));
        dp[2] += dJ[0][0] * (-fx / (z * z)) + dJ[1][1] * (-fy / (z * z));
        if (!clx) {       /* J02 = -fx x / z^2 */
            dp[0] += dJ[0][2] * (-fx / (z * z));
            dp[2] += dJ[0][2] * (2.0 * fx * x / (z * z * z));
        } else {          /* J02 = -fx (x/z clamped) / z */
            dp[2] += dJ[0][2] * (fx * (xg / z) / (z * z));
        }
        if (!cly) {
            dp[1] += dJ[1][2] * (-fy / (z * z));
            dp[2] += dJ[1][2] * (2.0 * fy * y / (z * z * z));
        } else {
            dp[2] += dJ[1][2] * (fy * (yg / z) / (z * z));
        }
        double dmu[3];
        for (int j = 0; j < 3; j++) dmu[j] = W[0][j] * dp[0] + W[1][j] * dp[1] + W[2][j] * dp[2];

        /* Sigma = M M^T */
        double dM[3][3], ds[3] = {0, 0, 0}, dR[3][3];
        for (int i = 0; i < 3; i++)
            for (int j = 0; j < 3; j++)
                dM[i][j] = 2.0 * (dS[i][0] * M[0][j] + dS[i][1] * M[1][j] + dS[i][2] * M[2][j]);
        for (int j = 0; j < 3; j++)
            for (int i = 0; i < 3; i++) ds[j] += R[i][j] * dM[i][j];
        for (int i = 0; i < 3; i++)
            for (int j = 0; j < 3; j++) dR[i][j] = dM[i][j] * s[j];
        /* rotation polynomial in (w, a, b, c) */
        double dqh[4];
        dqh[0] = 2.0 * (-c * dR[0][1] + b * dR[0][2] + c * dR[1][0] - a * dR[1][2] - b * dR[2][0] + a * dR[2][1]);
        dqh[1] = 2.0 * (b * dR[0][1] + c * dR[0][2] + b * dR[1][0] - w * dR[1][2] + c * dR[2][0] + w * dR[2][1])
                 - 4.0 * a * (dR[1][1] + dR[2][2]);
        dqh[2] = 2.0 * (a * dR[0][1] + w * dR[0][2] + a * dR[1][0] + c * dR[1][2] - w * dR[2][0] + c * dR[2][1])
                 - 4.0 * b * (dR[0][0] + dR[2][2]);
        dqh[3] = 2.0 * (-w * dR[0][1] + a * dR[0][2] + w * dR[1][0] + b * dR[1][2] + a * dR[2][0] + b * dR[2][1])
                 - 4.0 * c * (dR[0][0] + dR[1][1]);
        const double qh[4] = {w, a, b, c};
        const double dot = qh[0] * dqh[0] + qh[1] * dqh[1] + qh[2] * dqh[2] + qh[3] * dqh[3];

        /* colour */
        double d[3] = {mu[0] - cc[0], mu[1] - cc[1], mu[2] - cc[2]};
        const double dn = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
        for (int i = 0; i < 3; i++) d[i] /= dn;
        double Y[16], dY[48];
        orc_sh_basis(d, Y, dY);
        double dd[3] = {0, 0, 0};
        for (int ch = 0; ch < 3; ch++) {
            if ((clamped[g] >> ch) & 1u) continue;
            for (int j = 0; j < K; j++) {
                d_sh[((int64_t)j * 3 + ch) * n + g] += Y[j] * grgb[ch];
                const double kj = sh[((int64_t)j * 3 + ch) * n + g];
                for (int r = 0; r < 3; r++) dd[r] += kj * dY[j * 3 + r] * grgb[ch];
            }
        }
        const double ddot = d[0] * dd[0] + d[1] * dd[1] + d[2] * dd[2];
        for (int r = 0; r < 3; r++) dmu[r] += (dd[r] - d[r] * ddot) / dn;

        for (int r = 0; r < 3; r++) d_means[r * n + g] += dmu[r];
        for (int r = 0; r < 3; r++) d_log_scales[r * n + g] += s[r] * ds[r];
        for (int r = 0; r < 4; r++) d_quats[r * n + g] += (dqh[r] - qh[r] * dot) / qn;
        d_logits[g] += opac[g] * (1.0 - opac[g]) * go;
    }
}

/* ------------------------------------------------------------------------ */
/* Importance mask (BlitzGS page, section 2.3: skip Gaussians whose importance
 * weight is low).  Reading: one global mask keeping the k highest scores,
 * ties to the lower index. */
typedef struct { float s; int64_t g; } score_entry;

static int score_cmp(const void *pa, const void *pb)
{
    const score_entry *a = (const score_entry *)pa, *b = (const score_entry *)pb;
    if (a->s != b->s) return a->s > b->s ? -1 : 1;
    return a->g < b->g ? -1 : (a->g > b->g ? 1 : 0);
}

void orc_topk_mask(int64_t n, const float *scores, int64_t k, uint8_t *mask)
{
    score_entry *e = (score_entry *)malloc(sizeof(score_entry) * (size_t)(n > 0 ? n : 1));
    for (int64_t g = 0; g < n; g++) { e[g].s = scores[g]; e[g].g = g; mask[g] = 0; }
    qsort(e, (size_t)n, sizeof(score_entry), score_cmp);
    for (int64_t i = 0; i < k && i < n; i++) mask[e[i].g] = 1;
    free(e);
}

/* ------------------------------------------------------------------------ */
/* 8-bit block quantization of SH rows (see gs_oracle.h for the readings).   */
void orc_sh_quantize8(int64_t n, int rows, const float *x, uint8_t *q, float *bounds)
{
    const int64_t nb = (n + 255) / 256;
    for (int r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const int64_t g0 = b * 256, g1 = g0 + 256 < n ? g0 + 256 : n;
            const float *row = x + (int64_t)r * n;
            float lo = row[g0], hi = row[g0];
            for (int64_t g = g0 + 1; g < g1; g++) {
                if (row[g] < lo) lo = row[g];
                if (row[g] > hi) hi = row[g];
            }
            bounds[((int64_t)r * nb + b) * 2] = lo;
            bounds[((int64_t)r * nb + b) * 2 + 1] = hi;
            const float d = hi - lo;
            for (int64_t g = g0; g < g1; g++) {
                uint8_t c = 0;
                if (d > 0.0f) {
                    const float t = ((row[g] - lo) * 255.0f) / d;
                    const float f = floorf(t + 0.5f);
                    c = f >= 255.0f ? (uint8_t)255 : (uint8_t)f;
                }
                q[(int64_t)r * n + g] = c;
            }
        }
}

void orc_sh_dequantize8(int64_t n, int rows, const uint8_t *q, const float *bounds, float *x)
{
    const int64_t nb = (n + 255) / 256;
    for (int r = 0; r < rows; r++)
        for (int64_t g = 0; g < n; g++) {
            const float lo = bounds[((int64_t)r * nb + g / 256) * 2];
            const float hi = bounds[((int64_t)r * nb + g / 256) * 2 + 1];
            const float step = (hi - lo) * (1.0f / 255.0f);
            x[(int64_t)r * n + g] = lo + (float)q[(int64_t)r * n + g] * step;
        }
}

int orc_num_threads(void) { return omp_get_max_threads(); }

/* Threads for the OpenMP loops of the following calls (the CPU baseline
 * times the oracle on one core and on all of them). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
