/*
 * Driver for the sanitizer run of the CPU oracle (tests/test_sanitizers_cpu.py):
 * every entry point of oracle/gs_oracle.h on a small generated scene, on
 * degenerate inputs (no Gaussians, all culled, a tile mask, fp64 projection)
 * and on the 8-bit SH and importance-mask helpers.  Built with
 * -fsanitize=address,undefined; any report fails the test.  Test
 * infrastructure only.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gs_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static void *xcalloc(size_t n, size_t s)
{
    void *p = calloc(n ? n : 1, s);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

typedef struct {
    double *u, *v, *z, *conic, *opac, *rgb, *rgb_raw;
    int32_t *radius, *rect, *tiles;
    uint8_t *clamped;
} proj_bufs;

static void proj_alloc(proj_bufs *b, int64_t n)
{
    b->u = xcalloc(n, 8); b->v = xcalloc(n, 8); b->z = xcalloc(n, 8);
    b->conic = xcalloc(3 * n, 8); b->opac = xcalloc(n, 8); b->rgb = xcalloc(3 * n, 8);
    b->rgb_raw = xcalloc(3 * n, 8); b->radius = xcalloc(n, 4); b->rect = xcalloc(4 * n, 4);
    b->tiles = xcalloc(n, 4); b->clamped = xcalloc(n, 1);
}

static void proj_free(proj_bufs *b)
{
    free(b->u); free(b->v); free(b->z); free(b->conic); free(b->opac); free(b->rgb);
    free(b->rgb_raw); free(b->radius); free(b->rect); free(b->tiles); free(b->clamped);
}

static orc_proj_out proj_out(proj_bufs *b)
{
    orc_proj_out o = {b->u, b->v, b->z, b->radius, b->rect, b->conic, b->opac, b->rgb, b->tiles, b->clamped,
                      b->rgb_raw};
    return o;
}

static int run_scene(int64_t n, int W, int H, int deg, int all_culled, int use_mask)
{
    const int K = (deg + 1) * (deg + 1);
    float *means = xcalloc(3 * n, 4), *scales = xcalloc(3 * n, 4), *quats = xcalloc(4 * n, 4);
    float *opac = xcalloc(n, 4), *sh = xcalloc((size_t)K * 3 * n, 4);
    double *means64 = xcalloc(3 * n, 8), *scales64 = xcalloc(3 * n, 8), *quats64 = xcalloc(4 * n, 8);
    double *opac64 = xcalloc(n, 8), *sh64 = xcalloc((size_t)K * 3 * n, 8);
    uint8_t *active = xcalloc(n, 1);
    for (int64_t g = 0; g < n; g++) {
        means[g] = (float)(urand() * 2 - 1);
        means[n + g] = (float)(urand() * 2 - 1);
        means[2 * n + g] = all_culled ? -1.0f : (float)(1.5 + 3 * urand());
        for (int k = 0; k < 3; k++) scales[k * n + g] = (float)exp(-4.0 + 3.0 * urand());
        for (int k = 0; k < 4; k++) quats[k * n + g] = (float)(urand() - 0.5);
        opac[g] = (float)(0.02 + 0.97 * urand());
        for (int j = 0; j < K * 3; j++) sh[(int64_t)j * n + g] = (float)(j < 3 ? urand() : 0.4 * (urand() - 0.5));
        active[g] = (uint8_t)(urand() < 0.8);
    }
    for (int64_t i = 0; i < 3 * n; i++) { means64[i] = means[i]; scales64[i] = scales[i]; }
    for (int64_t i = 0; i < 4 * n; i++) quats64[i] = quats[i];
    for (int64_t i = 0; i < n; i++) opac64[i] = opac[i];
    for (int64_t i = 0; i < (int64_t)K * 3 * n; i++) sh64[i] = sh[i];

    orc_cam cam;
    memset(&cam, 0, sizeof cam);
    cam.width = W; cam.height = H; cam.fx = cam.fy = 0.8 * W; cam.cx = 0.5 * W; cam.cy = 0.5 * H;
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0;
    cam.znear = 0.2; cam.guard = 1.3; cam.lod_px = use_mask ? 0.5 : 0.0;

    proj_bufs pb, pb64;
    proj_alloc(&pb, n);
    proj_alloc(&pb64, n);
    orc_proj_out po = proj_out(&pb), po64 = proj_out(&pb64);
    orc_project_f32(n, means, scales, quats, opac, deg, sh, use_mask ? active : NULL, &cam, &po);
    orc_project_f64(n, means64, scales64, quats64, opac64, deg, sh64, NULL, &cam, &po64);

    const int TX = (W + 15) / 16, TY = (H + 15) / 16, T = TX * TY;
    int64_t Kk = 0;
    for (int64_t g = 0; g < n; g++) Kk += pb.tiles[g];
    uint32_t *vals = xcalloc(Kk, 4), *tile_of = xcalloc(Kk, 4), *ranges = xcalloc(2 * T, 4);
    const int64_t K2 = orc_bin(n, pb.rect, pb.z, TX, TY, vals, tile_of, ranges);
    if (K2 != Kk) {
        fprintf(stderr, "K mismatch %lld %lld\n", (long long)K2, (long long)Kk);
        return 1;
    }

    const int64_t HW = (int64_t)W * H;
    double *image = xcalloc(3 * HW, 8), *final_T = xcalloc(HW, 8), *weight = xcalloc(n, 8);
    int32_t *n_contrib = xcalloc(HW, 4), *events = xcalloc(HW, 4);
    uint8_t *capflag = xcalloc(HW, 1), *tile_mask = xcalloc(T, 1);
    for (int t = 0; t < T; t++) tile_mask[t] = (uint8_t)(t % 3 != 1);
    const double bg[3] = {0.1, 0.2, 0.3};
    orc_bands bands = {3e-5, 2e-3, 3e-5, 1e-6};
    orc_render(&cam, pb.u, pb.v, pb.conic, pb.opac, pb.rgb, n, vals, ranges, bg, NULL, &bands, image, final_T,
               n_contrib, events, capflag, weight);
    orc_render(&cam, pb.u, pb.v, pb.conic, pb.opac, pb.rgb, n, vals, ranges, bg, tile_mask, &bands, image,
               final_T, n_contrib, events, capflag, NULL);
    double px_rgb[3], px_T;
    int32_t px_n;
    for (int k = 0; k < 8; k++)
        orc_render_pixel(&cam, pb.u, pb.v, pb.conic, pb.opac, pb.rgb, n, vals, ranges, bg, &bands,
                         (int)(urand() * W), (int)(urand() * H), (uint32_t)k, px_rgb, &px_T, &px_n);

    double *dL = xcalloc(3 * HW, 8), *grad2d = xcalloc(9 * n, 8);
    for (int64_t i = 0; i < 3 * HW; i++) dL[i] = urand() - 0.5;
    orc_render_bwd(&cam, pb64.u, pb64.v, pb64.conic, pb64.opac, pb64.rgb, n, vals, ranges, bg, NULL, &bands, dL,
                   grad2d);
    orc_render_bwd(&cam, pb64.u, pb64.v, pb64.conic, pb64.opac, pb64.rgb, n, vals, ranges, bg, tile_mask,
                   &bands, dL, grad2d);
    double *dm = xcalloc(3 * n, 8), *ds = xcalloc(3 * n, 8), *dq = xcalloc(4 * n, 8), *dlo = xcalloc(n, 8);
    double *dsh = xcalloc((size_t)K * 3 * n, 8);
    orc_project_bwd(n, means64, scales64, quats64, opac64, deg, sh64, &cam, pb.radius, pb.clamped, grad2d, dm, ds,
                    dq, dlo, dsh);

    float *scores = xcalloc(n, 4);
    uint8_t *mask = xcalloc(n, 1);
    for (int64_t g = 0; g < n; g++) scores[g] = (float)floor(urand() * 7);
    orc_topk_mask(n, scores, n / 3, mask);
    orc_topk_mask(n, scores, n, mask);
    orc_topk_mask(n, scores, 0, mask);

    const int64_t nb = (n + 255) / 256;
    uint8_t *codes = xcalloc((size_t)K * 3 * n, 1);
    float *bounds = xcalloc((size_t)K * 3 * nb * 2, 4), *dec = xcalloc((size_t)K * 3 * n, 4);
    orc_sh_quantize8(n, K * 3, sh, codes, bounds);
    orc_sh_dequantize8(n, K * 3, codes, bounds, dec);

    double d[3] = {0.3, -0.4, 0.866}, Y[16], dY[48];
    orc_sh_basis(d, Y, dY);

    double chk = 0.0;
    for (int64_t i = 0; i < 3 * HW; i++) chk += image[i];
    for (int64_t i = 0; i < 3 * n; i++) chk += dm[i];
    for (int64_t i = 0; i < (int64_t)K * 3 * n; i++) chk += dsh[i] + dec[i];
    for (int64_t i = 0; i < n; i++) chk += weight[i] + mask[i];
    printf("scene n=%lld %dx%d deg=%d culled=%d mask=%d K=%lld check=%.6g\n", (long long)n, W, H, deg, all_culled,
           use_mask, (long long)Kk, chk);

    free(means); free(scales); free(quats); free(opac); free(sh);
    free(means64); free(scales64); free(quats64); free(opac64); free(sh64); free(active);
    proj_free(&pb); proj_free(&pb64);
    free(vals); free(tile_of); free(ranges); free(image); free(final_T); free(weight); free(n_contrib);
    free(events); free(capflag); free(tile_mask); free(dL); free(grad2d); free(dm); free(ds); free(dq); free(dlo);
    free(dsh); free(scores); free(mask); free(codes); free(bounds); free(dec);
    return 0;
}

int main(void)
{
    orc_set_num_threads(2);
    int bad = 0;
    bad |= run_scene(300, 64, 48, 3, 0, 0);
    bad |= run_scene(257, 40, 33, 1, 0, 1);   /* ragged tiles, LOD gate and an active mask */
    bad |= run_scene(1, 16, 16, 0, 0, 0);
    bad |= run_scene(50, 32, 32, 2, 1, 0);    /* every Gaussian behind the camera: K = 0 */
    bad |= run_scene(0, 8, 8, 0, 0, 0);       /* no Gaussians */
    printf("num_threads %d\n", orc_num_threads());
    return bad;
}
