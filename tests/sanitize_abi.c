/*
 * Driver for the sanitizer run of the C ABI's host code
 * (tests/test_sanitizers_cpu.py): every call of include/gs.h on arguments
 * the host rejects or sizes, none of which reaches a device, plus the size
 * queries over a range of shapes.  Built with the host code instrumented by
 * -fsanitize=address,undefined; any report fails the test.  Test
 * infrastructure only.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "gs.h"

#define EXPECT(expr, want)                                                                 \
    do {                                                                                  \
        const int got_ = (int)(expr);                                                     \
        if (got_ != (int)(want)) {                                                        \
            printf("FAIL %s:%d: %s = %d, expected %d\n", __FILE__, __LINE__, #expr, got_, \
                   (int)(want));                                                          \
            failures++;                                                                   \
        }                                                                                 \
    } while (0)

int main(void)
{
    int failures = 0;
    void *const dev = (void *)0x1000;     /* never dereferenced: every call below fails its checks first */
    for (int s = -1; s <= 6; s++) {
        const char *t = gs_status_string((gs_status)s);
        if (!t || !t[0]) failures++;
    }
    EXPECT(gs_version() >= 1, 1);

    /* size queries over shapes, including empty, ragged and the largest */
    size_t acc = 0;
    const int64_t ns[] = {-1, 0, 1, 255, 256, 257, 1000000, 2147483647LL};
    for (unsigned i = 0; i < sizeof ns / sizeof ns[0]; i++) {
        acc += gs_bin_sort_workspace_bytes(ns[i], ns[i] > 0 ? 4 * ns[i] : ns[i], 8160);
        acc += gs_render_bwd_workspace_bytes(ns[i], ns[i] > 0 ? 3 * ns[i] : 0);
        acc += gs_render_bwd_screen_workspace_bytes(ns[i]);
        acc += gs_active_mask_workspace_bytes(ns[i]);
        acc += gs_bwd_index_words(ns[i], ns[i] > 0 ? 2 * ns[i] : 0);
        acc += gs_sh_q8_bounds_floats(ns[i], 48);
    }
    const int32_t sizes[][2] = {{0, 0}, {1, 1}, {128, 128}, {1920, 1080}, {32768, 32768}, {32769, 1}};
    for (unsigned i = 0; i < sizeof sizes / sizeof sizes[0]; i++) acc += gs_schedule_words(sizes[i][0], sizes[i][1]);
    acc += gs_active_mask_static_scratch_bytes();

    gs_camera cam;
    memset(&cam, 0, sizeof cam);
    cam.width = 64; cam.height = 48; cam.fx = cam.fy = 50.0f; cam.cx = 32.0f; cam.cy = 24.0f;
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0f;
    cam.znear = 0.2f; cam.guard = 1.3f;
    gs_camera bad = cam;
    bad.znear = -0.5f;
    gs_camera nanc = cam;
    nanc.fx = NAN;

    gs_gaussians g;
    memset(&g, 0, sizeof g);
    g.n = 10; g.sh_degree = 3; g.sh_dtype = GS_SH_F32;
    g.means = g.scales = g.quats = g.opacities = (const float *)dev;
    g.sh = dev;
    EXPECT(gs_project(NULL, &cam, (gs_splat *)dev, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project(&g, &bad, (gs_splat *)dev, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project(&g, &nanc, (gs_splat *)dev, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project(&g, &cam, (gs_splat *)0x1004, NULL), GS_ERR_INVALID_ARG);    /* misaligned */
    g.sh_degree = 4;
    EXPECT(gs_project(&g, &cam, (gs_splat *)dev, NULL), GS_ERR_UNSUPPORTED);
    g.sh_degree = 3;
    g.velocity = (const float *)dev;                                                 /* without t_offset */
    EXPECT(gs_project(&g, &cam, (gs_splat *)dev, NULL), GS_ERR_INVALID_ARG);
    g.velocity = NULL;
    gs_splat *const splat_list[2] = {(gs_splat *)dev, NULL};
    EXPECT(gs_project_views(&g, 2, (const gs_camera[]){cam, cam}, splat_list, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project_views(&g, -1, NULL, NULL, NULL), GS_ERR_INVALID_ARG);
    gs_bin_keys bk[2];
    memset(bk, 0, sizeof bk);
    gs_splat *const splat_ok[2] = {(gs_splat *)dev, (gs_splat *)dev};
    EXPECT(gs_project_views_binned(&g, 2, (const gs_camera[]){cam, cam}, splat_ok, NULL, NULL), GS_ERR_INVALID_ARG);
    bk[1].tile_rects = (uint32_t *)dev;                                              /* rects without keys */
    EXPECT(gs_project_views_binned(&g, 2, (const gs_camera[]){cam, cam}, splat_ok, bk, NULL), GS_ERR_INVALID_ARG);
    bk[1].depth_keys = (uint32_t *)0x1002;                                           /* misaligned keys */
    EXPECT(gs_project_views_binned(&g, 2, (const gs_camera[]){cam, cam}, splat_ok, bk, NULL), GS_ERR_INVALID_ARG);
    bk[1].depth_keys = (uint32_t *)dev;
    bk[1].tile_rects = (uint32_t *)0x1004;                                           /* misaligned rects */
    EXPECT(gs_project_views_binned(&g, 2, (const gs_camera[]){cam, cam}, splat_ok, bk, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project_views_binned(&g, 2, (const gs_camera[]){cam, bad}, splat_ok, bk, NULL), GS_ERR_INVALID_ARG);
    gs_gaussians g0 = g;
    g0.n = 0;
    EXPECT(gs_project(&g0, &cam, NULL, NULL), GS_OK);                                /* nothing to do */

    uint32_t *u32 = (uint32_t *)dev;
    uint64_t *u64 = (uint64_t *)dev;
    EXPECT(gs_bin_sort((const gs_splat *)dev, -1, &cam, 16, u32, u32, u32, NULL, NULL, u64, dev, 1 << 20, NULL),
           GS_ERR_INVALID_ARG);
    EXPECT(gs_bin_sort((const gs_splat *)dev, 100, &cam, 400, u32, u32, u32, NULL, NULL, u64, dev, 16, NULL),
           GS_ERR_WORKSPACE);
    EXPECT(gs_bin_sort((const gs_splat *)dev, 100, &cam, (int64_t)1 << 33, u32, u32, u32, NULL, NULL, u64, dev,
                       1 << 20, NULL),
           GS_ERR_INVALID_ARG);
    gs_sort_view sv[2];
    memset(sv, 0, sizeof sv);
    EXPECT(gs_bin_sort_views(2, NULL, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_bin_sort_views(2, sv, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_bin_sort_views(0, NULL, NULL), GS_OK);
    sv[0].camera = cam;                                                              /* keys without rects, no reach */
    sv[0].tile_ranges = sv[0].schedule = u32;
    sv[0].k_total = u64;
    sv[0].workspace = dev;
    sv[0].workspace_bytes = (size_t)1 << 30;
    sv[0].depth_keys = u32;
    EXPECT(gs_bin_sort_views(1, sv, NULL), GS_ERR_INVALID_ARG);
    sv[0].depth_keys = NULL;

    const float bg[3] = {0.0f, 0.0f, 0.0f};
    const float bgnan[3] = {0.0f, NAN, 0.0f};
    float *f32 = (float *)dev;
    EXPECT(gs_render_fwd(NULL, u32, u32, u32, &cam, bg, f32, f32, u32, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_render_fwd((const gs_splat *)dev, NULL, u32, u32, &cam, bg, f32, f32, u32, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_render_fwd((const gs_splat *)dev, u32, u32, u32, &cam, bgnan, f32, f32, u32, NULL),
           GS_ERR_INVALID_ARG);
    gs_fwd_view fv[9];
    memset(fv, 0, sizeof fv);
    EXPECT(gs_render_fwd_views(9, fv, bg, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_render_fwd_views(0, NULL, bg, NULL), GS_OK);

    gs_grads gr;
    memset(&gr, 0, sizeof gr);
    EXPECT(gs_render_bwd(&g, &cam, (const gs_splat *)dev, u32, u32, u32, u32, 100, bg, f32, u32, f32, &gr, dev,
                         1 << 20, NULL),
           GS_ERR_INVALID_ARG);
    EXPECT(gs_render_bwd_screen(&cam, 10, (const gs_splat *)dev, u32, u32, u32, u32, 100, bg, f32, u32, f32, f32,
                                dev, 8, NULL),
           GS_ERR_WORKSPACE);
    gs_bwd_view bv[2];
    memset(bv, 0, sizeof bv);
    EXPECT(gs_render_bwd_screen_views(2, bv, bg, NULL), GS_ERR_INVALID_ARG);
    const gs_splat *const sp[1] = {(const gs_splat *)dev};
    const float *const g2[1] = {f32};
    EXPECT(gs_project_bwd(&g, 1, &cam, sp, g2, &gr, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project_bwd(&g, -3, &cam, sp, g2, &gr, NULL), GS_ERR_INVALID_ARG);
    const uint32_t *const dk_odd[1] = {(const uint32_t *)((char *)dev + 2)};
    EXPECT(gs_project_bwd_binned(&g, 1, &cam, sp, g2, NULL, &gr, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_project_bwd_binned(&g, 1, &cam, sp, g2, dk_odd, &gr, NULL), GS_ERR_INVALID_ARG);

    EXPECT(gs_active_mask((const float *)dev, 10, 11, (uint8_t *)dev, dev, 1 << 20, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_active_mask((const float *)dev, 1000, 10, (uint8_t *)dev, dev, 4, NULL), GS_ERR_WORKSPACE);
    EXPECT(gs_active_mask_static((const float *)dev, ((int64_t)1 << 30) + 1, 10, (uint8_t *)dev, NULL),
           GS_ERR_WORKSPACE);
    EXPECT(gs_active_mask_static(NULL, 10, 3, (uint8_t *)dev, NULL), GS_ERR_INVALID_ARG);

    EXPECT(gs_sh_quantize8(NULL, 10, 48, NULL, NULL, NULL), GS_ERR_INVALID_ARG);
    EXPECT(gs_sh_quantize8(NULL, 0, 48, NULL, NULL, NULL), GS_OK);
    gs_sh_adam ad;
    memset(&ad, 0, sizeof ad);
    ad.n = 100; ad.rows = 45; ad.value_dtype = GS_SH_F16; ad.state_dtype = GS_ADAM_Q8LOG; ad.step = 1;
    ad.lr = 1e-3f; ad.beta1 = 0.9f; ad.beta2 = 0.999f; ad.eps = 1e-15f; ad.update = GS_ADAM_LAZY;
    ad.grad = f32; ad.value = dev; ad.m = dev; ad.v = dev; ad.m_bounds = f32; ad.v_bounds = f32;
    gs_sh_adam a2 = ad;
    a2.update = 7;
    EXPECT(gs_sh_adam_step(&a2, NULL), GS_ERR_INVALID_ARG);
    a2 = ad;
    a2.beta2 = 1.0f;
    EXPECT(gs_sh_adam_step(&a2, NULL), GS_ERR_INVALID_ARG);
    a2 = ad;
    a2.n = 0;
    EXPECT(gs_sh_adam_step(&a2, NULL), GS_OK);
    EXPECT(gs_sh_adam_step(NULL, NULL), GS_ERR_INVALID_ARG);

    printf("abi host checks: %d failures (size checksum %zu)\n", failures, acc);
    return failures != 0;
}
