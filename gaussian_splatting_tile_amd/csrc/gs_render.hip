// Per-pixel alpha compositing, forward and backward (gfx950).
//
// One 256-lane block (four wave64) per 16x16 tile, one lane per pixel.  The
// tile's depth-sorted list is consumed in batches of 256 records: the block
// gathers the batch into LDS once (the on-chip caching of intermediate
// results that the "Gsplat" section of the pixel-diffusion page prescribes),
// then every lane walks it from LDS.  Compositing is VALU-bound: per
// (pixel, Gaussian) pair it costs ~17 fp32 VALU operations and one v_exp_f32.
//
// Rules (readings; the pages name tiled alpha blending but give no formula):
//   alpha = min(0.99, o exp(-1/2 d^T conic d)),  d = mean - pixel centre
//   an entry with alpha < 1/255 is skipped;
//   a pixel stops at the first entry it meets with T < 1e-4 (the entry that
//   took T below 1e-4 was composited);
//   C = sum alpha_i T_i rgb_i,  image = C + T_final bg.
//
// The forward and the backward evaluate alpha with the same function below
// (contraction off, explicit fma, v_exp_f32), so the backward retraces the
// forward's skip decisions exactly.
#include "gs_internal.h"

namespace gsi {
namespace {

constexpr int kBatch = kBlock;               // records staged per batch
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTMin = 1e-4f;

// Block index -> tile, so that each XCD (blocks are dealt to the 8 XCDs
// round robin) walks a contiguous band of tiles: neighbouring tiles share
// most of their Gaussians, and the band's records then stay in one L2.
__device__ __forceinline__ int tile_of_block(int n_tiles)
{
    const int per_xcd = (n_tiles + 7) / 8;
    return (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

struct Staged {
    float4 uvo;    // u, v, opacity, -
    float4 q;      // -a/2 log2e, -b log2e, -c/2 log2e, -   (exp2 form of the conic)
    float4 rgb;    // r, g, b, -
};

__device__ __forceinline__ Staged stage(const Splat &s)
{
    Staged t;
    t.uvo = make_float4(s.a.x, s.a.y, s.b.w, 0.0f);
    t.q = make_float4(-0.5f * kLog2e * s.b.x, -kLog2e * s.b.y, -0.5f * kLog2e * s.b.z, 0.0f);
    t.rgb = make_float4(s.c.x, s.c.y, s.c.z, 0.0f);
    return t;
}

// exp(power) at the pixel, in the exp2 form: exp2(a' dx^2 + b' dx dy + c' dy^2).
__device__ __forceinline__ float gauss_at(const float4 &uvo, const float4 &q, float px, float py,
                                          float &dx, float &dy)
{
#pragma clang fp contract(off)
    dx = uvo.x - px;
    dy = uvo.y - py;
    const float t = fmaf(q.y, dy, q.x * dx);       // a' dx + b' dy
    const float e = fmaf(q.z * dy, dy, t * dx);    // a' dx^2 + b' dx dy + c' dy^2
    return __builtin_amdgcn_exp2f(e);
}

__global__ __launch_bounds__(kBlock) void render_fwd_kernel(
    const Splat *__restrict__ splats, const uint32_t *__restrict__ vals,
    const uint32_t *__restrict__ ranges, Cam cam, float bg0, float bg1, float bg2,
    float *__restrict__ image, float *__restrict__ final_T, uint32_t *__restrict__ n_contrib)
{
    __shared__ float4 s_uvo[kBatch];
    __shared__ float4 s_q[kBatch];
    __shared__ float4 s_rgb[kBatch];

    const int n_tiles = cam.tiles_x * cam.tiles_y;
    const int tile = tile_of_block(n_tiles);
    if (tile >= n_tiles) return;
    const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
    const int i = tx * kTile + (threadIdx.x & (kTile - 1));
    const int j = ty * kTile + (threadIdx.x >> 4);
    const bool inside = i < cam.width && j < cam.height;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;

    const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
    float T = 1.0f, c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
    uint32_t last = 0;
    bool done = !inside;

    for (uint32_t b0 = start; b0 < end; b0 += kBatch) {
        if (__syncthreads_and(done)) break;
        const uint32_t m = b0 + threadIdx.x;
        if (m < end) {
            const Staged st = stage(splats[vals[m]]);
            s_uvo[threadIdx.x] = st.uvo;
            s_q[threadIdx.x] = st.q;
            s_rgb[threadIdx.x] = st.rgb;
        }
        __syncthreads();
        const int nb = (int)min((uint32_t)kBatch, end - b0);
        if (!__all(done)) {
            for (int k = 0; k < nb; k++) {
                float dx, dy;
                const float4 uvo = s_uvo[k];
                const float raw = uvo.z * gauss_at(uvo, s_q[k], px, py, dx, dy);
                const float alpha = fminf(kAlphaMax, raw);
                const bool take = !done && alpha >= kAlphaMin;
                const float w = take ? alpha * T : 0.0f;
                const float4 col = s_rgb[k];
                c0 = fmaf(col.x, w, c0);
                c1 = fmaf(col.y, w, c1);
                c2 = fmaf(col.z, w, c2);
                T = T - w;
                last = take ? (b0 - start) + (uint32_t)k + 1u : last;
                done = done || T < kTMin;
                if ((k & 15) == 15 && __all(done)) break;
            }
        }
        __syncthreads();
    }
    if (inside) {
        const size_t hw = (size_t)cam.width * cam.height;
        const size_t p = (size_t)j * cam.width + i;
        image[p] = c0 + T * bg0;
        image[hw + p] = c1 + T * bg1;
        image[2 * hw + p] = c2 + T * bg2;
        final_T[p] = T;
        n_contrib[p] = last;
    }
}

// ---------------------------------------------------------------------------
// Backward.  Per pixel, walk the composited entries back to front:
//   T_i = T_{i+1} / (1 - alpha_i)                (T before entry i)
//   A   = colour of everything behind entry i, normalised by T_{i+1}
//         (A starts at bg and A <- alpha_i rgb_i + (1 - alpha_i) A)
//   dL/drgb_i   = alpha_i T_i G
//   dL/dalpha_i = T_i <rgb_i - A, G>
//   below the cap: dL/do = exp(power) dL/dalpha, dL/dpower = alpha dL/dalpha
//   power = -1/2 (a dx^2 + c dy^2) - b dx dy (dx = u - px):
//     d/du = -(a dx + b dy), d/dv = -(c dy + b dx),
//     d/da = -dx^2/2, d/db = -dx dy, d/dc = -dy^2/2.
// The 9 per-pixel values of an entry are summed over the wave with cross-lane
// moves, over the block's waves in LDS, then added to grad2d[9][n] with one
// atomic per value per (Gaussian, tile).

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__global__ __launch_bounds__(kBlock) void render_bwd_kernel(
    const Splat *__restrict__ splats, const uint32_t *__restrict__ vals,
    const uint32_t *__restrict__ ranges, Cam cam, float bg0, float bg1, float bg2,
    const float *__restrict__ final_T, const uint32_t *__restrict__ n_contrib,
    const float *__restrict__ dL_dimage, int n, float *__restrict__ grad2d)
{
    __shared__ float4 s_uvo[kBatch];
    __shared__ float4 s_q[kBatch];
    __shared__ float4 s_rgb[kBatch];
    __shared__ float4 s_conic[kBatch];
    __shared__ uint32_t s_g[kBatch];
    __shared__ float s_acc[9][kBatch];
    __shared__ uint32_t s_max;

    const int n_tiles = cam.tiles_x * cam.tiles_y;
    const int tile = tile_of_block(n_tiles);
    if (tile >= n_tiles) return;
    const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
    const int i = tx * kTile + (threadIdx.x & (kTile - 1));
    const int j = ty * kTile + (threadIdx.x >> 4);
    const bool inside = i < cam.width && j < cam.height;
    const float px = (float)i + 0.5f, py = (float)j + 0.5f;
    const int lane = threadIdx.x & 63;

    const uint32_t start = ranges[2 * tile];
    float T = 1.0f, G0 = 0.0f, G1 = 0.0f, G2 = 0.0f;
    uint32_t last = 0;
    if (inside) {
        const size_t hw = (size_t)cam.width * cam.height;
        const size_t p = (size_t)j * cam.width + i;
        T = final_T[p];
        last = n_contrib[p];
        G0 = dL_dimage[p];
        G1 = dL_dimage[hw + p];
        G2 = dL_dimage[2 * hw + p];
    }
    float A0 = bg0, A1 = bg1, A2 = bg2;

    if (threadIdx.x == 0) s_max = 0;
    __syncthreads();
    atomicMax(&s_max, last);
    __syncthreads();
    const uint32_t stop = start + s_max;      // entries at or past this are unused

    for (int64_t bend = (int64_t)stop; bend > (int64_t)start; bend -= kBatch) {
        const uint32_t bbeg = (uint32_t)max((int64_t)start, bend - kBatch);
        const int nb = (int)(bend - bbeg);
        if ((int)threadIdx.x < nb) {
            const uint32_t g = vals[bbeg + threadIdx.x];
            const Splat s = splats[g];
            const Staged st = stage(s);
            s_uvo[threadIdx.x] = st.uvo;
            s_q[threadIdx.x] = st.q;
            s_rgb[threadIdx.x] = st.rgb;
            s_conic[threadIdx.x] = s.b;
            s_g[threadIdx.x] = g;
        }
        for (int q = threadIdx.x; q < 9 * kBatch; q += kBlock) (&s_acc[0][0])[q] = 0.0f;
        __syncthreads();
        for (int k = nb - 1; k >= 0; k--) {
            const uint32_t pos = bbeg + (uint32_t)k - start;    // list position
            float dx, dy;
            const float4 uvo = s_uvo[k];
            const float gexp = gauss_at(uvo, s_q[k], px, py, dx, dy);
            const float raw = uvo.z * gexp;
            const float alpha = fminf(kAlphaMax, raw);
            const bool take = inside && pos < last && alpha >= kAlphaMin;
            if (__ballot(take) == 0) continue;
            float v[9];
#pragma unroll
            for (int q = 0; q < 9; q++) v[q] = 0.0f;
            if (take) {
                const float4 col = s_rgb[k];
                const float4 cn = s_conic[k];
                const float one_m = 1.0f - alpha;
                T = T * __builtin_amdgcn_rcpf(one_m);
                const float w = alpha * T;
                v[6] = w * G0;
                v[7] = w * G1;
                v[8] = w * G2;
                const float dla = T * ((col.x - A0) * G0 + (col.y - A1) * G1 + (col.z - A2) * G2);
                A0 = alpha * col.x + one_m * A0;
                A1 = alpha * col.y + one_m * A1;
                A2 = alpha * col.z + one_m * A2;
                if (raw < kAlphaMax) {
                    v[5] = dla * gexp;
                    const float dp = dla * alpha;
                    v[0] = -dp * (cn.x * dx + cn.y * dy);
                    v[1] = -dp * (cn.z * dy + cn.y * dx);
                    v[2] = -0.5f * dp * dx * dx;
                    v[3] = -dp * dx * dy;
                    v[4] = -0.5f * dp * dy * dy;
                }
            }
#pragma unroll
            for (int q = 0; q < 9; q++) {
                const float s = wave_sum(v[q]);
                if (lane == 0) atomicAdd(&s_acc[q][k], s);
            }
        }
        __syncthreads();
        for (int q = threadIdx.x; q < 9 * nb; q += kBlock) {
            const int comp = q / nb, k = q % nb;
            const float val = s_acc[comp][k];
            if (val != 0.0f) atomicAdd(&grad2d[(size_t)comp * n + s_g[k]], val);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_render_fwd(const Splat *splats, const uint32_t *vals, const uint32_t *ranges,
                             const Cam &cam, const float bg[3], float *image, float *final_T,
                             uint32_t *n_contrib, hipStream_t s)
{
    const int n_tiles = cam.tiles_x * cam.tiles_y;
    const int grid = 8 * ((n_tiles + 7) / 8);
    render_fwd_kernel<<<grid, kBlock, 0, s>>>(splats, vals, ranges, cam, bg[0], bg[1], bg[2], image,
                                              final_T, n_contrib);
    return hipGetLastError();
}

hipError_t launch_render_bwd(const Splat *splats, const uint32_t *vals, const uint32_t *ranges,
                             const Cam &cam, const float bg[3], const float *final_T,
                             const uint32_t *n_contrib, const float *dL_dimage, int64_t n,
                             float *grad2d, hipStream_t s)
{
    const int n_tiles = cam.tiles_x * cam.tiles_y;
    const int grid = 8 * ((n_tiles + 7) / 8);
    render_bwd_kernel<<<grid, kBlock, 0, s>>>(splats, vals, ranges, cam, bg[0], bg[1], bg[2], final_T,
                                              n_contrib, dL_dimage, (int)n, grad2d);
    return hipGetLastError();
}

}  // namespace gsi
