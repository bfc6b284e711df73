// Fused SH Adam step for gfx950: one pass over the SH gradients, values and
// both Adam moments, updating values and moments in place (the fused SH
// optimizer of the Spirula Studio page, with its 16-bit values and 8-bit
// log-domain moments in 256-Gaussian blocks).
//
// The step is HBM-bound: per unit (one SH coefficient of one channel of one
// Gaussian) the 8-bit state moves 8 bytes in (fp32 gradient, fp16 value, two
// codes) and 4 out, the full-precision state 16 in and 12 out.  Loads and
// stores are coalesced along the Gaussian axis of the [rows][n] arrays; when
// n is a multiple of 4 a lane moves 4 consecutive units with one vector load
// per array.  For the 8-bit state one wave owns one 256-unit block, so the
// block's bounds come in by scalar loads and its new min/max is a wave
// reduction with no LDS and no barrier.
#include "gs_adam.h"

#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>

namespace gsi {
namespace {

constexpr int kAdamThreads = 256;              // 4 waves per workgroup
constexpr int kUnitsPerBlock = 256;            // units sharing one (lo, hi) pair
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

struct AdamCoef {
    float lr, b1, b2, omb1, omb2;              // omb = 1 - b
    float rbc1, rbc2;                          // 1 / (1 - b^t)
    float eps, reps;                           // eps and 1 / eps
    int lazy;                                  // 1: zero-gradient units keep their state
};

struct AdamArgs {
    AdamCoef k;
    const float *grad;
    void *value;
    void *m, *v;
    float *mb, *vb;
    int n, nb;
    long long total;                           // rows * n
};

// Streaming accesses: the gradients and the moments are touched once per
// step, so their loads and stores carry the non-temporal hint (native vector
// types, as the builtins require).  At 5M x 45 units it took the fp32 state
// from 1.14 to about 1.0 ms and the 8-bit state from 0.50 to 0.49 ms; the
// hint on the values' accesses measured no better and is left off.
typedef float nf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float *p)
{
    const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float *p, float a, float b, float c, float d)
{
    nf4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<nf4 *>(p));
}

template <typename TV> __device__ __forceinline__ float to_f(TV x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<__half>(__half x) { return __half2float(x); }
template <typename TV> __device__ __forceinline__ TV from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __half from_f<__half>(float x) { return __float2half_rn(x); }

// Four consecutive values of type TV as one vector access.
template <typename TV> struct Vec4;
template <> struct Vec4<float> { using T = float4; };
template <> struct Vec4<__half> { using T = uint2; };

template <typename TV>
__device__ __forceinline__ void load4(const TV *p, float out[4])
{
    const typename Vec4<TV>::T w = *reinterpret_cast<const typename Vec4<TV>::T *>(p);
    const TV *e = reinterpret_cast<const TV *>(&w);
#pragma unroll
    for (int j = 0; j < 4; j++) out[j] = to_f<TV>(e[j]);
}

template <typename TV>
__device__ __forceinline__ void store4(TV *p, const float in[4])
{
    typename Vec4<TV>::T w;
    TV *e = reinterpret_cast<TV *>(&w);
#pragma unroll
    for (int j = 0; j < 4; j++) e[j] = from_f<TV>(in[j]);
    *reinterpret_cast<typename Vec4<TV>::T *>(p) = w;
}

// Whether a unit moves this step: every unit (dense), or only those with a
// non-zero gradient (lazy: a Gaussian none of the step's views saw keeps
// its value and moments).
__device__ __forceinline__ bool unit_live(float g, const AdamCoef &k) { return !k.lazy || g != 0.0f; }

// The bias-corrected Adam update of one unit; m and v are replaced by the
// new moments, the new value is returned (fp32, before storage rounding).
__device__ __forceinline__ float adam_unit(float th, float &m, float &v, float g, const AdamCoef &k)
{
    const bool live = unit_live(g, k);
    const float m1 = k.b1 * m + k.omb1 * g;
    const float v1 = k.b2 * v + k.omb2 * (g * g);
    const float den = __builtin_amdgcn_sqrtf(v1 * k.rbc2) + k.eps;
    const float th1 = th - k.lr * (m1 * k.rbc1) * __builtin_amdgcn_rcpf(den);
    m = live ? m1 : m;
    v = live ? v1 : v;
    return live ? th1 : th;
}

// ---------------------------------------------------------------------------
// Full-precision state: an elementwise pass over the flat [rows * n] arrays.
template <typename TV, bool kVec>
__global__ __launch_bounds__(kAdamThreads) void adam_f32_kernel(AdamArgs a)
{
    const float *__restrict__ gp = a.grad;
    TV *__restrict__ vp = static_cast<TV *>(a.value);
    float *__restrict__ mp = static_cast<float *>(a.m);
    float *__restrict__ sp = static_cast<float *>(a.v);
    const long long stride = (long long)gridDim.x * kAdamThreads * 4;
    for (long long i = ((long long)blockIdx.x * kAdamThreads + threadIdx.x) * 4; i < a.total; i += stride) {
        float g[4], th[4], m[4], v[4];
        if (kVec) {
            const float4 g4 = ld_nt(gp + i);
            const float4 m4 = ld_nt(mp + i);
            const float4 v4 = ld_nt(sp + i);
            load4<TV>(vp + i, th);
            g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
            m[0] = m4.x; m[1] = m4.y; m[2] = m4.z; m[3] = m4.w;
            v[0] = v4.x; v[1] = v4.y; v[2] = v4.z; v[3] = v4.w;
#pragma unroll
            for (int j = 0; j < 4; j++) th[j] = adam_unit(th[j], m[j], v[j], g[j], a.k);
            store4<TV>(vp + i, th);
            st_nt(mp + i, m[0], m[1], m[2], m[3]);
            st_nt(sp + i, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if (i + j >= a.total) break;
                float mj = mp[i + j], vj = sp[i + j];
                const float t = adam_unit(to_f<TV>(vp[i + j]), mj, vj, gp[i + j], a.k);
                vp[i + j] = from_f<TV>(t);
                mp[i + j] = mj;
                sp[i + j] = vj;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 8-bit state.  Decode as documented for block-quantized storage: lo + q *
// step, step = (hi - lo) * fp32(1/255), one rounding per operation.
__device__ __forceinline__ float decode8(float lo, float step, uint32_t q)
{
#pragma clang fp contract(off)
    return lo + (float)q * step;
}

// Order-preserving map of a float onto a signed integer (and back: the map
// is its own inverse), so that block minima and maxima are integer minima.
__device__ __forceinline__ int fkey(float x)
{
    const int b = __float_as_int(x);
    return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float unkey(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, true); }

__device__ __forceinline__ int min_swap32(int v)
{
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return min((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int min_swap16(int v)
{
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return min((int)r[0], (int)r[1]);
}

// Minimum over the wave, in every lane: DPP quad, 8- and 16-lane steps, then
// the 32- and 64-lane steps on lane swaps.
__device__ __forceinline__ int wave_min_i(int v)
{
    v = min(v, dpp_i<0xB1>(v));     // quad_perm [1,0,3,2]
    v = min(v, dpp_i<0x4E>(v));     // quad_perm [2,3,0,1]
    v = min(v, dpp_i<0x141>(v));    // row_half_mirror
    v = min(v, dpp_i<0x128>(v));    // row_ror:8
    v = min_swap16(v);
    return min_swap32(v);
}

// Nearest code of x >= lo in a block with minimum lo and 255 / (hi - lo) =
// scale (0 for a constant block): t >= 1/2, and truncation is floor.
__device__ __forceinline__ uint32_t encode8(float x, float lo, float scale)
{
    const float t = (x - lo) * scale + 0.5f;
    return min((uint32_t)t, 255u);
}

// One wave per (row, 256-unit block); blockIdx.y is the row and the 4 waves
// of a workgroup take 4 consecutive blocks.  kVec: lane l holds units
// 4l .. 4l+3 of the block (n % 4 == 0, so they are all valid or all past the
// end); otherwise units l, l+64, l+128, l+192.
template <typename TV, bool kVec>
__global__ __launch_bounds__(kAdamThreads) void adam_q8_kernel(AdamArgs a)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int blk = blockIdx.x * (kAdamThreads / 64) + wave;
    if (blk >= a.nb) return;
    const size_t row0 = (size_t)blockIdx.y * a.n;
    const size_t bi = ((size_t)blockIdx.y * a.nb + blk) * 2;
    const float mlo = a.mb[bi], mhi = a.mb[bi + 1];
    const float slo = a.vb[bi], shi = a.vb[bi + 1];
    const float mst = (mhi - mlo) * (1.0f / 255.0f);
    const float sst = (shi - slo) * (1.0f / 255.0f);

    const float *__restrict__ gp = a.grad + row0;
    TV *__restrict__ vp = static_cast<TV *>(a.value) + row0;
    uint8_t *__restrict__ mp = static_cast<uint8_t *>(a.m) + row0;
    uint8_t *__restrict__ sp = static_cast<uint8_t *>(a.v) + row0;
    const int u0 = blk * kUnitsPerBlock;

    float g[4] = {0.0f, 0.0f, 0.0f, 0.0f}, th[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t cm[4] = {0u, 0u, 0u, 0u}, cs[4] = {0u, 0u, 0u, 0u};
    bool ok[4];
    if (kVec) {
        // lanes past the end of the row re-read the row's last 4 units (n >= 4)
        // and take no part in the bounds or the stores
        const int u = u0 + 4 * lane;
        const bool valid = u < a.n;
        const int ul = valid ? u : a.n - 4;
        const float4 g4 = ld_nt(gp + ul);
        g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
        load4<TV>(vp + ul, th);
        const uint32_t wm = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(mp + ul));
        const uint32_t ws = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sp + ul));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            cm[j] = (wm >> (8 * j)) & 255u;
            cs[j] = (ws >> (8 * j)) & 255u;
            ok[j] = valid;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int u = u0 + lane + 64 * j;
            ok[j] = u < a.n;
            if (ok[j]) {
                g[j] = gp[u];
                th[j] = to_f<TV>(vp[u]);
                cm[j] = mp[u];
                cs[j] = sp[u];
            }
        }
    }

    // Adam in fp32; the second moment leaves and re-enters the log domain,
    // handled in base 2 inside the kernel (s log2(e) in, log2 out; the
    // block's new bounds go back to natural-log units once per block).
    const float slo2 = slo * kLog2e, sst2 = sst * kLog2e;
    float m1[4], s1[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float s2 = decode8(slo2, sst2, cs[j]);                                   // s / ln 2
        const float r = a.k.eps * (__builtin_amdgcn_exp2f(s2) - 1.0f);                   // sqrt(v)
        float m = decode8(mlo, mst, cm[j]), v = r * r;
        th[j] = adam_unit(th[j], m, v, g[j], a.k);
        m1[j] = m;
        const float s2n = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_sqrtf(v) * a.k.reps);
        s1[j] = unit_live(g[j], a.k) ? s2n : s2;          // an untouched unit keeps its s
    }
    // the block's new bounds: lane minima and maxima in fp32, then wave
    // minima of (m, -m, s, -s) as integer keys (s >= 0 is its own key)
    float lo_m, hi_m, lo_s, hi_s;
    if (kVec) {
        lo_m = fminf(fminf(m1[0], m1[1]), fminf(m1[2], m1[3]));
        hi_m = fmaxf(fmaxf(m1[0], m1[1]), fmaxf(m1[2], m1[3]));
        lo_s = fminf(fminf(s1[0], s1[1]), fminf(s1[2], s1[3]));
        hi_s = fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]));
        if (!ok[0]) {
            lo_m = lo_s = INFINITY;
            hi_m = -INFINITY;
            hi_s = 0.0f;
        }
    } else {
        lo_m = lo_s = INFINITY;
        hi_m = -INFINITY;
        hi_s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            lo_m = fminf(lo_m, ok[j] ? m1[j] : INFINITY);
            hi_m = fmaxf(hi_m, ok[j] ? m1[j] : -INFINITY);
            lo_s = fminf(lo_s, ok[j] ? s1[j] : INFINITY);
            hi_s = fmaxf(hi_s, ok[j] ? s1[j] : 0.0f);
        }
    }
    const float mlo1 = unkey(wave_min_i(fkey(lo_m))), mhi1 = unkey(~wave_min_i(~fkey(hi_m)));
    const float slo2n = __int_as_float(wave_min_i(__float_as_int(lo_s)));
    const float shi2n = __int_as_float(~wave_min_i(~__float_as_int(hi_s)));
    const float slo1 = slo2n * kLn2, shi1 = shi2n * kLn2;
    const float md = mhi1 - mlo1, sd = shi2n - slo2n;
    const float mscale = md > 0.0f ? 255.0f * __builtin_amdgcn_rcpf(md) : 0.0f;
    const float sscale = sd > 0.0f ? 255.0f * __builtin_amdgcn_rcpf(sd) : 0.0f;

    if (lane == 0) {                              // bounds need only 4-byte alignment
        a.mb[bi] = mlo1;
        a.mb[bi + 1] = mhi1;
        a.vb[bi] = slo1;
        a.vb[bi + 1] = shi1;
    }
    if (kVec) {
        const int u = u0 + 4 * lane;
        if (u < a.n) {
            uint32_t wm = 0, ws = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                wm |= encode8(m1[j], mlo1, mscale) << (8 * j);
                ws |= encode8(s1[j], slo2n, sscale) << (8 * j);
            }
            store4<TV>(vp + u, th);
            __builtin_nontemporal_store(wm, reinterpret_cast<uint32_t *>(mp + u));
            __builtin_nontemporal_store(ws, reinterpret_cast<uint32_t *>(sp + u));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int u = u0 + lane + 64 * j;
            if (!ok[j]) continue;
            vp[u] = from_f<TV>(th[j]);
            mp[u] = (uint8_t)encode8(m1[j], mlo1, mscale);
            sp[u] = (uint8_t)encode8(s1[j], slo2n, sscale);
        }
    }
}

template <typename TV>
hipError_t launch_typed(const AdamArgs &a, int rows, bool q8, bool vec, hipStream_t s)
{
    if (q8) {
        const dim3 grid((unsigned)((a.nb + 3) / 4), (unsigned)rows);
        if (vec)
            adam_q8_kernel<TV, true><<<grid, kAdamThreads, 0, s>>>(a);
        else
            adam_q8_kernel<TV, false><<<grid, kAdamThreads, 0, s>>>(a);
    } else {
        const long long groups = (a.total + 4LL * kAdamThreads - 1) / (4LL * kAdamThreads);
        const unsigned grid = (unsigned)(groups < (1LL << 20) ? groups : (1LL << 20));
        if (vec)
            adam_f32_kernel<TV, true><<<grid, kAdamThreads, 0, s>>>(a);
        else
            adam_f32_kernel<TV, false><<<grid, kAdamThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

bool aligned(const void *p, uintptr_t bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

}  // namespace

hipError_t launch_sh_adam(const gs_sh_adam &p, hipStream_t s)
{
    if (p.n == 0) return hipSuccess;
    const double bc1 = 1.0 - pow((double)p.beta1, (double)p.step);
    const double bc2 = 1.0 - pow((double)p.beta2, (double)p.step);
    AdamArgs a;
    a.k.lr = p.lr;
    a.k.b1 = p.beta1;
    a.k.b2 = p.beta2;
    a.k.omb1 = (float)(1.0 - (double)p.beta1);
    a.k.omb2 = (float)(1.0 - (double)p.beta2);
    a.k.rbc1 = (float)(1.0 / bc1);
    a.k.rbc2 = (float)(1.0 / bc2);
    a.k.eps = p.eps;
    a.k.reps = (float)(1.0 / (double)p.eps);
    a.k.lazy = p.update == GS_ADAM_LAZY ? 1 : 0;
    a.grad = p.grad;
    a.value = p.value;
    a.m = p.m;
    a.v = p.v;
    a.mb = p.m_bounds;
    a.vb = p.v_bounds;
    a.n = (int)p.n;
    a.nb = (int)((p.n + kUnitsPerBlock - 1) / kUnitsPerBlock);
    a.total = (long long)p.rows * p.n;
    const bool q8 = p.state_dtype == GS_ADAM_Q8LOG;
    const bool f16 = p.value_dtype == GS_SH_F16;
    const uintptr_t vw = f16 ? 8 : 16;
    // vector path: every 4-unit group starts on a 4-unit boundary (of a row
    // for the 8-bit state, of the flat array otherwise) and every array is
    // aligned for its 4-unit vector access
    bool vec = aligned(p.grad, 16) && aligned(p.value, vw);
    if (q8)
        vec = vec && p.n % 4 == 0 && aligned(p.m, 4) && aligned(p.v, 4);
    else
        vec = vec && a.total % 4 == 0 && aligned(p.m, 16) && aligned(p.v, 16);
    return f16 ? launch_typed<__half>(a, p.rows, q8, vec, s) : launch_typed<float>(a, p.rows, q8, vec, s);
}

}  // namespace gsi
