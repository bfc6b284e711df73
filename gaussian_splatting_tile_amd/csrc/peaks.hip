// Measured peaks of the GPU the rasterizer runs on (gfx950): the rates that
// the roofline fractions of the blend kernels (VALU lane operations) and of
// the projection, sort and projection backward (HBM bytes) are taken
// against, besides the chip's published figures.
//
//   fma32   non-packed fp32 FMA, lane operations per second
//   fma64   fp64 FMA, lane operations per second
//   exp32   v_exp_f32 alone, lane operations per second
//   mix     one v_exp_f32 and four fp32 FMAs per round: whether the
//           transcendental shares the FMA issue slots (then a round costs
//           4 + cost(exp) FMA slots)
//   add32, mul32, sel32, add64   chains of one simple instruction class
//           (fp32 add, fp32 mul, compare + select, fp64 add), lane
//           operations per second: the classes that issue faster than an FMA
//   lds     LDS reads (16 bytes per lane per read, no bank conflicts),
//           bytes per second
//   copy    a device copy with 16-byte loads and stores, bytes moved
//           (read + written) per second
//
// Every arithmetic kernel runs independent chains (eight per lane) so that
// issue, not latency, bounds it, on a grid of many waves per SIMD.  Packed
// fp32 instructions are not generated (the library's build flags turn them
// off), so the fp32 figure is the non-packed rate the kernels use.  Nothing
// here is on the rendering path; bench.py calls it once before timing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void fma32_kernel(float *out, int iters, float m, float c)
{
    float a[kChains];
#pragma unroll
    for (int i = 0; i < kChains; i++) a[i] = (float)(threadIdx.x + i) * 1e-3f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
#pragma unroll
            for (int i = 0; i < kChains; i++) a[i] = __builtin_fmaf(a[i], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; i++) s += a[i];
    if (s == 12345.0f) out[blockIdx.x * kThreads + threadIdx.x] = s;   // keeps the chains live
}

__global__ __launch_bounds__(kThreads) void fma64_kernel(double *out, int iters, double m, double c)
{
    double a[kChains];
#pragma unroll
    for (int i = 0; i < kChains; i++) a[i] = (double)(threadIdx.x + i) * 1e-3;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
#pragma unroll
            for (int i = 0; i < kChains; i++) a[i] = __builtin_fma(a[i], m, c);
    }
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kChains; i++) s += a[i];
    if (s == 12345.0) out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// x <- 2^-x keeps every chain inside [1/2, 1] (the negation is a source
// modifier of the instruction, not a separate one).
__global__ __launch_bounds__(kThreads) void exp32_kernel(float *out, int iters)
{
    float a[kChains];
#pragma unroll
    for (int i = 0; i < kChains; i++) a[i] = (float)(threadIdx.x + i) * 1e-3f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
#pragma unroll
            for (int i = 0; i < kChains; i++) a[i] = __builtin_amdgcn_exp2f(-a[i]);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; i++) s += a[i];
    if (s == 12345.0f) out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Chains of one simple instruction each: fp32 add (x <- x + c), fp32 mul
// (x <- x * m, m close to 1), select (x <- x > t ? x : y, a compare and a
// v_cndmask each), fp64 add; they tell which instruction classes issue faster
// than the FMA.
template <int kOp>
__global__ __launch_bounds__(kThreads) void simple_kernel(float *out, int iters, float m, float c)
{
    float a[kChains];
    double d[kChains];
#pragma unroll
    for (int i = 0; i < kChains; i++) {
        a[i] = (float)(threadIdx.x + i) * 1e-3f;
        d[i] = (double)a[i];
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
#pragma unroll
            for (int i = 0; i < kChains; i++) {
                if (kOp == 0) a[i] = a[i] + c;
                if (kOp == 1) a[i] = a[i] * m;
                if (kOp == 2) a[i] = a[i] > c ? a[i] : m;
                if (kOp == 3) d[i] = d[i] + (double)c;
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; i++) s += a[i] + (float)d[i];
    if (s == 12345.0f) out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Per round and chain pair: one exp on the first chain, four FMAs spread
// over the second.
__global__ __launch_bounds__(kThreads) void mix_kernel(float *out, int iters, float m, float c)
{
    float e[kChains / 2], f[kChains / 2];
#pragma unroll
    for (int i = 0; i < kChains / 2; i++) {
        e[i] = (float)(threadIdx.x + i) * 1e-3f;
        f[i] = (float)(threadIdx.x + 2 * i) * 1e-3f;
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
#pragma unroll
            for (int i = 0; i < kChains / 2; i++) {
                e[i] = __builtin_amdgcn_exp2f(-e[i]);
                f[i] = __builtin_fmaf(f[i], m, c);
                f[i] = __builtin_fmaf(f[i], m, c);
                f[i] = __builtin_fmaf(f[i], m, c);
                f[i] = __builtin_fmaf(f[i], m, c);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains / 2; i++) s += e[i] + f[i];
    if (s == 12345.0f) out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Each lane reads 16 bytes per access from a 16 KiB LDS array: the lanes of
// a wave read 64 consecutive 16-byte words (no bank conflicts), the sixteen
// reads of a round are sixteen distinct 1 KiB stripes, and the stripe
// rotates every round.
__global__ __launch_bounds__(kThreads) void lds_kernel(float *out, int iters)
{
    __shared__ float4 buf[1024];
    for (int i = threadIdx.x; i < 1024; i += kThreads)
        buf[i] = make_float4((float)i, 1.0f, 2.0f, 3.0f);
    __syncthreads();
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int idx = threadIdx.x;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const float4 v = buf[(idx + k * 64) & 1023];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        idx += 64;
    }
    if (acc.x + acc.y + acc.z + acc.w == 12345.0f) out[blockIdx.x * kThreads + threadIdx.x] = acc.x;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                        size_t n)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

int resident_grid(const void *kernel)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess) return 0;
    return cus * (per_cu > 0 ? per_cu : 1);
}

}  // namespace

extern "C" {

// Kinds of gsp_measure.
enum { GSP_FMA32 = 0, GSP_FMA64 = 1, GSP_EXP32 = 2, GSP_MIX = 3, GSP_LDS = 4, GSP_COPY = 5,
       GSP_ADD32 = 6, GSP_MUL32 = 7, GSP_SEL32 = 8, GSP_ADD64 = 9 };

static const void *arith_kernel(int kind)
{
    switch (kind) {
    case GSP_FMA32: return (const void *)fma32_kernel;
    case GSP_FMA64: return (const void *)fma64_kernel;
    case GSP_EXP32: return (const void *)exp32_kernel;
    case GSP_MIX: return (const void *)mix_kernel;
    case GSP_LDS: return (const void *)lds_kernel;
    case GSP_ADD32: return (const void *)simple_kernel<0>;
    case GSP_MUL32: return (const void *)simple_kernel<1>;
    case GSP_SEL32: return (const void *)simple_kernel<2>;
    case GSP_ADD64: return (const void *)simple_kernel<3>;
    default: return (const void *)copy_kernel;
    }
}

// Runs one measurement on the current device and stream (synchronising it)
// and returns the rate: lane operations per second for GSP_FMA32, GSP_FMA64,
// GSP_EXP32 (one per exp), GSP_MIX (rounds of one exp + four FMAs per second),
// bytes per second for GSP_LDS and GSP_COPY.  `scratch` is device memory of
// at least `scratch_bytes`: 8 bytes per thread of the grid for the arithmetic
// kinds (gsp_scratch_bytes; never written in practice), the two halves of
// the copy for GSP_COPY.  `iters` scales the work (rounds of 16 per lane, or copy
// repetitions).  Returns a negative value on a HIP error.
size_t gsp_scratch_bytes(int kind)
{
    return (size_t)8 * resident_grid(arith_kernel(kind)) * kThreads * sizeof(double);
}

double gsp_measure(int kind, int iters, void *scratch, size_t scratch_bytes, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (kind < GSP_FMA32 || kind > GSP_ADD64 || iters < 1 || !scratch) return -3.0;
    double work = 0.0;
    hipError_t err = hipSuccess;
    const void *kern = arith_kernel(kind);
    // eight resident waves' worth of blocks per slot, so that the tail is short
    const int grid = 8 * resident_grid(kern);
    if (grid <= 0) return -1.0;
    if (kind != GSP_COPY && scratch_bytes < (size_t)grid * kThreads * sizeof(double)) return -2.0;
    if (kind == GSP_COPY && scratch_bytes < 2 * sizeof(float4)) return -2.0;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -1.0;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -1.0;
    }
    const double lanes = (double)grid * kThreads;
    for (int rep = 0; rep < 2 && err == hipSuccess; rep++) {      // the first run warms up
        (void)hipEventRecord(e0, s);
        switch (kind) {
        case GSP_FMA32:
            fma32_kernel<<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_FMA64:
            fma64_kernel<<<grid, kThreads, 0, s>>>((double *)scratch, iters, 0.9999, 1e-4);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_EXP32:
            exp32_kernel<<<grid, kThreads, 0, s>>>((float *)scratch, iters);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_MIX:
            mix_kernel<<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * (kChains / 2);
            break;
        case GSP_ADD32:
            simple_kernel<0><<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_MUL32:
            simple_kernel<1><<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_SEL32:
            simple_kernel<2><<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_ADD64:
            simple_kernel<3><<<grid, kThreads, 0, s>>>((float *)scratch, iters, 0.9999f, 1e-4f);
            work = lanes * iters * 16.0 * kChains;
            break;
        case GSP_LDS:
            lds_kernel<<<grid, kThreads, 0, s>>>((float *)scratch, iters);
            work = lanes * iters * 16.0 * 16.0;
            break;
        case GSP_COPY: {
            const size_t n = scratch_bytes / 2 / sizeof(float4);
            const float4 *src = (const float4 *)scratch;
            float4 *dst = (float4 *)scratch + n;
            const int cgrid = resident_grid((const void *)copy_kernel);
            for (int r = 0; r < iters; r++) copy_kernel<<<cgrid, kThreads, 0, s>>>(src, dst, n);
            work = 2.0 * (double)n * sizeof(float4) * iters;
            break;
        }
        default:
            break;
        }
        err = hipGetLastError();
        (void)hipEventRecord(e1, s);
    }
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (err != hipSuccess || ms <= 0.0f) return -1.0;
    return work / (ms * 1e-3);
}

}  // extern "C"
