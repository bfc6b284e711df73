// Importance mask (gfx950): mask[g] = 1 for the `keep` Gaussians with the
// highest scores, ties to the lower index (BlitzGS page, section 2.3: a
// global pruning mask from accumulated importance, applied before the
// per-view level-of-detail gate).
//
// Radix select, MSB first, on an order-preserving 32-bit key of the score:
// four 8-bit histogram passes over the Gaussians whose key agrees with the
// digits chosen so far narrow the key down to the threshold T, the key of
// the keep-th largest score, and the number `need` of Gaussians with key T
// that still belong to the kept set.  A last pass writes the mask: key > T
// keeps, key == T keeps the first `need` in index order (a block-ordered
// rank), key < T drops.  Everything stays on the device; the selection
// state lives in the workspace.
#include <mutex>

#include "gs_internal.h"

namespace gsi {
namespace {

constexpr int kMaskItems = 4;                       // scores per thread per round (one float4)
constexpr int kMaskRounds = 4;
constexpr int kMaskBlockItems = kBlock * kMaskItems * kMaskRounds;   // 4096 scores per block

// Order-preserving key: larger score -> larger key; -0 and +0 are one value.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct MaskState {
    uint32_t prefix;     // digits chosen so far
    uint32_t need;       // kept Gaussians still to find inside the prefix bucket
};

struct MaskWs {
    uint32_t *hist;      // [4][256]
    MaskState *state;
    uint32_t *block_eq;  // [blocks] count of key == T per block, then its exclusive scan
};

__global__ __launch_bounds__(kBlock) void mask_init(uint32_t *__restrict__ hist, MaskState *__restrict__ st,
                                                    uint32_t keep)
{
    for (int i = threadIdx.x; i < 4 * 256; i += kBlock) hist[i] = 0;
    if (threadIdx.x == 0) {
        st->prefix = 0;
        st->need = keep;
    }
}

__device__ __forceinline__ void load_keys(const float *__restrict__ scores, uint32_t n, uint32_t i0,
                                          uint32_t k[kMaskItems], bool ok[kMaskItems])
{
    if (i0 + kMaskItems <= n && ((uintptr_t)(scores + i0) & 15u) == 0u) {
        const float4 v = *(const float4 *)(scores + i0);
        k[0] = score_key(v.x);
        k[1] = score_key(v.y);
        k[2] = score_key(v.z);
        k[3] = score_key(v.w);
#pragma unroll
        for (int j = 0; j < kMaskItems; j++) ok[j] = true;
    } else {
#pragma unroll
        for (int j = 0; j < kMaskItems; j++) {
            ok[j] = i0 + j < n;
            k[j] = ok[j] ? score_key(scores[i0 + j]) : 0u;
        }
    }
}

// Histogram of digit `pass` (bits 31-8*pass .. 24-8*pass) over the keys
// whose higher digits equal the chosen prefix.
__global__ __launch_bounds__(kBlock) void mask_hist(const float *__restrict__ scores, uint32_t n, int pass,
                                                    uint32_t *__restrict__ hist, const MaskState *__restrict__ st)
{
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : ~((1u << (shift + 8)) - 1u);
    const uint32_t prefix = st->prefix & hi_mask;
    const uint32_t base = blockIdx.x * (uint32_t)kMaskBlockItems;
    for (int r = 0; r < kMaskRounds; r++) {
        const uint32_t i0 = base + ((uint32_t)r * kBlock + threadIdx.x) * kMaskItems;
        if (i0 >= n) break;
        uint32_t k[kMaskItems];
        bool ok[kMaskItems];
        load_keys(scores, n, i0, k, ok);
#pragma unroll
        for (int j = 0; j < kMaskItems; j++)
            if (ok[j] && (k[j] & hi_mask) == prefix) atomicAdd(&h[(k[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&hist[pass * 256 + threadIdx.x], h[threadIdx.x]);
}

// Exclusive prefix of one count per thread over a block of NT threads;
// *total receives the block sum.  wsum holds NT / 64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_prefix(uint32_t x, uint32_t *wsum, uint32_t &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        if (i < w) before += wsum[i];
        total += wsum[i];
    }
    __syncthreads();
    return before + inc - x;
}

// Pick the digit holding the need-th largest key of the current bucket.
__global__ __launch_bounds__(kBlock) void mask_select(const uint32_t *__restrict__ hist, int pass,
                                                      MaskState *__restrict__ st)
{
    __shared__ uint32_t wsum[kBlock / 64];
    // thread t holds digit 255 - t, so its exclusive prefix counts the
    // keys in the larger digits
    const int d = 255 - (int)threadIdx.x;
    const uint32_t c = hist[pass * 256 + d];
    uint32_t all;
    const uint32_t before = block_prefix<kBlock>(c, wsum, all);
    const uint32_t need = st->need;
    __syncthreads();
    if (before < need && need <= before + c) {
        st->prefix |= (uint32_t)d << (24 - 8 * pass);
        st->need = need - before;
    }
}

// Per block: how many keys equal the threshold.
__global__ __launch_bounds__(kBlock) void mask_count_eq(const float *__restrict__ scores, uint32_t n,
                                                        const MaskState *__restrict__ st,
                                                        uint32_t *__restrict__ block_eq)
{
    __shared__ uint32_t total;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    const uint32_t T = st->prefix;
    const uint32_t base = blockIdx.x * (uint32_t)kMaskBlockItems;
    uint32_t c = 0;
    for (int r = 0; r < kMaskRounds; r++) {
        const uint32_t i0 = base + ((uint32_t)r * kBlock + threadIdx.x) * kMaskItems;
        if (i0 >= n) break;
        uint32_t k[kMaskItems];
        bool ok[kMaskItems];
        load_keys(scores, n, i0, k, ok);
#pragma unroll
        for (int j = 0; j < kMaskItems; j++) c += (ok[j] && k[j] == T) ? 1u : 0u;
    }
    if (c) atomicAdd(&total, c);
    __syncthreads();
    if (threadIdx.x == 0) block_eq[blockIdx.x] = total;
}

// Exclusive scan of the per-block counts (one block of 1024 threads).
__global__ __launch_bounds__(1024) void mask_scan_eq(uint32_t *__restrict__ block_eq, int blocks)
{
    __shared__ uint32_t wsum[1024 / 64];
    const int per = (blocks + 1023) / 1024;
    const int b0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int i = 0; i < per; i++)
        if (b0 + i < blocks) local += block_eq[b0 + i];
    uint32_t all;
    uint32_t run = block_prefix<1024>(local, wsum, all);
    for (int i = 0; i < per; i++)
        if (b0 + i < blocks) {
            const uint32_t v = block_eq[b0 + i];
            block_eq[b0 + i] = run;
            run += v;
        }
    if (threadIdx.x == 0) block_eq[blocks] = all;
}

__global__ __launch_bounds__(kBlock) void mask_write(const float *__restrict__ scores, uint32_t n,
                                                     const MaskState *__restrict__ st,
                                                     const uint32_t *__restrict__ block_eq,
                                                     uint8_t *__restrict__ mask)
{
    __shared__ uint32_t wsum[kBlock / 64];
    const uint32_t T = st->prefix, need = st->need;
    const uint32_t base = blockIdx.x * (uint32_t)kMaskBlockItems;
    // rank of the next key == T inside the whole array, in index order
    uint32_t rank = block_eq[blockIdx.x];
    const bool ties_here = block_eq[blockIdx.x + 1] > rank;
    for (int r = 0; r < kMaskRounds; r++) {
        const uint32_t i0 = base + ((uint32_t)r * kBlock + threadIdx.x) * kMaskItems;
        uint32_t k[kMaskItems];
        bool ok[kMaskItems];
        load_keys(scores, n, i0 < n ? i0 : n, k, ok);
        uint32_t eq = 0;
#pragma unroll
        for (int j = 0; j < kMaskItems; j++) eq += (ok[j] && k[j] == T) ? 1u : 0u;
        uint32_t my = rank, round_total = 0;
        if (ties_here) {
            my = rank + block_prefix<kBlock>(eq, wsum, round_total);
            rank += round_total;
        }
        uint8_t m[kMaskItems];
#pragma unroll
        for (int j = 0; j < kMaskItems; j++) {
            bool keepit = ok[j] && k[j] > T;
            if (ok[j] && k[j] == T) {
                keepit = my < need;
                my++;
            }
            m[j] = keepit ? 1 : 0;
        }
        if (i0 + kMaskItems <= n && ((uintptr_t)(mask + i0) & 3u) == 0u) {
            uchar4 v;
            v.x = m[0];
            v.y = m[1];
            v.z = m[2];
            v.w = m[3];
            *(uchar4 *)(mask + i0) = v;
        } else {
#pragma unroll
            for (int j = 0; j < kMaskItems; j++)
                if (i0 + j < n) mask[i0 + j] = m[j];
        }
    }
}

__global__ __launch_bounds__(kBlock) void fill_u8(uint8_t *__restrict__ p, uint8_t v, uint32_t n)
{
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < n) p[i] = v;
}

uint32_t mask_blocks(int64_t n) { return (uint32_t)((n + kMaskBlockItems - 1) / kMaskBlockItems); }

size_t carve_mask(char *base, int64_t n, MaskWs *ws)
{
    size_t off = 0;
    MaskWs w;
    w.hist = (uint32_t *)((uintptr_t)base + off);     // integer: also sized on a null base
    off = align_up(off + 4 * 256 * sizeof(uint32_t), 256);
    w.state = (MaskState *)((uintptr_t)base + off);
    off = align_up(off + sizeof(MaskState), 256);
    w.block_eq = (uint32_t *)((uintptr_t)base + off);
    off = align_up(off + (size_t)(mask_blocks(n) + 1) * sizeof(uint32_t), 256);
    if (ws) *ws = w;
    return off;
}

}  // namespace

size_t active_mask_workspace(int64_t n) { return carve_mask(nullptr, n > 0 ? n : 0, nullptr) + 256; }

}  // namespace gsi

// ---- allocation-free variant -------------------------------------------------
// For callers that cannot allocate device memory: the selection state
// (histograms, threshold, per-block tie counts) lives in this fixed array,
// one copy per GPU, held until the process ends.  Its size is carve_mask's
// layout for GS_ACTIVE_MASK_STATIC_MAX_N scores: 4 KiB of histograms, the
// state, and one word per 4096-score block (+1), each part 256-byte aligned.
// Every word a call reads is first written by that call's own kernels
// (mask_init clears the histograms and sets the state; mask_count_eq writes
// every block count before the scan), so nothing carries over between calls.
// Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, once per device.
namespace {
constexpr size_t kStaticMaskBlocks =
    (size_t)((GS_ACTIVE_MASK_STATIC_MAX_N + gsi::kMaskBlockItems - 1) / gsi::kMaskBlockItems);
constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kStaticMaskBytes =
    align256(align256(align256(4 * 256 * sizeof(uint32_t)) + sizeof(gsi::MaskState)) +
             (kStaticMaskBlocks + 1) * sizeof(uint32_t));
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];          // device address of `scratch` per device
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticMaskBytes];

namespace gsi {

size_t static_mask_scratch_bytes() { return kStaticMaskBytes; }

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current.
static hipError_t static_mask_scratch(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

hipError_t launch_active_mask_static(const float *scores, int64_t n, int64_t keep, uint8_t *mask, hipStream_t s)
{
    if (carve_mask(nullptr, n, nullptr) > kStaticMaskBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = static_mask_scratch(&ws);
    if (e != hipSuccess) return e;
    return launch_active_mask(scores, n, keep, mask, ws, kStaticMaskBytes, s);
}

hipError_t launch_active_mask(const float *scores, int64_t n64, int64_t keep, uint8_t *mask, void *ws_ptr,
                              size_t ws_bytes, hipStream_t s)
{
    (void)ws_bytes;
    if (n64 == 0) return hipSuccess;
    const uint32_t n = (uint32_t)n64;
    if (keep == 0 || keep == n64) {
        fill_u8<<<(n + kBlock - 1) / kBlock, kBlock, 0, s>>>(mask, keep == 0 ? 0 : 1, n);
        return hipGetLastError();
    }
    char *base = (char *)align_up((size_t)ws_ptr, 256);
    MaskWs w;
    carve_mask(base, n64, &w);
    const uint32_t blocks = mask_blocks(n64);
    mask_init<<<1, kBlock, 0, s>>>(w.hist, w.state, (uint32_t)keep);
    for (int pass = 0; pass < 4; pass++) {
        mask_hist<<<blocks, kBlock, 0, s>>>(scores, n, pass, w.hist, w.state);
        mask_select<<<1, kBlock, 0, s>>>(w.hist, pass, w.state);
    }
    mask_count_eq<<<blocks, kBlock, 0, s>>>(scores, n, w.state, w.block_eq);
    mask_scan_eq<<<1, 1024, 0, s>>>(w.block_eq, (int)blocks);
    mask_write<<<blocks, kBlock, 0, s>>>(scores, n, w.state, w.block_eq, mask);
    return hipGetLastError();
}

}  // namespace gsi
