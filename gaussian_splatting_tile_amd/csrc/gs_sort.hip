// Tile binning and depth sort (gfx950).
//
// The result is the stable LSB radix sort of the 64-bit keys
//     key = tile << 32 | bits(depth)      (depth > 0, so the bits are monotone)
// emitted in (Gaussian index, tile row-major) order, i.e. every tile's list
// ordered by depth with the lower Gaussian index first among equal depths.
//
// An LSB radix sort handles the low digits first.  The low 32 bits (the
// depth) are the same for every key a Gaussian emits, so the depth passes run
// on the N projected Gaussians instead of on the K >= N duplicated keys:
//   1. depth passes: stable 4 x 8-bit LSB sort of (depth bits, g) over the
//      visible Gaussians (culled ones drop out in the first pass);
//   2. duplication in that order: an exclusive scan of tiles_touched gives
//      each Gaussian its slots, where it writes (tile, g) for its rect (or,
//      with reach lists, for the tiles of its rect it can reach with
//      alpha >= 1/255: counted in the scan, the rest never emitted);
//   3. tile passes: stable LSB passes of <= 8 bits over the tile id (the high
//      digits of the key) on the K entries;
//   4. tile ranges from the boundaries of the sorted tile ids.
// Duplication keeps the relative order of the Gaussians, so this is the same
// permutation as sorting all K 64-bit keys, with the depth digits moved
// before the duplication.  The depth keys and tile rects come from the
// projection when it wrote them, else from the records (bin_init).
//
// No host round trip: item counts (visible Gaussians, K) stay in device
// memory; every grid is sized from host-known upper bounds and blocks past
// the live count exit early.  Each radix pass is reduce-then-scan:
// per-block digit counts (upsweep), a per-digit scan across blocks, then a
// downsweep that ranks each 4096-item tile with wave ballots (match of equal
// digits), orders it in LDS and writes every digit's run contiguously.
#include "gs_internal.h"

namespace gsi {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;          // 4
constexpr int kIpt = 16;                        // items per thread per tile
constexpr int kTileItems = kBlock * kIpt;       // 4096
constexpr int kWaveItems = kWave * kIpt;        // 1024
constexpr int kMaxGrid = 512;                   // radix blocks per pass

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// DPP lane moves for the wave scans: row_shr:n takes the value of lane
// i - n of the same 16-lane row, row_bcast:15 / row_bcast:31 the last lane
// of the previous row / of the first two rows, for the rows row_mask
// enables.  Lanes without a source (or disabled) read 0.
constexpr int kDppRowShr = 0x110;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v)
{
    const uint32_t lo = dpp_move<kCtrl, kRowMask>((uint32_t)v);
    const uint32_t hi = dpp_move<kCtrl, kRowMask>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan across one wave64: Kogge-Stone inside each 16-lane row on
// DPP row shifts, then the rows' totals carried forward by the two row
// broadcasts.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x)
{
    x += dpp_move<kDppRowShr + 1>(x);
    x += dpp_move<kDppRowShr + 2>(x);
    x += dpp_move<kDppRowShr + 4>(x);
    x += dpp_move<kDppRowShr + 8>(x);
    x += dpp_move<kDppRowBcast15, 0xA>(x);     // rows 1, 3 += last lane of rows 0, 2
    x += dpp_move<kDppRowBcast31, 0xC>(x);     // rows 2, 3 += last lane of row 1
    return x;
}

// Exclusive scan of one value per thread across the 256-thread block;
// returns the exclusive prefix, *total receives the block sum.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T x, T *total)
{
    __shared__ T wsum[kWaves];
    const T inc = wave_inclusive_scan(x);
    if (lane_id() == kWave - 1) wsum[wave_id()] = inc;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        if (w < wave_id()) before += wsum[w];
        all += wsum[w];
    }
    __syncthreads();
    if (total) *total = all;
    return before + inc - x;
}

__device__ __forceinline__ void chunk_of(uint32_t n, uint32_t &begin, uint32_t &end)
{
    const uint32_t G = gridDim.x;
    uint32_t chunk = (n + G - 1) / G;
    chunk = (chunk + kTileItems - 1) / kTileItems * kTileItems;
    const uint64_t b = (uint64_t)blockIdx.x * chunk;
    begin = b < n ? (uint32_t)b : n;
    const uint64_t e = b + chunk;
    end = e < n ? (uint32_t)e : n;
}

// ---------------------------------------------------------------------------
// Every kernel below runs over a batch of views: blockIdx.y picks the view,
// whose arguments sit in the kernel argument segment; the x grid is sized
// for the largest view and blocks past a view's own extent exit early.
template <typename A>
struct Batch {
    int count;
    A v[kMaxSortViews];
};

// Per-view arguments of one radix pass.  vals_in NULL means the identity
// (the item's input index); vals2_in/vals2_out (both or neither) carry a
// second value array.
struct PassArgs {
    const uint32_t *keys_in, *vals_in, *vals2_in;
    uint32_t *keys_out, *vals_out, *vals2_out;
    const uint32_t *n_ptr;       // live items
    uint32_t *n_out_ptr;         // items kept (optional)
    uint32_t *counts;            // per-digit, per-block counts [256][grid]
    uint32_t *digit_total;       // [256]
    int shift, bits;
    int key16;                   // keys stored as 16-bit (tile ids of views with <= 65536 tiles)
};

// Tile ids of views with at most 65536 tiles travel as 16-bit keys (half the
// key bytes of every tile pass); depths and larger tile ids as 32-bit.
__device__ __forceinline__ uint32_t ld_key(const uint32_t *p, size_t i, int k16)
{
    return k16 ? (uint32_t)reinterpret_cast<const uint16_t *>(p)[i] : p[i];
}
__device__ __forceinline__ void st_key(uint32_t *p, size_t i, uint32_t v, int k16)
{
    if (k16)
        reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)v;
    else
        p[i] = v;
}

__global__ __launch_bounds__(kBlock) void radix_upsweep(const Batch<PassArgs> b, int drop_sentinel)
{
    __shared__ uint32_t hist[kWaves][256];
    const PassArgs &a = b.v[blockIdx.y];
    const uint32_t *__restrict__ keys = a.keys_in;
    uint32_t *__restrict__ counts = a.counts;
    const int shift = a.shift, bits = a.bits;
    const uint32_t n = *a.n_ptr;
    uint32_t begin, end;
    chunk_of(n, begin, end);
    const uint32_t mask = (1u << bits) - 1u;
    for (int i = threadIdx.x; i < kWaves * 256; i += kBlock) (&hist[0][0])[i] = 0;
    __syncthreads();
    uint32_t *h = hist[wave_id()];
    // kIpt independent loads in flight per thread (indexes past the end are
    // clamped to the last item and not counted)
    for (uint32_t base = begin; base < end; base += kTileItems) {
        uint32_t k[kIpt];
#pragma unroll
        for (int r = 0; r < kIpt; r++) {
            const uint32_t i = base + r * kBlock + threadIdx.x;
            k[r] = ld_key(keys, i < end ? i : end - 1, a.key16);
        }
        // Lanes that share the first lane's digit (often most of the wave:
        // the high digits of depths and tiles take few values) are counted
        // with one add; the others add one each.  (Grouping the other lanes
        // by digit with one ballot per digit bit, one add per group, was
        // slower: 0.38 -> 0.60 ms of upsweeps per 8-view step at 1080p.)
#pragma unroll
        for (int r = 0; r < kIpt; r++) {
            const uint32_t i = base + r * kBlock + threadIdx.x;
            const bool valid = i < end && !(drop_sentinel && k[r] == kSentinel);
            const uint32_t d = (k[r] >> shift) & mask;
            const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
            const uint64_t same = __ballot(valid && d == d0);
            if (lane_id() == 0 && same != 0ull) atomicAdd(&h[d0], (uint32_t)__popcll(same));
            if (valid && d != d0) atomicAdd(&h[d], 1u);
        }
    }
    __syncthreads();
    const int d = threadIdx.x;   // 256 threads = 256 digits
    counts[(size_t)d * gridDim.x + blockIdx.x] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
}

// One block per digit: exclusive scan of that digit's per-block counts.
__global__ __launch_bounds__(kBlock) void radix_scan(const Batch<PassArgs> b, int G)
{
    const PassArgs &a = b.v[blockIdx.y];
    uint32_t *__restrict__ digit_total = a.digit_total;
    uint32_t *row = a.counts + (size_t)blockIdx.x * G;
    const int per = (G + kBlock - 1) / kBlock;
    const int b0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int i = 0; i < per; i++)
        if (b0 + i < G) local += row[b0 + i];
    uint32_t total;
    uint32_t run = block_exclusive_scan(local, &total);
    for (int i = 0; i < per; i++)
        if (b0 + i < G) {
            const uint32_t c = row[b0 + i];
            row[b0 + i] = run;
            run += c;
        }
    if (threadIdx.x == 0) digit_total[blockIdx.x] = total;
}

// With kTwo, the views that have a second value array carry it along.
template <bool kTwo>
__global__ __launch_bounds__(kBlock) void radix_downsweep(const Batch<PassArgs> b, int drop_sentinel)
{
    const PassArgs &a = b.v[blockIdx.y];
    const uint32_t *__restrict__ keys_in = a.keys_in;
    const uint32_t *__restrict__ vals_in = a.vals_in;
    const uint32_t *__restrict__ vals2_in = a.vals2_in;
    uint32_t *__restrict__ keys_out = a.keys_out;
    uint32_t *__restrict__ vals_out = a.vals_out;
    uint32_t *__restrict__ vals2_out = a.vals2_out;
    uint32_t *__restrict__ n_out_ptr = a.n_out_ptr;
    const uint32_t *__restrict__ counts = a.counts;
    const uint32_t *__restrict__ digit_total = a.digit_total;
    const int shift = a.shift, bits = a.bits;
    const bool two = kTwo && vals2_out != nullptr;
    __shared__ uint32_t digit_base[256];
    __shared__ uint32_t tile_start[256];
    __shared__ uint32_t tile_cnt[256];
    __shared__ uint32_t wave_cnt[kWaves][256];
    __shared__ uint32_t sk[kTileItems];
    __shared__ uint32_t sv[kTileItems];
    __shared__ uint32_t sv2[kTwo ? kTileItems : 1];
    __shared__ uint32_t s_tile_total;

    const uint32_t n = *a.n_ptr;
    uint32_t begin, end;
    chunk_of(n, begin, end);
    const uint32_t mask = (1u << bits) - 1u;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();

    {   // global start of each digit for this block
        const uint32_t t = digit_total[tid];
        uint32_t all;
        const uint32_t ex = block_exclusive_scan(t, &all);
        digit_base[tid] = ex + counts[(size_t)tid * gridDim.x + blockIdx.x];
        if (blockIdx.x == 0 && tid == 0 && n_out_ptr) *n_out_ptr = all;
    }
    __syncthreads();

    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    // The items of tile tb + kTileItems are loaded while tile tb is ranked
    // and written (indexes past the end are clamped to the last item; those
    // lanes are not ranked).
    uint32_t k[kIpt], v[kIpt], v2[kIpt];
    auto load_tile = [&](uint32_t tb, uint32_t *kk, uint32_t *vv, uint32_t *vv2) {
#pragma unroll
        for (int r = 0; r < kIpt; r++) {
            const uint32_t idx = tb + w * kWaveItems + r * kWave + lane;
            const uint32_t ci = idx < end ? idx : end - 1;
            kk[r] = ld_key(keys_in, ci, a.key16);
            vv[r] = vals_in ? vals_in[ci] : idx;
            if (two) vv2[r] = vals2_in[ci];
        }
    };
    if (begin < end) load_tile(begin, k, v, v2);
    for (uint32_t tb = begin; tb < end; tb += kTileItems) {
        uint32_t nk[kIpt], nv[kIpt], nv2[kIpt];
        const bool more = tb + kTileItems < end;
        if (more) load_tile(tb + kTileItems, nk, nv, nv2);
        for (int i = lane; i < 256; i += kWave) wave_cnt[w][i] = 0;
        // the wave's own row is written by its own lanes only; no barrier needed
        uint32_t loc[kIpt];
        bool ok[kIpt];
#pragma unroll
        for (int r = 0; r < kIpt; r++) {
            const uint32_t idx = tb + w * kWaveItems + r * kWave + lane;
            bool valid = idx < end;
            if (drop_sentinel && k[r] == kSentinel) valid = false;
            const uint32_t d = (k[r] >> shift) & mask;
            uint64_t peers = __ballot(valid);
            // one ballot per digit bit of the pass (a uniform bound)
#pragma unroll
            for (int bit = 0; bit < 8; bit++) {
                if (bit >= bits) break;
                const uint64_t bb = __ballot((d >> bit) & 1u);
                peers &= ((d >> bit) & 1u) ? bb : ~bb;
            }
            const uint32_t rank = (uint32_t)__popcll(peers & lt_mask);
            uint32_t before = 0;
            if (valid) before = wave_cnt[w][d];
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) wave_cnt[w][d] = before + (uint32_t)__popcll(peers);
            __builtin_amdgcn_wave_barrier();
            loc[r] = before + rank;
            ok[r] = valid;
        }
        __syncthreads();
        {   // per digit: exclusive prefix over waves, tile totals, tile starts
            const int d = tid;
            uint32_t run = 0;
#pragma unroll
            for (int ww = 0; ww < kWaves; ww++) {
                const uint32_t c = wave_cnt[ww][d];
                wave_cnt[ww][d] = run;
                run += c;
            }
            tile_cnt[d] = run;
            uint32_t all;
            tile_start[d] = block_exclusive_scan(run, &all);
            if (tid == 0) s_tile_total = all;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kIpt; r++) {
            if (!ok[r]) continue;
            const uint32_t d = (k[r] >> shift) & mask;
            const uint32_t pos = tile_start[d] + wave_cnt[w][d] + loc[r];
            sk[pos] = k[r];
            sv[pos] = v[r];
            if (two) sv2[pos] = v2[r];
        }
        __syncthreads();
        const uint32_t tot = s_tile_total;
        for (uint32_t i = tid; i < tot; i += kBlock) {
            const uint32_t kk = sk[i];
            const uint32_t d = (kk >> shift) & mask;
            const uint32_t o = digit_base[d] + (i - tile_start[d]);
            st_key(keys_out, o, kk, a.key16);
            vals_out[o] = sv[i];
            if (two) vals2_out[o] = sv2[i];
        }
        __syncthreads();
        digit_base[tid] += tile_cnt[tid];
        __syncthreads();
        if (more) {
#pragma unroll
            for (int r = 0; r < kIpt; r++) {
                k[r] = nk[r];
                v[r] = nv[r];
                if (two) v2[r] = nv2[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Setup: counters, empty tile ranges, depth keys of the visible Gaussians
// and, in index order, their tile rects (x0 | y0 << 16, w | h << 16), so the
// scan after the depth sort gathers 8 bytes per Gaussian instead of a record.
struct InitArgs {
    const Splat *splats;
    uint32_t n, n_ranges;
    int tiles_x, tiles_y;
    uint32_t *dkeys, *ranges, *counters;
    uint2 *grect;                // null: no rects needed (only reached tiles listed)
    int prebinned;               // depth keys and rects came from the projection
};

__global__ __launch_bounds__(kBlock) void bin_init(const Batch<InitArgs> b)
{
    const InitArgs &a = b.v[blockIdx.y];
    const Splat *__restrict__ splats = a.splats;
    const uint32_t n = a.n, n_ranges = a.n_ranges;
    uint32_t *__restrict__ dkeys = a.dkeys;
    uint32_t *__restrict__ ranges = a.ranges;
    uint32_t *__restrict__ counters = a.counters;
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < n && !a.prebinned) {
        const float4 sa = splats[i].a;
        const uint32_t tiles = __float_as_uint(splats[i].c.w);
        dkeys[i] = tiles ? __float_as_uint(sa.z) : kSentinel;   // the first pass takes i as the value
        // written for every Gaussian (culled ones get an unused value): a
        // full, coalesced row costs less than scattered partial lines
        if (a.grect) {
            uint2 gr = make_uint2(0u, 0u);
            if (tiles) gr = pack_rect(tile_rect(sa.x, sa.y, (float)__float_as_int(sa.w), (float)a.tiles_x,
                                                (float)a.tiles_y));
            a.grect[i] = gr;
        }
    }
    if (i < n_ranges) ranges[i] = 0;
    if (i == 0) {
        counters[0] = n;   // items entering the first depth pass
        counters[1] = 0;   // visible Gaussians after it
        counters[2] = 0;   // K clamped to the capacity
    }
}

// Per depth-ordered Gaussian j (256 per block): its tile rect (x0, y0 packed,
// width) and tile count for the duplication, and the block's sum of tiles
// touched.
constexpr int kScanItems = kBlock;               // Gaussians per scan / duplication block

// Per-view arguments of the slot scan and the duplication.
struct DupArgs {
    const uint2 *grect;          // tile rects by Gaussian index (bin_init or the projection)
    const uint32_t *order;       // visible Gaussians in depth order
    const uint32_t *m_ptr;       // their number
    int tiles_x, tiles_y;
    uint64_t cap;                // key capacity
    uint2 *rect_info;            // [n] the rects in depth order
    uint32_t *counts;            // [n] pairs per depth-ordered Gaussian
    uint64_t *block_sums;        // per 256 Gaussians: pairs, then their exclusive scan
    uint64_t *k_total;
    uint32_t *k_eff;             // K clamped to the capacity
    uint32_t *tile_keys, *gslot; // duplicated entries
    uint32_t *bwd_order, *bwd_off, *bwd_count;   // optional backward index parts
    int key16;                   // tile ids stored as 16-bit keys
    const Splat *splats;         // records (means and conics for the reach test)
    uint32_t *reach_mask;        // [n] reached tiles of rects up to 32 tiles, row-major bits
    int reach;                   // list only the tiles each Gaussian reaches
};

// For the reach test of a Gaussian's tiles: its conic and mean (fp64), the
// slopes of the edge vertices (dy = -b dx / c on an edge of fixed dx,
// dx = -b dy / a on an edge of fixed dy) and the largest Q at which
// o exp(-Q / 2) still reaches (1/255)(1 - 1e-3), 2 ln(255 o / (1 - 1e-3)).
// The slopes only place the point where Q is evaluated, and Q is stationary
// along the edge there, so their fp32 rounding moves Q by a second-order
// amount; the bound is formed in fp32 (error ~1e-7): a decision can differ
// from an exact one only within ~1e-7 of the bound, relative.
struct ReachG {
    double a, b, c, sx, sy, u, v, qlim;
};

__device__ __forceinline__ ReachG reach_of(const float4 &sa, const float4 &sb)
{
    ReachG r;
    r.a = sb.x;
    r.b = sb.y;
    r.c = sb.z;
    r.sx = (double)(-sb.y * __builtin_amdgcn_rcpf(sb.z));
    r.sy = (double)(-sb.y * __builtin_amdgcn_rcpf(sb.x));
    r.u = sa.x;
    r.v = sa.y;
    r.qlim = (double)(2.0f * 0.6931471805599453f *
                      __builtin_amdgcn_logf(sb.w * (255.0f / (1.0f - 1e-3f))));
    return r;
}

__device__ __forceinline__ ReachG reach_of(const Splat *__restrict__ splats, uint32_t g)
{
    return reach_of(splats[g].a, splats[g].b);
}

// Does the Gaussian reach alpha >= (1/255)(1 - 1e-3) on the box of tile
// (tx, ty)'s pixel centres, i.e. is the minimum there of
// Q(d) = a dx^2 + 2 b dx dy + c dy^2 (d = pixel centre - mean) at most qlim?
// The minimum is 0 if the box holds the mean.  Otherwise it lies on an edge
// that faces the mean (the mean outside that edge's half-plane): at a
// minimiser inside another edge, or at a corner of two others, the
// optimality condition -Q d in the box's normal cone would give d^T Q d <= 0
// with d != 0, impossible for a positive definite Q.  So at most one
// vertical and one horizontal edge are evaluated, each at its vertex clamped
// to the edge, all in fp64.  (The blend kernels apply an fp32 variant of
// the same test, with the same margin, to every entry they stage.)
__device__ __forceinline__ bool reaches(const ReachG &r, uint32_t tx, uint32_t ty)
{
    const double xl = (double)(tx * kTile) + 0.5 - r.u, xh = xl + (double)(kTile - 1);
    const double yl = (double)(ty * kTile) + 0.5 - r.v, yh = yl + (double)(kTile - 1);
    const bool out_x = xl > 0.0 || xh < 0.0, out_y = yl > 0.0 || yh < 0.0;
    double q = 0.0;
    if (out_x || out_y) {
        q = INFINITY;
        if (out_x) {
            const double dx = xl > 0.0 ? xl : xh;
            const double dy = fmin(fmax(r.sx * dx, yl), yh);
            q = fmin(q, dx * (r.a * dx + 2.0 * r.b * dy) + r.c * dy * dy);
        }
        if (out_y) {
            const double dy = yl > 0.0 ? yl : yh;
            const double dx = fmin(fmax(r.sy * dy, xl), xh);
            q = fmin(q, dx * (r.a * dx + 2.0 * r.b * dy) + r.c * dy * dy);
        }
    }
    return q <= r.qlim;
}

constexpr uint32_t kMaskTiles = 32;   // rects up to this size keep their reached tiles as bits
constexpr uint32_t kLaneTiles = 16;   // rects up to this size are tested by their own lane

// Per depth-ordered Gaussian j (256 per block): its tile rect and its number
// of pairs, and the block's sum.  A view that lists only reached tiles counts
// the tiles of the rect the Gaussian reaches: a lane tests a rect of up to 16
// tiles itself, the wave takes larger rects together (64 tiles per round),
// and rects of up to 32 tiles keep their reached tiles as a row-major bit
// mask for the duplication.
template <bool kReach>
__global__ __launch_bounds__(kBlock) void scan_reduce(const Batch<DupArgs> b)
{
    const DupArgs &a = b.v[blockIdx.y];
    const uint32_t m = *a.m_ptr;
    const uint32_t j = blockIdx.x * kScanItems + threadIdx.x;
    if (blockIdx.x * kScanItems >= m) return;
    uint32_t c = 0, g = 0;
    uint2 r = make_uint2(0u, 0u);
    float4 sa = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sb = sa;
    if (j < m) {
        g = a.order[j];
        if (kReach && a.reach) {
            // the reach test reads the record's mean and conic anyway; the
            // rect follows from them by the projection's own function (the
            // same bits), which saves gathering it
            sa = a.splats[g].a;
            sb = a.splats[g].b;
            r = pack_rect(tile_rect(sa.x, sa.y, (float)__float_as_int(sa.w), (float)a.tiles_x, (float)a.tiles_y));
        } else {
            r = a.grect[g];
        }
        c = (r.y & 0xFFFFu) * (r.y >> 16);
        a.rect_info[j] = r;
    }
    if (kReach && a.reach) {
        const uint32_t x0 = r.x & 0xFFFFu, y0 = r.x >> 16, w = r.y & 0xFFFFu, h = r.y >> 16;
        uint32_t mask = 0;
        const bool own = j < m && c <= kLaneTiles;
        if (own) {
            const ReachG rg = reach_of(sa, sb);
            uint32_t bit = 1u;
            for (uint32_t ty = y0; ty < y0 + h; ty++)
                for (uint32_t tx = x0; tx < x0 + w; tx++, bit <<= 1)
                    if (reaches(rg, tx, ty)) mask |= bit;
        }
        // the wave's larger rects, one after another, 64 tiles per round in
        // row-major order
        const int lane = threadIdx.x & (kWave - 1);
        uint64_t shared_rects = __ballot(j < m && c > kLaneTiles);
        uint32_t kept_shared = 0;
        while (shared_rects) {
            const int src = __builtin_ctzll(shared_rects);
            shared_rects &= shared_rects - 1;
            const uint32_t sg = (uint32_t)__shfl((int)g, src, kWave);
            const uint32_t sxy = (uint32_t)__shfl((int)r.x, src, kWave);
            const uint32_t swh = (uint32_t)__shfl((int)r.y, src, kWave);
            const uint32_t sw = swh & 0xFFFFu, sn = sw * (swh >> 16);
            const ReachG rg = reach_of(a.splats, sg);
            uint32_t kept = 0, first_bits = 0;
            for (uint32_t t0 = 0; t0 < sn; t0 += kWave) {
                const uint32_t t = t0 + (uint32_t)lane;
                bool k = false;
                if (t < sn) {
                    const uint32_t q = t / sw;
                    k = reaches(rg, (sxy & 0xFFFFu) + (t - q * sw), (sxy >> 16) + q);
                }
                const uint64_t bits = __ballot(k);
                if (t0 == 0) first_bits = (uint32_t)bits;
                kept += (uint32_t)__popcll(bits);
            }
            if (lane == src) {
                kept_shared = kept;
                if (sn <= kMaskTiles) mask = first_bits;
            }
        }
        if (j < m) {
            c = own ? (uint32_t)__popc(mask) : kept_shared;
            a.reach_mask[j] = mask;
        }
    }
    if (j < m) a.counts[j] = c;
    uint64_t total;
    block_exclusive_scan((uint64_t)c, &total);
    if (threadIdx.x == 0) a.block_sums[blockIdx.x] = total;
}

// Exclusive scan of the block sums (one block per view); K and the clamped
// count.  The sums go through in chunks of 1024, one per thread (coalesced
// loads and stores), each chunk scanned across the block and carried into
// the next.
__global__ __launch_bounds__(1024) void scan_blocks(const Batch<DupArgs> b)
{
    constexpr int kThreads = 1024, kW = kThreads / kWave;
    __shared__ uint64_t wsum[kW];
    const DupArgs &a = b.v[blockIdx.y];
    uint64_t *__restrict__ block_sums = a.block_sums;
    const uint64_t cap = a.cap;
    uint32_t *__restrict__ bwd_off = a.bwd_off;
    const uint32_t m = *a.m_ptr;
    const int nb = (int)((m + kScanItems - 1) / kScanItems);
    const int w = threadIdx.x / kWave;
    uint64_t carry = 0;
    for (int base = 0; base < nb; base += kThreads) {
        const int i = base + threadIdx.x;
        const uint64_t x = i < nb ? block_sums[i] : 0ull;
        const uint64_t inc = wave_inclusive_scan(x);
        if (lane_id() == kWave - 1) wsum[w] = inc;
        __syncthreads();
        uint64_t before = 0, total = 0;
#pragma unroll
        for (int j = 0; j < kW; j++) {
            if (j < w) before += wsum[j];
            total += wsum[j];
        }
        __syncthreads();
        if (i < nb) block_sums[i] = carry + before + inc - x;
        carry += total;
    }
    if (threadIdx.x == 0) {
        *a.k_total = carry;
        *a.k_eff = (uint32_t)(carry < cap ? carry : cap);
        if (bwd_off) {
            bwd_off[m] = (uint32_t)(carry < 0xFFFFFFFFull ? carry : 0xFFFFFFFFull);
            *a.bwd_count = m;
        }
    }
}

// The 256 depth-ordered Gaussians of a duplication block in LDS: the first
// pair of each within the block (exclusive scan of their pair counts), its
// Gaussian, rect and (reach views) reached-tile mask.
struct DupBlock {
    uint32_t off[kScanItems];
    uint32_t g[kScanItems];
    uint32_t xy[kScanItems];
    uint32_t wh[kScanItems];
    uint32_t mask[kScanItems];
    float inv[kScanItems];
};

// Position of the k-th set bit (k from 0) of m, which has more than k.
__device__ __forceinline__ uint32_t select_bit(uint32_t m, uint32_t k)
{
    uint32_t pos = 0;
#pragma unroll
    for (uint32_t s = 16; s > 0; s >>= 1) {
        const uint32_t low = (uint32_t)__popc(m & ((1u << s) - 1u));
        if (k >= low) {
            k -= low;
            m >>= s;
            pos += s;
        }
    }
    return pos;
}

// Each depth-ordered Gaussian writes (tile id, g) for every tile of its rect
// (or, in a reach view, every tile it reaches), row-major, at its slots.  A
// block takes 256 Gaussians, scans their counts in LDS, then hands the
// block's entries out 256 at a time: each lane finds its Gaussian by binary
// search over the block's offsets, so the work is balanced however unequal
// the rects are.  In a reach view an entry's tile is the matching set bit of
// its Gaussian's mask; rects of more than 32 tiles are left to a second
// pass in which a wave tests each of its own such rects 64 tiles at a time
// and compacts the reached ones in order with ballots.
template <bool kReach>
__global__ __launch_bounds__(kBlock) void duplicate_keys(const Batch<DupArgs> b)
{
    __shared__ DupBlock s;
    const DupArgs &a = b.v[blockIdx.y];
    const uint64_t *__restrict__ block_offsets = a.block_sums;
    const int tiles_x = a.tiles_x;
    const uint64_t cap = a.cap;
    uint32_t *__restrict__ tile_keys = a.tile_keys;
    uint32_t *__restrict__ gslot = a.gslot;
    const bool reach = kReach && a.reach != 0;
    const uint32_t m = *a.m_ptr;
    const uint32_t base = blockIdx.x * kScanItems;
    if (base >= m) return;
    const uint32_t n_items = min((uint32_t)kScanItems, m - base);
    const uint32_t j = base + threadIdx.x;
    uint32_t c = 0;
    if (threadIdx.x < n_items) {
        const uint2 ri = a.rect_info[j];
        c = a.counts[j];
        s.g[threadIdx.x] = a.order[j];
        s.xy[threadIdx.x] = ri.x;
        s.wh[threadIdx.x] = ri.y;
        s.mask[threadIdx.x] = reach ? a.reach_mask[j] : 0u;
        s.inv[threadIdx.x] = 1.0f / (float)(ri.y & 0xFFFFu);
    }
    uint32_t total;
    s.off[threadIdx.x] = block_exclusive_scan(c, &total);
    __syncthreads();
    const uint64_t blk = block_offsets[blockIdx.x];
    if (a.bwd_order && threadIdx.x < n_items) {
        // backward index: the depth-ordered Gaussians and their first slots
        const uint64_t f = blk + s.off[threadIdx.x];
        a.bwd_order[j] = s.g[threadIdx.x];
        a.bwd_off[j] = (uint32_t)(f < 0xFFFFFFFFull ? f : 0xFFFFFFFFull);
    }
    for (uint32_t e = threadIdx.x; e < total; e += kBlock) {
        const uint64_t slot = blk + e;
        if (slot >= cap) break;
        // the last li with off[li] <= e (every Gaussian with an entry here has >= 1)
        int lo = 0;
#pragma unroll
        for (int step = kScanItems / 2; step > 0; step >>= 1)
            if (lo + step < (int)n_items && s.off[lo + step] <= e) lo += step;
        const uint32_t wh = s.wh[lo], w = wh & 0xFFFFu;
        uint32_t t = e - s.off[lo];
        if (reach) {
            if (w * (wh >> 16) > kMaskTiles) continue;           // the second pass
            t = select_bit(s.mask[lo], t);
        }
        // t / w via the reciprocal, corrected to the exact quotient
        uint32_t q = (uint32_t)((float)t * s.inv[lo]);
        if (q * w > t) q--;
        else if ((q + 1) * w <= t) q++;
        const uint32_t xy = s.xy[lo];
        const uint32_t ty = (xy >> 16) + q;
        const uint32_t tx = (xy & 0xFFFFu) + (t - q * w);
        st_key(tile_keys, slot, ty * (uint32_t)tiles_x + tx, a.key16);
        gslot[slot] = s.g[lo];
    }
    if (!kReach || !reach) return;
    // rects of more than 32 tiles: the wave of their Gaussian, in order
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wh = threadIdx.x < n_items ? s.wh[threadIdx.x] : 0u;
    uint64_t large = __ballot(threadIdx.x < n_items && (wh & 0xFFFFu) * (wh >> 16) > kMaskTiles);
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    while (large) {
        const int src = __builtin_ctzll(large);
        large &= large - 1;
        const int li = (int)(threadIdx.x & ~(kWave - 1)) + src;
        const uint32_t sxy = s.xy[li], swh = s.wh[li], sg = s.g[li];
        const uint32_t sw = swh & 0xFFFFu, sn = sw * (swh >> 16);
        const ReachG rg = reach_of(a.splats, sg);
        uint64_t slot0 = blk + s.off[li];
        for (uint32_t t0 = 0; t0 < sn; t0 += kWave) {
            const uint32_t t = t0 + (uint32_t)lane;
            bool k = false;
            uint32_t tx = 0, ty = 0;
            if (t < sn) {
                const uint32_t q = t / sw;
                tx = (sxy & 0xFFFFu) + (t - q * sw);
                ty = (sxy >> 16) + q;
                k = reaches(rg, tx, ty);
            }
            const uint64_t bits = __ballot(k);
            const uint64_t slot = slot0 + (uint64_t)__popcll(bits & lt);
            if (k && slot < cap) {
                st_key(tile_keys, slot, ty * (uint32_t)tiles_x + tx, a.key16);
                gslot[slot] = sg;
            }
            slot0 += (uint64_t)__popcll(bits);
        }
    }
}

// Tile ranges from the boundaries of the sorted tile ids and the optional
// 64-bit keys.  Without tile passes (a one-tile image) the duplication order
// is final: the entries' Gaussians are copied from gslot and their slots are
// the identity.
struct RangeArgs {
    const uint32_t *tile_keys;   // sorted tile ids
    const uint32_t *k_ptr;       // K clamped to the capacity
    const Splat *splats;
    const uint32_t *gslot;       // without tile passes: the duplication order's Gaussians
    uint32_t *ranges, *vals, *entry_slots;
    uint64_t *keys64;
    int key16;                   // tile ids stored as 16-bit keys
};

// Each thread takes kRangeItems consecutive entries (one 16-byte load of
// 16-bit tile ids when the run is whole) and writes the boundaries between
// them and the entry before: the start of the tile at position p and the end
// of the tile at p - 1 wherever the ids at p - 1 and p differ.
constexpr int kRangeItems = 8;

__global__ __launch_bounds__(kBlock) void tile_ranges_kernel(const Batch<RangeArgs> b)
{
    const RangeArgs &a = b.v[blockIdx.y];
    const uint32_t *__restrict__ tile_keys = a.tile_keys;
    const Splat *__restrict__ splats = a.splats;
    const uint32_t *__restrict__ gslot = a.gslot;
    uint32_t *__restrict__ ranges = a.ranges;
    uint32_t *__restrict__ vals = a.vals;
    uint32_t *__restrict__ entry_slots = a.entry_slots;
    uint64_t *__restrict__ keys64 = a.keys64;
    const uint32_t k = *a.k_ptr;
    const uint64_t i64 = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * kRangeItems;
    if (i64 >= k) return;
    const uint32_t i0 = (uint32_t)i64;
    const uint32_t n = k - i0 < (uint32_t)kRangeItems ? k - i0 : (uint32_t)kRangeItems;
    const int k16 = a.key16;
    uint32_t t[kRangeItems];
    if (k16 && n == (uint32_t)kRangeItems) {
        // i0 is a multiple of 8, so the 16 bytes are aligned
        const uint4 w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(tile_keys) + i0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            t[2 * j] = ws[j] & 0xFFFFu;
            t[2 * j + 1] = ws[j] >> 16;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kRangeItems; j++) t[j] = (uint32_t)j < n ? ld_key(tile_keys, i0 + j, k16) : 0u;
    }
    uint32_t prev = i0 == 0 ? 0u : ld_key(tile_keys, i0 - 1, k16);
#pragma unroll
    for (int j = 0; j < kRangeItems; j++) {
        if ((uint32_t)j >= n) break;
        const uint32_t p = i0 + j;
        if (p == 0) {
            ranges[2 * t[j]] = 0;
        } else if (t[j] != prev) {
            ranges[2 * t[j]] = p;
            ranges[2 * prev + 1] = p;
        }
        prev = t[j];
    }
    if (i0 + n == k) ranges[2 * prev + 1] = k;
    for (uint32_t j = 0; j < n; j++) {
        const uint32_t p = i0 + j;
        uint32_t g = 0;
        if (gslot) {
            g = gslot[p];
            vals[p] = g;
            if (entry_slots) entry_slots[p] = p;
        } else if (keys64) {
            g = vals[p];
        }
        if (keys64) keys64[p] = ((uint64_t)t[j] << 32) | __float_as_uint(splats[g].a.z);
    }
}

// Tile schedule for the blend kernels.  Per-tile work varies by two orders
// of magnitude (list lengths 1 .. ~3000 at 1080p) and the blend puts every
// tile of a view in flight at once, so a static tile -> wave mapping leaves
// the busiest SIMD with ~2x the mean load.  One block buckets the tiles by
// list length (~1.4x wide buckets, longest first, empty tiles last); the
// blend kernels pull tiles from a counter in that order (longest-processing-
// time-first list scheduling).  The schedule is order[n_tiles] followed by
// two counter pairs (forward, backward), zeroed here and reset by the last
// wave of each blend launch.
constexpr int kSchedBins = 66;
constexpr int kSchedThreads = 1024;

__device__ __forceinline__ int length_bin(uint32_t L)
{
    if (L == 0) return 0;
    const int lg = 31 - __clz(L);                  // floor(log2 L)
    const int half = lg > 0 ? (int)((L >> (lg - 1)) & 1u) : 0;
    return 1 + 2 * lg + half;
}

struct SchedArgs {
    const uint32_t *ranges;
    int n_tiles;
    uint32_t *sched;
    uint64_t *k_total;           // for a view without Gaussians: K = 0 is written here
    uint32_t *bwd_tail;          // and here its backward index's K and visible count (0, 0)
};

__global__ __launch_bounds__(kSchedThreads) void schedule_tiles(const Batch<SchedArgs> b)
{
    const SchedArgs &a = b.v[blockIdx.y];
    const uint32_t *__restrict__ ranges = a.ranges;
    const int n_tiles = a.n_tiles;
    uint32_t *__restrict__ sched = a.sched;
    if (a.k_total != nullptr && threadIdx.x == 0) *a.k_total = 0;
    if (a.bwd_tail != nullptr && threadIdx.x < 2) a.bwd_tail[threadIdx.x] = 0;
    __shared__ uint32_t hist[kSchedBins];
    __shared__ uint32_t base[kSchedBins];
    const int tid = threadIdx.x;
    if (tid < kSchedBins) hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < n_tiles; t += kSchedThreads)
        atomicAdd(&hist[length_bin(ranges[2 * t + 1] - ranges[2 * t])], 1u);
    __syncthreads();
    if (tid == 0) {
        uint32_t run = 0;
        for (int b = kSchedBins - 1; b >= 0; b--) {
            base[b] = run;
            run += hist[b];
        }
    }
    if (tid < 4) sched[n_tiles + tid] = 0;
    __syncthreads();
    for (int t = tid; t < n_tiles; t += kSchedThreads) {
        const int b = length_bin(ranges[2 * t + 1] - ranges[2 * t]);
        sched[atomicAdd(&base[b], 1u)] = (uint32_t)t;
    }
}

// ---------------------------------------------------------------------------
// Workspace carving (also run on a null base to size the workspace, so the
// addresses are formed as integers: no pointer arithmetic on null).
struct Carve {
    char *p;
    size_t off = 0;
    template <typename T>
    T *take(size_t count)
    {
        off = align_up(off, 256);
        T *r = (T *)((uintptr_t)p + off);
        off += count * sizeof(T);
        return r;
    }
};

int radix_grid(uint64_t max_items)
{
    uint64_t g = (max_items + kTileItems - 1) / kTileItems;
    if (g < 1) g = 1;
    if (g > kMaxGrid) g = kMaxGrid;
    return (int)g;
}

int bits_for(uint32_t count)
{
    int b = 0;
    while ((1ull << b) < count) b++;
    return b;
}

struct BinWs {
    uint32_t *dk[2], *dv[2];           // depth sort ping-pong [n]
    uint2 *grect;                      // [n] tile rect by Gaussian index
    uint2 *rect_info;                  // [n] per depth-ordered Gaussian
    uint32_t *counts;                  // [n] tiles touched (or reached), depth order
    uint32_t *reach_mask;              // [n] reached tiles of small rects, depth order
    uint64_t *block_sums;              // [ceil(n / 256)]
    uint32_t *tk[2], *tv[2], *ts[2];   // tile keys, Gaussians, slots ping-pong [cap]
    uint32_t *gslot;                   // [cap] Gaussian of each duplication slot
    uint32_t *digit_counts;            // [256 * kMaxGrid]
    uint32_t *digit_total;             // [256]
    uint32_t *counters;                // [4]
};

size_t carve_bin(char *base, int64_t n, int64_t cap, BinWs *ws)
{
    Carve c{base};
    const size_t nn = (size_t)(n > 0 ? n : 1), kk = (size_t)(cap > 0 ? cap : 1);
    BinWs w;
    w.dk[0] = c.take<uint32_t>(nn);
    w.dv[0] = c.take<uint32_t>(nn);
    w.dk[1] = c.take<uint32_t>(nn);
    w.dv[1] = c.take<uint32_t>(nn);
    w.grect = c.take<uint2>(nn);
    w.rect_info = c.take<uint2>(nn);
    w.counts = c.take<uint32_t>(nn);
    w.reach_mask = c.take<uint32_t>(nn);
    w.block_sums = c.take<uint64_t>((nn + kScanItems - 1) / kScanItems);
    w.tk[0] = c.take<uint32_t>(kk);
    w.tk[1] = c.take<uint32_t>(kk);
    w.tv[0] = c.take<uint32_t>(kk);
    w.tv[1] = c.take<uint32_t>(kk);
    w.ts[0] = c.take<uint32_t>(kk);
    w.ts[1] = c.take<uint32_t>(kk);
    w.gslot = c.take<uint32_t>(kk);
    w.digit_counts = c.take<uint32_t>(256 * kMaxGrid);
    w.digit_total = c.take<uint32_t>(256);
    w.counters = c.take<uint32_t>(4);
    if (ws) *ws = w;
    return c.off + 256;
}

// One stable pass over the views of a batch (grid: G blocks per view).
hipError_t radix_pass(const Batch<PassArgs> &b, int G, int drop, bool two, hipStream_t s)
{
    radix_upsweep<<<dim3(G, b.count), kBlock, 0, s>>>(b, drop);
    radix_scan<<<dim3(256, b.count), kBlock, 0, s>>>(b, G);
    if (two)
        radix_downsweep<true><<<dim3(G, b.count), kBlock, 0, s>>>(b, drop);
    else
        radix_downsweep<false><<<dim3(G, b.count), kBlock, 0, s>>>(b, drop);
    return hipGetLastError();
}

}  // namespace

size_t bin_sort_workspace(int64_t n, int64_t k_capacity, int n_tiles)
{
    (void)n_tiles;
    return carve_bin(nullptr, n, k_capacity, nullptr);
}

// The views of a batch go through every step together, one launch per step
// (blockIdx.y = view), so small views still fill the device.
hipError_t launch_bin_sort_views(int count, const SortJob *jobs, hipStream_t s)
{
    if (count < 1 || count > kMaxSortViews) return hipErrorInvalidValue;
    hipError_t e;
    BinWs w[kMaxSortViews];
    uint32_t n_max = 0, init_max = 0, tbits_max = 0;
    uint64_t cap_max = 0;
    bool any_bwd = false;
    for (int v = 0; v < count; v++) {
        const SortJob &J = jobs[v];
        carve_bin((char *)J.ws, J.n, J.cap, &w[v]);
        const uint32_t n = (uint32_t)J.n;
        const uint32_t n_ranges = 2u * (uint32_t)(J.cam.tiles_x * J.cam.tiles_y);
        n_max = n > n_max ? n : n_max;
        if (J.dkeys == nullptr) init_max = n > init_max ? n : init_max;
        init_max = n_ranges > init_max ? n_ranges : init_max;
        const uint32_t tb = (uint32_t)bits_for((uint32_t)(J.cam.tiles_x * J.cam.tiles_y));
        tbits_max = tb > tbits_max ? tb : tbits_max;
        cap_max = (uint64_t)J.cap > cap_max ? (uint64_t)J.cap : cap_max;
        any_bwd = any_bwd || J.bwd_index != nullptr;
    }

    {   // counters, empty ranges, depth keys and rects (unless the projection wrote them)
        Batch<InitArgs> b;
        b.count = count;
        for (int v = 0; v < count; v++) {
            const SortJob &J = jobs[v];
            b.v[v] = InitArgs{J.splats, (uint32_t)J.n, 2u * (uint32_t)(J.cam.tiles_x * J.cam.tiles_y),
                              J.cam.tiles_x, J.cam.tiles_y, w[v].dk[0], J.ranges, w[v].counters,
                              J.reach ? nullptr : w[v].grect, J.dkeys != nullptr ? 1 : 0};
        }
        bin_init<<<dim3((init_max + kBlock - 1) / kBlock, count), kBlock, 0, s>>>(b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // the views with Gaussians go through the sort; the others have K = 0
    int live[kMaxSortViews], n_live = 0;
    for (int v = 0; v < count; v++)
        if (jobs[v].n > 0) live[n_live++] = v;

    if (n_live > 0) {
        // 1. depth: 4 x 8-bit passes over the Gaussians; the first drops the
        // culled ones
        int cur = 0;
        for (int pass = 0; pass < 4; pass++) {
            Batch<PassArgs> b;
            b.count = n_live;
            for (int i = 0; i < n_live; i++) {
                const BinWs &W = w[live[i]];
                const uint32_t *kin = pass == 0 && jobs[live[i]].dkeys ? jobs[live[i]].dkeys : W.dk[cur];
                b.v[i] = PassArgs{kin, pass == 0 ? nullptr : W.dv[cur], nullptr, W.dk[cur ^ 1], W.dv[cur ^ 1],
                                  nullptr,
                                  pass == 0 ? &W.counters[0] : &W.counters[1], &W.counters[1],
                                  W.digit_counts, W.digit_total, 8 * pass, 8};
            }
            if ((e = radix_pass(b, radix_grid(n_max), pass == 0, false, s)) != hipSuccess) return e;
            cur ^= 1;
        }

        // 2. slots and duplication (K clamped to the capacity in counters[2])
        const int key16 = tbits_max <= 16 ? 1 : 0;
        Batch<DupArgs> d;
        d.count = n_live;
        bool any_reach = false;
        for (int i = 0; i < n_live; i++) {
            const SortJob &J = jobs[live[i]];
            const BinWs &W = w[live[i]];
            const size_t n = (size_t)J.n, cap = (size_t)J.cap;
            // backward index: [entry slot: cap][depth-ordered Gaussian: n][first slot: n + 1][visible count]
            uint32_t *bi = J.bwd_index;
            d.v[i] = DupArgs{J.grect ? J.grect : W.grect, W.dv[cur], &W.counters[1], J.cam.tiles_x, J.cam.tiles_y, (uint64_t)J.cap,
                             W.rect_info, W.counts, W.block_sums, J.k_total, &W.counters[2], W.tk[0], W.gslot,
                             bi ? bi + cap : nullptr, bi ? bi + cap + n : nullptr,
                             bi ? bi + cap + 2 * n + 1 : nullptr, key16, J.splats, W.reach_mask, J.reach ? 1 : 0};
            any_reach = any_reach || J.reach;
        }
        const uint32_t nblk = (n_max + kScanItems - 1) / kScanItems;
        if (any_reach) scan_reduce<true><<<dim3(nblk, n_live), kBlock, 0, s>>>(d);
        else scan_reduce<false><<<dim3(nblk, n_live), kBlock, 0, s>>>(d);
        scan_blocks<<<dim3(1, n_live), 1024, 0, s>>>(d);
        if (any_reach) duplicate_keys<true><<<dim3(nblk, n_live), kBlock, 0, s>>>(d);
        else duplicate_keys<false><<<dim3(nblk, n_live), kBlock, 0, s>>>(d);
        if ((e = hipGetLastError()) != hipSuccess) return e;

        // 3. tile passes over the tile ids, carrying each entry's Gaussian
        // and, for the backward index, its duplication slot (the identity on
        // the way in); the last pass writes straight into the outputs.  A
        // view with fewer tile bits than the batch's widest takes zero-bit
        // passes (a stable copy).
        const int passes = tbits_max == 0 ? 0 : ((int)tbits_max + 7) / 8;
        for (int p = 0; p < passes; p++) {
            const bool last = p == passes - 1;
            Batch<PassArgs> b;
            b.count = n_live;
            for (int i = 0; i < n_live; i++) {
                const SortJob &J = jobs[live[i]];
                const BinWs &W = w[live[i]];
                // the view's tile bits split as evenly as the passes allow
                // (13 bits: 7 + 6, not 8 + 5: longer digit runs, fuller
                // writes in the first pass)
                const int tbits = bits_for((uint32_t)(J.cam.tiles_x * J.cam.tiles_y));
                const int base_bits = tbits / passes, extra = tbits % passes;
                const int bits = base_bits + (p < extra ? 1 : 0);
                const int shift = p * base_bits + (p < extra ? p : extra);
                const uint32_t *gin = p == 0 ? W.gslot : W.tv[(p - 1) & 1];
                uint32_t *gout = last ? J.vals : W.tv[p & 1];
                uint32_t *entry_slots = J.bwd_index;                  // [cap], optional
                if (entry_slots) {
                    const uint32_t *sin = p == 0 ? nullptr : W.ts[(p - 1) & 1];
                    uint32_t *sout = last ? entry_slots : W.ts[p & 1];
                    b.v[i] = PassArgs{W.tk[p & 1], sin, gin, W.tk[(p + 1) & 1], sout, gout, &W.counters[2],
                                      nullptr, W.digit_counts, W.digit_total, shift, bits, key16};
                } else {
                    b.v[i] = PassArgs{W.tk[p & 1], gin, nullptr, W.tk[(p + 1) & 1], gout, nullptr,
                                      &W.counters[2], nullptr, W.digit_counts, W.digit_total, shift, bits, key16};
                }
            }
            if ((e = radix_pass(b, radix_grid(cap_max), 0, any_bwd, s)) != hipSuccess) return e;
        }

        // 4. ranges and the optional 64-bit keys
        Batch<RangeArgs> r;
        r.count = n_live;
        for (int i = 0; i < n_live; i++) {
            const SortJob &J = jobs[live[i]];
            const BinWs &W = w[live[i]];
            r.v[i] = RangeArgs{W.tk[passes & 1], &W.counters[2], J.splats, passes == 0 ? W.gslot : nullptr,
                               J.ranges, J.vals, J.bwd_index, J.keys, key16};
        }
        const uint64_t per_block = (uint64_t)kBlock * kRangeItems;
        const uint64_t kgrid = (cap_max + per_block - 1) / per_block;
        if (kgrid > 0) tile_ranges_kernel<<<dim3((unsigned)kgrid, n_live), kBlock, 0, s>>>(r);
    }

    // 5. longest-first tile schedule for the blend kernels
    Batch<SchedArgs> sb;
    sb.count = count;
    for (int v = 0; v < count; v++) {
        const SortJob &J = jobs[v];
        const bool empty = J.n == 0;
        sb.v[v] = SchedArgs{J.ranges, J.cam.tiles_x * J.cam.tiles_y, J.schedule, empty ? J.k_total : nullptr,
                            empty && J.bwd_index ? J.bwd_index + J.cap : nullptr};
    }
    schedule_tiles<<<dim3(1, count), kSchedThreads, 0, s>>>(sb);
    return hipGetLastError();
}

size_t schedule_words(int n_tiles) { return (size_t)n_tiles + 4; }

}  // namespace gsi
