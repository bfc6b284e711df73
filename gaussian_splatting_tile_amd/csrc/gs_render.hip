// Per-pixel alpha compositing, forward and backward (gfx950).
//
// One wave64 per 16x16 tile, four pixels per lane: lane l owns column
// l & 15 and rows (l >> 4) + 4 r, r = 0..3.  The tile's depth-sorted list is
// consumed in batches of 64 records: each lane gathers one record into LDS
// (the on-chip caching of intermediate results that the "Gsplat" section of
// the pixel-diffusion page prescribes), then every lane walks the batch from
// LDS with broadcast reads.  The four pixels of a lane share their column, so
// the x-offset terms of the quadratic form are computed once per record and
// the LDS reads and loop control are spread over four pixels.  A tile is one
// wave, so no block barrier is ever needed beyond the LDS fill.
//
// Rules (readings; the pages name tiled alpha blending but give no formula):
//   alpha = min(0.99, o exp(-1/2 d^T conic d)),  d = mean - pixel centre
//   an entry with alpha < 1/255 is skipped;
//   a pixel stops at the first entry it meets with T < 1e-4 (the entry that
//   took T below 1e-4 was composited);
//   C = sum alpha_i T_i rgb_i,  image = C + T_final bg.
//
// Before a batch is walked, each lane tests the record it staged against the
// whole tile: if the minimum of the conic's quadratic form over the box of
// the tile's pixel centres still leaves o exp(power) below 1/255 (with a
// margin far above the arithmetic error), no pixel of the tile can composite
// it, and the record is dropped from the batch by a ballot compaction.  The
// binning's square 3-sigma rects make ~40 % of a tile's list such records.
// Outputs are unchanged: a dropped record would have been skipped by every
// pixel, and list positions (n_contrib) are kept with each staged record.
//
// The exponent's quadratic form is evaluated in fp64: for thin Gaussians
// seen far along their major axis its three terms reach ~1e5 and cancel to a
// result of order 1, so any fp32 evaluation carries an exponent error near
// 1e-3; in fp64 it is exact to ~1e-11, and on this chip an fp64 FMA issues
// at the rate of a non-packed fp32 one.  The forward and the backward
// evaluate exp(power) with the same sequence of operations, so the backward
// retraces the forward's skip decisions exactly.
#include "gs_internal.h"

namespace gsi {
namespace {

constexpr int kLanes = 64;                   // one wave per tile
constexpr int kPx = 4;                       // pixels per lane
constexpr int kBatch = kLanes;               // records staged per batch
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTMin = 1e-4f;

// Tiles come from the longest-first schedule built by the binning: order[T]
// followed by a (head, done) counter pair per kernel.  Persistent waves take
// the next tile index from `head`; the last wave to finish resets both
// counters, so the next launch on the stream starts from zero again.
// (the item index is made wave-uniform, so per-view fields are read with
// scalar loads)
__device__ __forceinline__ int next_item(uint32_t *head, int n_items)
{
    uint32_t i = 0;
    if (threadIdx.x == 0) i = atomicAdd(head, 1u);
    i = __builtin_amdgcn_readfirstlane(i);
    return i < (uint32_t)n_items ? (int)i : -1;
}

__device__ __forceinline__ void retire_wave(uint32_t *head, uint32_t *done)
{
    if (threadIdx.x == 0) {
        // every wave's last head increment precedes its done increment, so the
        // last wave to get here knows no head increment is still to come
        if (atomicAdd(done, 1u) == gridDim.x - 1) {
            atomicExch(head, 0u);
            atomicExch(done, 0u);
        }
    }
}

// A staged record: the exponent in exp2 form with the opacity folded in,
//   o exp(power) = exp2(log2 o + qa dx^2 + qb dx dy + qc dy^2),
//   (qa, qb, qc) = -log2(e) (a/2, b, c/2),
// kept in fp64 together with the mean; the colour stays fp32.
__device__ __forceinline__ void stage_record(const Splat &s, double2 &uv, double4 &q, float4 &rgb)
{
    const double l = -(double)kLog2e;
    uv = make_double2((double)s.a.x, (double)s.a.y);
    q = make_double4(0.5 * l * (double)s.b.x, l * (double)s.b.y, 0.5 * l * (double)s.b.z,
                     (double)__builtin_amdgcn_logf(s.b.w));
    rgb = make_float4(s.c.x, s.c.y, s.c.z, s.b.w);
}

// The strips of a tile whose pixel rows lie within the vertical reach of a
// record: for a fixed dy, Q(dx, dy) is smallest at dx = -b dy / a, where it
// equals dy^2 det / a (det = ac - b^2), so a pixel of that row can reach
// alpha >= 1/255 only if dy^2 <= 2 ln(255 o) a / det.  The bound is widened
// by the relative margin of 1e-3 on alpha that box_may_contribute uses, far
// above the error of the per-pixel evaluation, so a strip outside it holds no
// pixel that could take the record, and the blend skips pixel r of every
// lane for a record whose bit r is clear.  Strip r covers rows 4 r .. 4 r + 3
// of the tile (the rows a lane's pixel r covers across the wave).  The test
// ignores the tile's columns: weaker than a box test per strip, at a
// fraction of the cost (four box tests per staged record took the forward
// blend from 1.77 to 1.90 ms per 8 views at 1080p).
__device__ __forceinline__ uint32_t strips_in_reach(float fv, const float4 &conic_o, int y0)
{
    const double a = conic_o.x, b = conic_o.y, c = conic_o.z;
    const double det = a * c - b * b;
    if (!(det > 0.0) || !(a > 0.0)) return 0xFu;
    // 2 ln(255 o / (1 - 1e-3)), through log2 in fp32 (error ~1e-7, inside the margin)
    const float lim = 2.0f * 0.6931471805599453f * __builtin_amdgcn_logf(conic_o.w * (255.0f / (1.0f - 1e-3f)));
    if (!(lim > 0.0f)) return 0u;
    const double ext = sqrt((double)lim * a / det);
    const double lo = (double)fv - ext, hi = (double)fv + ext;
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const double ylo = (double)(y0 + 4 * r) + 0.5;
        if (hi >= ylo && lo <= ylo + 3.0) m |= 1u << r;
    }
    return m;
}

// Per record and column: the dx terms shared by the lane's four pixels.
// Contraction is off and the one fused step is an explicit fma, so the
// forward and the backward evaluate the same operations wherever the
// compiler inlines this.
struct ColTerms { double dx, a0, bdx; };

__device__ __forceinline__ ColTerms col_terms(const double2 &uv, const double4 &q, double px)
{
#pragma clang fp contract(off)
    ColTerms c;
    c.dx = uv.x - px;                 // exact: difference of two floats
    c.a0 = fma(q.x * c.dx, c.dx, q.w);
    c.bdx = q.y * c.dx;
    return c;
}

// o exp(power) at one pixel of the column, dy = v - py.  A lane's pixels sit
// at rows y0 + 4 r, so dy = (v - (y0 + 1/2)) - 4 r: both steps are exact in
// fp64 (v is a float, the rest small integers and halves).
__device__ __forceinline__ float alpha_raw(const ColTerms &c, double qc, double dy)
{
    const double e = fma(dy, fma(qc, dy, c.bdx), c.a0);
    return __builtin_amdgcn_exp2f((float)e);
}

// The backward writes all nine partial sums of every entry of a tile's list,
// zeros where the entry cannot reach any pixel that uses it.
__device__ __forceinline__ void zero_partial(float *__restrict__ partial, uint32_t entry_slot)
{
    float *p = partial + (size_t)entry_slot * 9;
#pragma unroll
    for (int q = 0; q < 9; q++) p[q] = 0.0f;
}

// A record fetched into registers ahead of its staging (software
// pipelining of the blend's global gathers across batches).
struct Fetched {
    uint32_t m;          // list position
    uint32_t g;          // Gaussian
    bool valid;
    float4 a, b, c;
};

__device__ __forceinline__ void fetch_record(const Splat *__restrict__ splats, uint32_t g, bool valid, Fetched &f)
{
    f.g = g;
    if (valid) {
        f.a = splats[g].a;
        f.b = splats[g].b;
        f.c = splats[g].c;
    }
}

// One record staged for the forward blend.  The whole wave reads the same
// record at once (LDS broadcast); keeping its fields together lets one
// address serve all five reads, at immediate offsets.
struct FwdRec {
    double2 uv;                   // mean
    double2 q01, q23;             // the exponent's terms, log2 o
    float4 rgb;                   // colour, opacity
    uint4 meta;                   // 1 + list position, strip mask, Gaussian, -
};
static_assert(sizeof(FwdRec) == 80, "five 16-byte LDS reads per record");

// Stage the fetched records of one batch into LDS with their strip masks
// (and, with kWeight, their Gaussians), dropping those that cannot reach a
// pixel of the tile that is still compositing; returns the number kept, in
// order.
template <bool kWeight>
__device__ __forceinline__ int stage_fetched(const Fetched &f, uint32_t start, int x0, int y0, uint32_t live,
                                             bool tile_test, FwdRec *s_rec)
{
    const int lane = threadIdx.x;
    // the cheap test first: most records that fail, fail it; strips whose
    // pixels have all stopped stay stopped, so they are left out here too.
    // Lists of reached tiles have passed the tile test in the sort.
    uint32_t strips = f.valid ? strips_in_reach(f.a.y, f.b, y0) & live : 0u;
    if (tile_test && strips != 0u && !box_may_contribute(f.a.x, f.a.y, f.b, x0, y0, kTile - 1, kTile - 1))
        strips = 0u;
    const bool keep = strips != 0u;
    const uint64_t mask = __ballot(keep);
    if (keep) {
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int slot = __popcll(mask & lt);
        Splat s;
        s.a = f.a;
        s.b = f.b;
        s.c = f.c;
        double2 uv;
        double4 q;
        float4 rgb;
        stage_record(s, uv, q, rgb);
        FwdRec &r = s_rec[slot];
        r.uv = uv;
        r.q01 = make_double2(q.x, q.y);
        r.q23 = make_double2(q.z, q.w);
        r.rgb = rgb;
        r.meta = make_uint4(f.m - start + 1u, strips, kWeight ? f.g : 0u, 0u);
    }
    return __popcll(mask);
}

// One record staged for the blend backward; as in the forward, the whole
// wave reads one record at once from one address, at immediate offsets.
struct BwdRec {
    double4 q;                    // the exponent's terms, log2 o
    double2 uv;                   // mean
    float4 rgb;                   // colour, 1 / opacity
    float4 P;                     // -P = -L V^T (the conic's principal frame)
    uint4 meta;                   // list position, duplication slot, strips in reach, -
};
static_assert(sizeof(BwdRec) == 96, "six 16-byte LDS reads per record");

// The backward's staging of fetched records: the strips in reach (left out:
// strips whose pixels all composited fewer entries than the record's list
// position) and the tile test, plus the entry's duplication slot and the
// principal frame of its conic; a dropped entry gets its nine partial sums
// zeroed.
__device__ __forceinline__ int stage_fetched_bwd(const Fetched &f, uint32_t entry_slot, uint32_t start, int x0,
                                                 int y0, const uint32_t lrow[4], bool tile_test, BwdRec *s_rec,
                                                 float *__restrict__ partial)
{
    const int lane = threadIdx.x;
    // strips in reach whose pixels composited entries at or past this one
    // (lists of reached tiles have passed the tile test in the sort)
    uint32_t alive = 0;
#pragma unroll
    for (int r = 0; r < 4; r++) alive |= (f.m - start < lrow[r] ? 1u : 0u) << r;
    const uint32_t strips = f.valid ? strips_in_reach(f.a.y, f.b, y0) & alive : 0u;
    const bool keep = strips != 0u &&
                      (!tile_test || box_may_contribute(f.a.x, f.a.y, f.b, x0, y0, kTile - 1, kTile - 1));
    if (f.valid && !keep) zero_partial(partial, entry_slot);
    const uint64_t mask = __ballot(keep);
    if (keep) {
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int slot = __popcll(mask & lt);
        Splat s;
        s.a = f.a;
        s.b = f.b;
        s.c = f.c;
        BwdRec &r = s_rec[slot];
        float4 rgb;
        stage_record(s, r.uv, r.q, rgb);
        // dL/do is a sum of dL/dalpha alpha / o: divided once per record
        r.rgb = make_float4(rgb.x, rgb.y, rgb.z, __builtin_amdgcn_rcpf(rgb.w));
        r.meta = make_uint4(f.m - start, entry_slot, strips, 0u);
        // -w' = -P d with P = L V^T (rows: l1 (ex, ey), l2 (-ey, ex)), stored
        // negated: the wave then sums -W1, -W2 directly (the products in
        // W11, W12, W22 do not change sign); formed in fp64, kept in fp32
        double ex, ey, l1, l2;
        conic_frame(s.b.x, s.b.y, s.b.z, ex, ey, l1, l2);
        r.P = make_float4((float)(-(l1 * ex)), (float)(-(l1 * ey)), (float)(l2 * ey), (float)(-(l2 * ex)));
    }
    return __popcll(mask);
}

// (every control used here reads a valid lane; old = 0 with bound_ctrl lets
// the compiler fold the move into the add that consumes it)
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    const int iv = __float_as_int(v);
    return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, kCtrl, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowRor8 = 0x128;     // row_ror:8 (lane i <- (i + 8) mod 16)
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror (lane i <- 7 - i within 8)

// Split exchange across lanes i and i ^ 32 (i ^ 16): lanes of the lower half
// (even rows) return a[i] + a[partner], lanes of the upper half (odd rows)
// b[i] + b[partner].  v_permlane32_swap / v_permlane16_swap swap the upper
// half of the first operand with the lower half of the second, so the sum of
// the two results is exactly that.
__device__ __forceinline__ float xchg32(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xchg16(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of one value over the wave, in every lane: quad, 8-lane and 16-lane
// steps on DPP moves folded into the adds, then the 32- and 64-lane steps on
// lane swaps.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppRowRor8>(v);
    v = xchg16(v, v);
    return xchg32(v, v);
}

// Bit r set while some lane's pixel r (strip r of the tile) has not stopped.
__device__ __forceinline__ uint32_t live_strips(const float T[4])
{
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; r++)
        if (__ballot(T[r] >= kTMin) != 0ull) m |= 1u << r;
    return m;
}

// Persistent waves take work items from one queue over the views of the
// batch: item i is view i mod V, the (i div V)-th tile of that view's
// longest-first order, so the views' long tiles come first together and one
// view's tail overlaps the others' work.
// With kWeight, each record's blending weights over the wave's pixels are
// summed across the wave and added to its Gaussian's entry of the view's
// weight array (views without one skip it).
template <bool kWeight>
__global__ __launch_bounds__(kLanes) void render_fwd_kernel(const FwdBatch batch)
{
    __shared__ FwdRec s_rec[kBatch];

    const int lane = threadIdx.x;
    const int n_items = batch.count * batch.max_tiles;
    uint32_t *head = batch.queue, *done = batch.queue + 1;
    for (int item = next_item(head, n_items); item >= 0; item = next_item(head, n_items)) {
        const int vi = item % batch.count;
        const FwdView &V = batch.v[vi];
        const Cam &cam = V.cam;
        const int n_tiles = cam.tiles_x * cam.tiles_y;
        const int rank = item / batch.count;
        if (rank >= n_tiles) continue;
        const int tile = (int)V.order[rank];
        const Splat *__restrict__ splats = V.splats;
        const uint32_t *__restrict__ vals = V.vals;
        const uint32_t *__restrict__ ranges = V.ranges;
        float *__restrict__ image = V.image;
        float *__restrict__ final_T = V.final_T;
        uint32_t *__restrict__ n_contrib = V.n_contrib;
        const float bg0 = batch.bg[0], bg1 = batch.bg[1], bg2 = batch.bg[2];
        const size_t hw = (size_t)cam.width * cam.height;
        const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
        const int x = tx * kTile + (lane & 15);
        const int y0 = ty * kTile + (lane >> 4);
        const double px = (double)x + 0.5;

        // A pixel is live while T >= 1e-4; pixels outside the image start at
        // T = 0 and never composite.
        const double py0 = (double)y0 + 0.5;
        float T[kPx], c0[kPx], c1[kPx], c2[kPx];
        uint32_t last[kPx];
#pragma unroll
        for (int r = 0; r < kPx; r++) {
            const int y = y0 + 4 * r;
            T[r] = (x < cam.width && y < cam.height) ? 1.0f : 0.0f;
            c0[r] = c1[r] = c2[r] = 0.0f;
            last[r] = 0;
        }

        const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
        // Two-stage pipeline over the batches: while batch i is blended, the
        // records of batch i + 1 and the list entries of batch i + 2 are in
        // flight.
        Fetched cur;
        cur.m = start + lane;
        cur.valid = cur.m < end;
        fetch_record(splats, cur.valid ? vals[cur.m] : 0u, cur.valid, cur);
        uint32_t next_m = start + kBatch + lane;
        bool next_valid = next_m < end;
        uint32_t next_g = next_valid ? vals[next_m] : 0u;
        for (uint32_t b0 = start; b0 < end; b0 += kBatch) {
            // strips whose pixels have all stopped, once per batch: testing
            // again every 8 (16, 32) records inside the batch cost more than
            // it saved (forward blend 1.46 ms per 8 views at 1080p against
            // 1.51, 1.48, 1.48)
            const uint32_t live = live_strips(T);
            if (live == 0u) break;
            const int nb = stage_fetched<kWeight>(cur, start, tx * kTile, ty * kTile, live, V.tile_test != 0, s_rec);
            cur.m = next_m;
            cur.valid = next_valid;
            fetch_record(splats, next_g, next_valid, cur);
            next_m += kBatch;
            next_valid = next_m < end;
            next_g = next_valid ? vals[next_m] : 0u;
            __syncthreads();
            for (int k = 0; k < nb; k++) {
                const FwdRec &R = s_rec[k];
                const double2 uv = R.uv;
                const double2 q01 = R.q01, q23 = R.q23;
                const double4 q = make_double4(q01.x, q01.y, q23.x, q23.y);
                const float4 rgb = R.rgb;
                const uint4 meta = R.meta;
                const uint32_t pos = meta.x;         // what n_contrib records
                // wave-uniform: the branches below are scalar; a strip whose
                // pixels had all stopped when the batch began is skipped too
                const uint32_t strips = __builtin_amdgcn_readfirstlane(meta.y) & live;
                const ColTerms ct = col_terms(uv, q, px);
                const double dy0 = uv.y - py0;
                float wsum = 0.0f;
#pragma unroll
                for (int r = 0; r < kPx; r++) {
                    if (!((strips >> r) & 1u)) continue;
                    const float raw = alpha_raw(ct, q.z, dy0 - 4.0 * r);
                    const bool take = T[r] >= kTMin && raw >= kAlphaMin;
                    const float alpha = take ? fminf(kAlphaMax, raw) : 0.0f;
                    const float w = alpha * T[r];
                    c0[r] = fmaf(rgb.x, w, c0[r]);
                    c1[r] = fmaf(rgb.y, w, c1[r]);
                    c2[r] = fmaf(rgb.z, w, c2[r]);
                    // T (1 - alpha) with one rounding: T - w would round
                    // alpha T first, an error of up to 50 ulp of the result
                    // at alpha = 0.99, which the backward's recovery of T
                    // by division then carries to every entry in front
                    T[r] = fmaf(-alpha, T[r], T[r]);
                    last[r] = take ? pos : last[r];
                    if (kWeight) wsum += w;
                }
                if (kWeight && V.weight != nullptr && __ballot(wsum > 0.0f) != 0ull) {
                    wsum = wave_sum(wsum);
                    if (lane == 0) atomicAdd(V.weight + meta.z, wsum);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < kPx; r++) {
            const int y = y0 + 4 * r;
            if (x < cam.width && y < cam.height) {
                const size_t p = (size_t)y * cam.width + x;
                image[p] = c0[r] + T[r] * bg0;
                image[hw + p] = c1[r] + T[r] * bg1;
                image[2 * hw + p] = c2[r] + T[r] * bg2;
                final_T[p] = T[r];
                n_contrib[p] = last[r];
            }
        }
    }
    retire_wave(head, done);
}

// ---------------------------------------------------------------------------
// Backward.  Per pixel, walk the composited entries back to front:
//   T_i = T_{i+1} / (1 - alpha_i)                (T before entry i)
//   A   = colour of everything behind entry i, normalised by T_{i+1}
//         (A starts at bg and A <- alpha_i rgb_i + (1 - alpha_i) A); only
//         <A, G> is needed, so that scalar is carried
//   dL/drgb_i   = alpha_i T_i G
//   dL/dalpha_i = T_i (<rgb_i, G> - <A, G>)
//   below the cap: dL/do = exp(power) dL/dalpha, dL/dpower = alpha dL/dalpha
//   power = -1/2 d^T Q d, d = (u - px, v - py), Q = Sigma'^-1 = [[a, b], [b, c]]:
//     with w = Q d:  d/d(u, v) = -w,  d/dSigma' = Q (d d^T / 2) Q = w w^T / 2.
// The gradient goes to the dilated 2D covariance Sigma', expressed in the
// principal frame V of Q (Q = V L V^T): w' = V^T w = L V^T d.  For a thin
// Gaussian Q's eigenvalues differ by up to ~1e4; summed as conic gradients
// or in image axes, fp32 rounding of the large-eigenvalue direction would
// swamp the small one after the change of variables.  In the principal
// frame each direction keeps its own relative precision.  P = L V^T is formed
// per record in fp64 and kept in fp32, w' = P d per pixel in fp32 (its two
// terms cancel by at most the square root of the eigenvalue ratio); a lane
// accumulates, over
// its pixels with dp = dL/dpower,
//   W1 = sum dp w'_1,  W2 = sum dp w'_2,  W11, W12, W22 = sum dp w' w'^T.
// The 9 per-lane values of a record, (-W1, -W2, W11, W12, W22, dL/do,
// dL/drgb), are then summed over the wave by a split
// butterfly on VALU lane swaps and DPP moves (each exchange halves the values
// a lane carries) and nine lanes store the totals at the record's
// duplication slot, partial[slot][9]: every (Gaussian, tile) pair owns one
// slot, the slots of a Gaussian are contiguous, and the projection backward
// sums them (halving the three second moments: d/dSigma' = w w^T / 2).  No
// atomics, so the gradients are bit-reproducible.

// Wave sums of v[0..8] by a split butterfly: each exchange halves the values
// a lane carries (9 -> 5 -> 3 -> 2 -> 1), then two plain steps finish.
// Lane 0, 4, 8, 16, 20, 32, 36, 40, 48 returns the total of value
// 0, 1, 2, 3, 4, 5, 6, 7, 8 (see reduce_slot).
__device__ __forceinline__ float wave_reduce9(const float v[9], int lane)
{
    float s[5];
#pragma unroll
    for (int i = 0; i < 4; i++) s[i] = xchg32(v[i], v[i + 5]);       // lanes >= 32 keep v[5..8]
    s[4] = xchg32(v[4], v[4]);
    const float n0 = xchg16(s[0], s[3]);                              // odd rows keep s3, s4
    const float n1 = xchg16(s[1], s[4]);
    const float n2 = xchg16(s[2], s[2]);
    bool hi = (lane & 8) != 0;                                        // i ^ 8: 3 -> 2
    const float m0 = (hi ? n2 : n0) + dpp_f<kDppRowRor8>(hi ? n0 : n2);
    const float m1 = n1 + dpp_f<kDppRowRor8>(n1);
    hi = (lane & 4) != 0;                                             // i ^ 7 within 8: 2 -> 1
    float f = (hi ? m1 : m0) + dpp_f<kDppHalfMirror>(hi ? m0 : m1);
    f += dpp_f<kDppQuadXor2>(f);
    f += dpp_f<kDppQuadXor1>(f);
    return f;
}

// The lanes where c holds, kept in scalar registers: tests of it are then
// scalar compares (a branch on the ballot itself is emitted as a vector
// select and compare per test).
__device__ __forceinline__ uint64_t lanes_where(bool c)
{
    uint64_t m = __builtin_amdgcn_ballot_w64(c);
    asm volatile("" : "+s"(m));
    return m;
}

// Which of the nine totals lane L holds after wave_reduce9, or -1.
__device__ __forceinline__ int reduce_slot(int lane)
{
    switch (lane) {
    case 0: return 0;
    case 4: return 1;
    case 8: return 2;
    case 16: return 3;
    case 20: return 4;
    case 32: return 5;
    case 36: return 6;
    case 40: return 7;
    case 48: return 8;
    default: return -1;
    }
}

// Work items as in the forward: one queue over the views of the batch.
__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(5))) void render_bwd_kernel(
    const BwdBatch batch)
{
    __shared__ BwdRec s_rec[kBatch];

    const int lane = threadIdx.x;
    const int slot = reduce_slot(lane);
    const int n_items = batch.count * batch.max_tiles;
    uint32_t *head = batch.queue, *done = batch.queue + 1;
    for (int item = next_item(head, n_items); item >= 0; item = next_item(head, n_items)) {
    const int vi = batch.view_major ? item / batch.max_tiles : item % batch.count;
    const BwdView &V = batch.v[vi];
    const Cam &cam = V.cam;
    const int n_tiles = cam.tiles_x * cam.tiles_y;
    const int rank = batch.view_major ? item % batch.max_tiles : item / batch.count;
    if (rank >= n_tiles) continue;
    const int tile = (int)V.order[rank];
    const Splat *__restrict__ splats = V.splats;
    const uint32_t *__restrict__ vals = V.vals;
    const uint32_t *__restrict__ ranges = V.ranges;
    const uint32_t *__restrict__ entry_slots = V.entry_slots;
    const float *__restrict__ final_T = V.final_T;
    const uint32_t *__restrict__ n_contrib = V.n_contrib;
    const float *__restrict__ dL_dimage = V.dL_dimage;
    float *__restrict__ partial = V.partial;
    const float bg0 = batch.bg[0], bg1 = batch.bg[1], bg2 = batch.bg[2];
    const size_t hw = (size_t)cam.width * cam.height;
    const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
    const int x = tx * kTile + (lane & 15);
    const int y0 = ty * kTile + (lane >> 4);
    const double px = (double)x + 0.5;

    const double py0 = (double)y0 + 0.5;
    float T[kPx], G0[kPx], G1[kPx], G2[kPx], AG[kPx];
    uint32_t last[kPx];
    uint32_t lmax = 0;
#pragma unroll
    for (int r = 0; r < kPx; r++) {
        const int y = y0 + 4 * r;
        T[r] = 1.0f;
        G0[r] = G1[r] = G2[r] = 0.0f;
        last[r] = 0;
        if (x < cam.width && y < cam.height) {
            const size_t p = (size_t)y * cam.width + x;
            T[r] = final_T[p];
            last[r] = n_contrib[p];
            G0[r] = dL_dimage[p];
            G1[r] = dL_dimage[hw + p];
            G2[r] = dL_dimage[2 * hw + p];
        }
        AG[r] = bg0 * G0[r] + bg1 * G1[r] + bg2 * G2[r];
    }
    // per strip, the largest number of entries a pixel composited: entries
    // at or past it cannot be taken by any pixel of the strip
    uint32_t lrow[kPx];
#pragma unroll
    for (int r = 0; r < kPx; r++) {
        uint32_t l = last[r];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) l = max(l, (uint32_t)__shfl_xor((int)l, off, 64));
        lrow[r] = __builtin_amdgcn_readfirstlane(l);
        lmax = max(lmax, lrow[r]);
    }

    const uint32_t start = ranges[2 * tile];
    const uint32_t stop = start + lmax;           // entries at or past this are unused
    // Batches back to front, pipelined as in the forward: while batch i is
    // processed, the records of batch i + 1 and the list entries (and slots)
    // of batch i + 2 are in flight.  Batch j covers [bend_j - 64, bend_j),
    // clipped at start.
    Fetched cur;
    uint32_t cur_slot = 0;
    {
        const int64_t m = (int64_t)stop - kBatch + lane;
        cur.valid = m >= (int64_t)start && m < (int64_t)stop;
        cur.m = cur.valid ? (uint32_t)m : 0u;
        uint32_t g = 0;
        if (cur.valid) {
            g = vals[cur.m];
            cur_slot = entry_slots[cur.m];
        }
        fetch_record(splats, g, cur.valid, cur);
    }
    int64_t next_m = (int64_t)stop - 2 * kBatch + lane;
    bool next_valid = next_m >= (int64_t)start && next_m < (int64_t)stop;
    uint32_t next_g = next_valid ? vals[(uint32_t)next_m] : 0u;
    uint32_t next_slot = next_valid ? entry_slots[(uint32_t)next_m] : 0u;
    for (int64_t bend = (int64_t)stop; bend > (int64_t)start; bend -= kBatch) {
        const int nb = stage_fetched_bwd(cur, cur_slot, start, tx * kTile, ty * kTile, lrow, V.tile_test != 0,
                                         s_rec, partial);
        cur.m = next_valid ? (uint32_t)next_m : 0u;
        cur.valid = next_valid;
        cur_slot = next_slot;
        fetch_record(splats, next_g, next_valid, cur);
        next_m -= kBatch;
        next_valid = next_m >= (int64_t)start && next_m < (int64_t)stop;
        next_g = next_valid ? vals[(uint32_t)next_m] : 0u;
        next_slot = next_valid ? entry_slots[(uint32_t)next_m] : 0u;
        __syncthreads();
        for (int k = nb - 1; k >= 0; k--) {
            const BwdRec &rec = s_rec[k];
            const uint32_t pos = __builtin_amdgcn_readfirstlane(rec.meta.x);   // list position
            const uint32_t strips = __builtin_amdgcn_readfirstlane(rec.meta.z);
            const double2 uv = rec.uv;
            const double4 q = rec.q;
            const ColTerms ct = col_terms(uv, q, px);
            const double dy0 = uv.y - py0;
            float raws[kPx];
            bool take[kPx];
            uint64_t rows[kPx];
#pragma unroll
            for (int r = 0; r < kPx; r++) {
                // a strip out of the record's reach, or past every pixel's
                // last entry, is not evaluated (scalar branch)
                raws[r] = 0.0f;
                take[r] = false;
                rows[r] = 0ull;
                if (((strips >> r) & 1u) && pos < lrow[r]) {
                    raws[r] = alpha_raw(ct, q.z, dy0 - 4.0 * r);
                    take[r] = pos < last[r] && raws[r] >= kAlphaMin;
                    rows[r] = lanes_where(pos < last[r]) & lanes_where(raws[r] >= kAlphaMin);
                }
            }
            // an entry no pixel of the tile uses gets zeros
            float tot = 0.0f;
            if ((rows[0] | rows[1] | rows[2] | rows[3]) != 0ull) {
                const float4 col = rec.rgb;
                // -w' = -P d per pixel in fp32: in the principal frame the terms
                // cancel by at most the square root of the conic's eigenvalue
                // ratio (~1e2), so fp32 keeps ~1e-5 relative accuracy
                const float4 P = rec.P;
                const float fdx = (float)ct.dx, fdy0 = (float)dy0;
                const float p1y = P.y, p2y = P.w;
                // w' at the lane's first row; a row 4 r further down adds -4 r (p1y, p2y)
                const float w10 = fmaf(p1y, fdy0, P.x * fdx), w20 = fmaf(p2y, fdy0, P.z * fdx);
                float go = 0.0f, g6 = 0.0f, g7 = 0.0f, g8 = 0.0f;
                float W1 = 0.0f, W2 = 0.0f, W11 = 0.0f, W12 = 0.0f, W22 = 0.0f;
#pragma unroll
                for (int r = 0; r < kPx; r++) {
                    // rows the wave skips as a whole; in the others the
                    // lanes that do not take the entry see alpha = 0, which
                    // leaves T and <A, G> as they are and adds nothing
                    if (rows[r] == 0ull) continue;
                    const float raw = take[r] ? raws[r] : 0.0f;
                    // min(0.99, raw) in one instruction (raw is finite: an exp2)
                    const float alpha = __builtin_amdgcn_fmed3f(raw, kAlphaMax, -3.0e38f);
                    const float one_m = 1.0f - alpha;
                    T[r] = T[r] * __builtin_amdgcn_rcpf(one_m);
                    const float w = alpha * T[r];
                    g6 = fmaf(w, G0[r], g6);
                    g7 = fmaf(w, G1[r], g7);
                    g8 = fmaf(w, G2[r], g8);
                    const float cg = fmaf(col.z, G2[r], fmaf(col.y, G1[r], col.x * G0[r]));
                    const float diff = cg - AG[r];
                    const float dla = T[r] * diff;
                    // alpha cg + (1 - alpha) AG, formed from the difference above
                    AG[r] = fmaf(alpha, diff, AG[r]);
                    // at the cap alpha does not depend on o or the power: no
                    // gradient through them (a select, not a branch)
                    const float dlc = raw < kAlphaMax ? dla : 0.0f;
                    go = fmaf(dlc, raw, go);                           // times 1/o once per record
                    const float dp = dlc * alpha;
                    const float w1 = r == 0 ? w10 : fmaf(p1y, -4.0f * r, w10);
                    const float w2 = r == 0 ? w20 : fmaf(p2y, -4.0f * r, w20);
                    const float t1 = dp * w1, t2 = dp * w2;
                    W1 += t1;
                    W2 += t2;
                    W11 = fmaf(t1, w1, W11);
                    W12 = fmaf(t1, w2, W12);
                    W22 = fmaf(t2, w2, W22);
                }
                float v[9];
                v[0] = W1;                                         // -W1, -W2 (P is negated)
                v[1] = W2;
                v[2] = W11;                                        // halved by the Gaussian's sum
                v[3] = W12;
                v[4] = W22;
                v[5] = go * col.w;
                v[6] = g6;
                v[7] = g7;
                v[8] = g8;
                tot = wave_reduce9(v, lane);
            }
            if (slot >= 0) partial[(size_t)rec.meta.y * 9 + slot] = tot;
        }
        __syncthreads();
    }
    // entries past the last one any pixel used
    const uint32_t end = ranges[2 * tile + 1];
    for (uint32_t m = stop + lane; m < end; m += kLanes) zero_partial(partial, entry_slots[m]);
    }
    retire_wave(head, done);
}

}  // namespace

// Persistent grid: as many one-wave blocks as fit on the device at once.
template <typename K>
int resident_blocks(K kernel, int n_tiles)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return n_tiles;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return n_tiles;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kLanes, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long long g = (long long)cus * per_cu;
    return (int)(g < n_tiles ? g : n_tiles);
}

hipError_t launch_render_fwd(const FwdBatch &batch, hipStream_t s)
{
    bool weights = false;
    for (int i = 0; i < batch.count; i++) weights = weights || batch.v[i].weight != nullptr;
    if (weights) {
        const int grid = resident_blocks(render_fwd_kernel<true>, batch.count * batch.max_tiles);
        render_fwd_kernel<true><<<grid, kLanes, 0, s>>>(batch);
    } else {
        const int grid = resident_blocks(render_fwd_kernel<false>, batch.count * batch.max_tiles);
        render_fwd_kernel<false><<<grid, kLanes, 0, s>>>(batch);
    }
    return hipGetLastError();
}

// The backward interleaves the views' tiles (as the forward does) while a
// view has few tiles per resident wave, where one view's tail would idle the
// device; with many (4K views: ~6 per wave) it runs the views one after
// another, so the records and list entries it gathers come from one view at a
// time and stay in the last-level cache (10M/4K: 18.5 -> 17.4 ms per 8 views;
// at 1080p the interleaved order is 5 % faster).
hipError_t launch_render_bwd(const BwdBatch &batch, hipStream_t s)
{
    const int grid = resident_blocks(render_bwd_kernel, batch.count * batch.max_tiles);
    BwdBatch b = batch;
    b.view_major = batch.max_tiles >= 4 * grid ? 1 : 0;
    render_bwd_kernel<<<grid, kLanes, 0, s>>>(b);
    return hipGetLastError();
}

}  // namespace gsi
