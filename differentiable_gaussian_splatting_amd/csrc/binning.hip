// binning.hip -- tile-intersection counting and the (tile, depth, slot)
// ordered lists of one leaf.
//
// BoundedGS page, "01": raster buffers grow with the overlaps of Gaussians
// and image tiles.  Design (MI355X), two levels:
//   - once per view the candidates are sorted by depth (stable LSD radix on
//     the f32 depth bits over slots in ascending order), giving the order
//     (depth, slot) that every tile list must follow, and the per-tile
//     candidate counts of the whole grid come from a 2D difference array
//     and a 2D prefix.  The difference array is built one row at a time
//     without global atomics: the rectangles' corners are bucketed by row
//     (per-block row counts, their scan, a scatter), then one workgroup per
//     row adds its corners in LDS and writes the row;
//   - a leaf's tile offsets are the exclusive scan of those counts over the
//     leaf's tiles (row-major inside the leaf);
//   - coarse level: the leaf is covered by the image-aligned super-tiles of
//     8 x 8 tiles that meet it (those on its border are partial); the leaf's
//     candidates, in depth order, emit one (super-tile, slot) pair per
//     super-tile their rectangle meets inside the leaf (load-balanced, coalesced writes at
//     offsets from an exclusive scan), and a stable radix sort on the
//     super-tile id groups them with the depth order kept;
//   - fine level: one workgroup per super-tile, each wavefront owning 2 x 8
//     of its tiles, walks the super-tile's group 64 entries at a time; for
//     each tile a ballot over the 64 rectangles gives the entries that cover
//     it, which are appended in order at the tile's offset (the rank of an
//     entry is the number of set ballot bits below its lane).
// Every tile list therefore comes out in (depth, slot) order, and the number
// of entries written to a tile equals its count from the difference array.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

constexpr int kBorderLds = 4096;

__global__ __launch_bounds__(256) void k_rect_diff(int64_t n, const uint32_t* __restrict__ list,
                                                   const int4* __restrict__ rect, int ltx0, int lty0, int ltx1,
                                                   int lty1, int32_t* __restrict__ diff)
{
    __shared__ int32_t col0[kBorderLds];   // cells (y, 0)
    __shared__ int32_t row0[kBorderLds];   // cells (0, x)
    const int TWL = ltx1 - ltx0, THL = lty1 - lty0;
    const bool lds = TWL <= kBorderLds && THL <= kBorderLds;
    if (lds) {
        for (int k = threadIdx.x; k < THL; k += blockDim.x) col0[k] = 0;
        for (int k = threadIdx.x; k < TWL; k += blockDim.x) row0[k] = 0;
        __syncthreads();
    }
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) {
        const int64_t j = list ? (int64_t)list[k] : k;
        const int4 r = rect[j];
        const int x0 = max(r.x, ltx0) - ltx0, x1 = min(r.z, ltx1) - ltx0;
        const int y0 = max(r.y, lty0) - lty0, y1 = min(r.w, lty1) - lty0;
        if (x0 < x1 && y0 < y1) {
            auto add = [&](int y, int x, int v) {
                if (lds && x == 0) atomicAdd(&col0[y], v);
                else if (lds && y == 0) atomicAdd(&row0[x], v);
                else atomicAdd(&diff[(int64_t)y * TWL + x], v);
            };
            add(y0, x0, 1);
            if (x1 < TWL) add(y0, x1, -1);
            if (y1 < THL) add(y1, x0, -1);
            if (x1 < TWL && y1 < THL) add(y1, x1, 1);
        }
    }
    if (lds) {
        __syncthreads();
        for (int q = threadIdx.x; q < THL; q += blockDim.x)
            if (col0[q]) atomicAdd(&diff[(int64_t)q * TWL], col0[q]);
        for (int q = threadIdx.x; q < TWL; q += blockDim.x)
            if (row0[q]) atomicAdd(&diff[q], row0[q]);
    }
}

// ---- difference array by rows, without global atomics -------------------
// Scattered integer atomics on device memory are slow (each one a separate
// memory-side operation), so the corners of the rectangles (+1 at (y0, x0)
// and (y1, x1), -1 at (y0, x1) and (y1, x0), those on the far edge dropped)
// are bucketed by grid row instead: per-block row counts (kRowRects
// rectangles per block), an exclusive scan of them in row-major order (row,
// block), a scatter of one u32 record per corner (x << 1 | negative) to its
// row's bucket, and one workgroup per row that adds its records into an LDS
// copy of the row and writes the row.
constexpr int kRowRects = 4096;    // rectangles per block of the bucketing passes
constexpr int kRowsMax = 8192;     // grid rows (LDS counters of the bucketing passes)
constexpr int kRowCellsMax = 16384; // grid columns (LDS row of the summing pass)

template <typename Fn>
__device__ __forceinline__ void leaf_corners(int4 r, int ltx0, int lty0, int ltx1, int lty1, Fn&& fn)
{
    const int TWL = ltx1 - ltx0, THL = lty1 - lty0;
    const int x0 = max(r.x, ltx0) - ltx0, x1 = min(r.z, ltx1) - ltx0;
    const int y0 = max(r.y, lty0) - lty0, y1 = min(r.w, lty1) - lty0;
    if (!(x0 < x1 && y0 < y1)) return;
    fn(y0, x0, 0u);
    if (x1 < TWL) fn(y0, x1, 1u);
    if (y1 < THL) {
        fn(y1, x0, 1u);
        if (x1 < TWL) fn(y1, x1, 0u);
    }
}

// hist[row * nblk + block] = corners of the block's rectangles in that row
__global__ __launch_bounds__(256) void k_row_hist(int64_t n, const int4* __restrict__ rect, int ltx0, int lty0,
                                                  int ltx1, int lty1, uint32_t* __restrict__ hist)
{
    __shared__ uint32_t cnt[kRowsMax];
    const int THL = lty1 - lty0;
    for (int y = threadIdx.x; y < THL; y += blockDim.x) cnt[y] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRowRects;
    const int64_t lim = min<int64_t>(n - base, kRowRects);
    for (int k = threadIdx.x; k < lim; k += blockDim.x)
        leaf_corners(rect[base + k], ltx0, lty0, ltx1, lty1, [&](int y, int, uint32_t) { atomicAdd(&cnt[y], 1u); });
    __syncthreads();
    for (int y = threadIdx.x; y < THL; y += blockDim.x) hist[(int64_t)y * gridDim.x + blockIdx.x] = cnt[y];
}

// the same blocks write their corner records at the scanned offsets
__global__ __launch_bounds__(256) void k_row_scatter(int64_t n, const int4* __restrict__ rect, int ltx0, int lty0,
                                                     int ltx1, int lty1, const uint32_t* __restrict__ off,
                                                     uint32_t* __restrict__ rec)
{
    __shared__ uint32_t pos[kRowsMax];
    const int THL = lty1 - lty0;
    for (int y = threadIdx.x; y < THL; y += blockDim.x) pos[y] = off[(int64_t)y * gridDim.x + blockIdx.x];
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRowRects;
    const int64_t lim = min<int64_t>(n - base, kRowRects);
    for (int k = threadIdx.x; k < lim; k += blockDim.x)
        leaf_corners(rect[base + k], ltx0, lty0, ltx1, lty1, [&](int y, int x, uint32_t neg) {
            rec[atomicAdd(&pos[y], 1u)] = ((uint32_t)x << 1) | neg;
        });
}

// one workgroup per row: its records [off[row * nblk], off[(row + 1) * nblk])
__global__ __launch_bounds__(256) void k_row_sum(const uint32_t* __restrict__ off, int nblk,
                                                 const uint32_t* __restrict__ rec, int TWL,
                                                 int32_t* __restrict__ diff)
{
    extern __shared__ int32_t row[];
    const int y = blockIdx.x;
    for (int x = threadIdx.x; x < TWL; x += blockDim.x) row[x] = 0;
    __syncthreads();
    const int64_t r0 = off[(int64_t)y * nblk], r1 = off[(int64_t)(y + 1) * nblk];
    constexpr int U = 8;   // independent loads in flight per thread
    const int64_t B = blockDim.x;
    int64_t k = r0 + threadIdx.x;
    for (; k + (U - 1) * B < r1; k += U * B) {
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = rec[k + u * B];
#pragma unroll
        for (int u = 0; u < U; ++u) atomicAdd(&row[v[u] >> 1], (v[u] & 1u) ? -1 : 1);
    }
    for (; k < r1; k += B) {
        const uint32_t v = rec[k];
        atomicAdd(&row[v >> 1], (v & 1u) ? -1 : 1);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < TWL; x += blockDim.x) diff[(int64_t)y * TWL + x] = row[x];
}

// The same difference array for a grid that fits in LDS (few tiles, so
// heavily contended cells): a block takes kDiffBlock rectangles into an LDS
// copy of the whole grid and then adds its nonzero cells to the global grid.
constexpr int kDiffBlock = 8192;
constexpr int kDiffLds = 16384;    // cells (64 KB)

__global__ __launch_bounds__(256) void k_rect_diff_lds(int64_t n, const uint32_t* __restrict__ list,
                                                       const int4* __restrict__ rect, int ltx0, int lty0, int ltx1,
                                                       int lty1, int32_t* __restrict__ diff)
{
    extern __shared__ int32_t hd[];
    const int TWL = ltx1 - ltx0, THL = lty1 - lty0;
    const int64_t cells = (int64_t)TWL * THL;
    for (int64_t k = threadIdx.x; k < cells; k += blockDim.x) hd[k] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * kDiffBlock;
    for (int64_t k = c0 + threadIdx.x; k < min<int64_t>(n, c0 + kDiffBlock); k += blockDim.x) {
        const int64_t j = list ? (int64_t)list[k] : k;
        const int4 r = rect[j];
        const int x0 = max(r.x, ltx0) - ltx0, x1 = min(r.z, ltx1) - ltx0;
        const int y0 = max(r.y, lty0) - lty0, y1 = min(r.w, lty1) - lty0;
        if (x0 < x1 && y0 < y1) {
            atomicAdd(&hd[(int64_t)y0 * TWL + x0], 1);
            if (x1 < TWL) atomicAdd(&hd[(int64_t)y0 * TWL + x1], -1);
            if (y1 < THL) atomicAdd(&hd[(int64_t)y1 * TWL + x0], -1);
            if (x1 < TWL && y1 < THL) atomicAdd(&hd[(int64_t)y1 * TWL + x1], 1);
        }
    }
    __syncthreads();
    for (int64_t k = threadIdx.x; k < cells; k += blockDim.x)
        if (hd[k]) atomicAdd(&diff[k], hd[k]);
}

// Super-cells (image-aligned blocks of 2^sh x 2^sh tiles) that the rectangle
// r meets inside the leaf: first cell (cx0, cy0) relative to the leaf's first
// super-cell, and extent (w, h); w = h = 0 when r misses the leaf.
struct Cells {
    int cx0, cy0, w, h;
};

__device__ __forceinline__ Cells leaf_cells(int4 r, int ltx0, int lty0, int ltx1, int lty1, int sh)
{
    const int x0 = max(r.x, ltx0), x1 = min(r.z, ltx1);
    const int y0 = max(r.y, lty0), y1 = min(r.w, lty1);
    Cells c{0, 0, 0, 0};
    if (x0 < x1 && y0 < y1) {
        c.cx0 = (x0 >> sh) - (ltx0 >> sh);
        c.cy0 = (y0 >> sh) - (lty0 >> sh);
        c.w = ((x1 - 1) >> sh) - (x0 >> sh) + 1;
        c.h = ((y1 - 1) >> sh) - (y0 >> sh) + 1;
    }
    return c;
}

// super-tiles of the leaf that each listed candidate's rectangle meets
// (list: positions in the depth order, NULL: all of them)
__global__ __launch_bounds__(256) void k_count_cells(int64_t n, const uint32_t* __restrict__ list,
                                                     const uint2* __restrict__ rect_d, int ltx0, int lty0, int ltx1,
                                                     int lty1, int sh, uint32_t* __restrict__ cnt)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const Cells c = leaf_cells(gsd::rect_unpack(rect_d[list ? list[k] : (uint32_t)k]), ltx0, lty0, ltx1, lty1, sh);
    cnt[k] = (uint32_t)(c.w * c.h);
}

// per-tile counts of the leaf, row-major inside the leaf, gathered from the
// counts of the whole grid
__global__ __launch_bounds__(256) void k_leaf_counts(const int32_t* __restrict__ grid, int TW, int ltx0, int lty0,
                                                     int TWL, int64_t n_tiles, uint32_t* __restrict__ out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_tiles) return;
    out[t] = (uint32_t)grid[(int64_t)(lty0 + t / TWL) * TW + ltx0 + t % TWL];
}

// coarse keys (kCellBits) carry the entry's rectangle inside its super-tile
// through the sort, for the fine level and the group-walking raster

// (super-tile, slot) pairs of the listed candidates, in list order and
// row-major super-tile order within a rectangle.  The list holds positions in
// the depth order (NULL: every position), so a candidate's slot and packed
// rectangle are read at its position in order and rect_d, near-contiguously
// for an ascending list.  eoff[k] - ebase is the
// first output of candidate k (exclusive scan of the per-candidate super-tile
// counts, n + 1 entries, ascending).  A block writes kEO consecutive outputs,
// so that one candidate with many super-tiles does not hold up a block:
//   - its first candidate (the last k with eoff[k] - ebase <= first output)
//     comes from a 256-ary search over eoff, three rounds of loads for up to
//     2^24 candidates;
//   - the offsets of the next kEO + 1 candidates are loaded (every listed
//     candidate meets the leaf, so no more can overlap the block's outputs),
//     and the slots and rectangles of those that start before the block's
//     last output are staged in LDS;
//   - each candidate whose outputs start inside the block marks that
//     position with its index, and a prefix maximum over the positions gives
//     every output its candidate;
//   - thread t writes outputs 4t .. 4t + 3 of the block.
// The super-cell row of output t of a candidate spanning w columns is t / w,
// from the f32 reciprocal of w with one correction (t < 2^23).  Outputs past
// the staged candidates (only if some candidate had no output) fall back to a
// binary search in eoff.
constexpr int kEO = 1024;          // outputs per emission block (4 per thread)

__device__ __forceinline__ int wave_prefix_max(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v = max(v, u);
    }
    return v;
}

// First candidate of every emission block (bst[b]: the candidate whose
// outputs hold output b kEO), written by the candidates whose output ranges
// cross a block start; every block start has exactly one such candidate.
__global__ __launch_bounds__(256) void k_emit_starts(int64_t n, const uint32_t* __restrict__ eoff, uint32_t ebase,
                                                     uint32_t* __restrict__ bst)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const uint64_t a = eoff[k] - ebase, b = eoff[k + 1] - ebase;
    for (uint64_t m = (a + kEO - 1) / kEO; m * kEO < b; ++m) bst[m] = (uint32_t)k;
}

__global__ __launch_bounds__(256) void k_emit_pairs(int64_t n, const uint32_t* __restrict__ list,
                                                    const uint32_t* __restrict__ order,
                                                    const uint2* __restrict__ rect_d, int ltx0, int lty0, int ltx1,
                                                    int lty1, int sh, int SW, const uint32_t* __restrict__ eoff,
                                                    uint32_t ebase, uint32_t total, const uint32_t* __restrict__ bst,
                                                    uint32_t* __restrict__ keys, uint32_t* __restrict__ vals)
{
    __shared__ uint32_t se[kEO + 2];
    __shared__ uint32_t sj[kEO + 1];   // slot of each staged candidate
    __shared__ uint2 sr[kEO + 1];      // its rectangle, packed (its super-cells follow per output)
    __shared__ int owner[kEO];         // candidate whose outputs start at this position, else -1
    __shared__ int wred[4];
    __shared__ int64_t s_lo;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t ob = blockIdx.x * (uint32_t)kEO;
    const uint32_t oe = min(ob + (uint32_t)kEO, total);
    // ---- first candidate: the last k with eoff[k] - ebase <= ob, from bst
    // or by a 256-ary search
    int64_t lo = bst ? (int64_t)bst[blockIdx.x] : 0, len = bst ? 1 : n;
    while (len > 1) {
        const int64_t st = (len + 255) / 256;
        const int64_t idx = lo + (int64_t)tid * st;
        const bool le = idx < lo + len && eoff[idx] - ebase <= ob;
        const uint64_t bm = gsd::ballot(le);
        if (lane == 0) wred[wave] = __popcll(bm);
        __syncthreads();
        const int64_t cnt = (int64_t)wred[0] + wred[1] + wred[2] + wred[3];   // >= 1: eoff[lo] - ebase <= ob
        __syncthreads();
        const int64_t nlo = lo + (cnt - 1) * st;
        len = min(st, lo + len - nlo);
        lo = nlo;
    }
    if (!bst) {
        if (tid == 0) s_lo = lo;
        __syncthreads();
        lo = s_lo;
    }
    const int64_t k0 = lo;
    const int nmax = (int)min<int64_t>(kEO + 1, n - k0);
    for (int i = tid; i <= nmax; i += 256) se[i] = eoff[k0 + i] - ebase;
    __syncthreads();
    // stage only the candidates that start before the block's last output
    {
        int c = 0;
        for (int i = tid; i < nmax; i += 256) c += se[i] < oe ? 1 : 0;
        c = (int)gsd::wave_sum_u64((uint64_t)c);
        if (lane == 0) wred[wave] = c;
    }
    __syncthreads();
    const int ns = wred[0] + wred[1] + wred[2] + wred[3];   // >= 1
    __syncthreads();
    for (int i = tid; i < ns; i += 256) {
        const uint32_t p = list ? list[k0 + i] : (uint32_t)(k0 + i);
        sj[i] = order[p];
        sr[i] = rect_d[p];
    }
    for (int i = tid; i < kEO; i += 256) owner[i] = -1;
    __syncthreads();
    for (int i = tid; i < ns; i += 256) {
        const uint32_t a = se[i], b = se[i + 1];
        if (b > a && a >= ob && a < oe) owner[a - ob] = i;
    }
    __syncthreads();
    // prefix maximum over positions 4 tid .. 4 tid + 3, then over the threads
    int om[4];
    int run = 0;   // staged candidate 0 starts at or before ob
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        run = max(run, owner[4 * tid + q]);
        om[q] = run;
    }
    const int inc = wave_prefix_max(run, lane);
    int exc = __shfl_up(inc, 1, 64);
    if (lane == 0) exc = 0;
    if (lane == 63) wred[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) exc = max(exc, wred[w]);
    const uint32_t end_staged = se[ns];
    uint32_t kq[4], vq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t o = ob + 4u * (uint32_t)tid + (uint32_t)q;
        kq[q] = 0u;
        vq[q] = 0u;
        if (o >= oe) continue;
        int v = max(om[q], exc);
        uint2 pr;
        uint32_t t, j;
        if (o < end_staged) {
            pr = sr[v];
            t = o - se[v];
            j = sj[v];
        } else {
            // past the staged candidates: the last k with eoff[k] - ebase <= o
            int64_t a = k0, b = n - 1;
            while (a < b) {
                const int64_t mid = (a + b + 1) >> 1;
                if (eoff[mid] - ebase <= o) a = mid;
                else b = mid - 1;
            }
            const uint32_t p = list ? list[a] : (uint32_t)a;
            j = order[p];
            pr = rect_d[p];
            t = o - (eoff[a] - ebase);
        }
        const int4 rr = gsd::rect_unpack(pr);
        const Cells c = leaf_cells(rr, ltx0, lty0, ltx1, lty1, sh);
        const int4 cl = make_int4(c.cx0, c.cy0, c.w, c.h);
        const int4 r = make_int4(max(rr.x, ltx0), max(rr.y, lty0), min(rr.z, ltx1), min(rr.w, lty1));
        const float rw = 1.0f / (float)max(c.w, 1);
        const uint32_t wd = (uint32_t)cl.z;
        uint32_t ty = (uint32_t)((float)t * rw);
        int32_t rem = (int32_t)(t - ty * wd);
        if (rem < 0) { ty -= 1u; rem += (int32_t)wd; }
        else if (rem >= (int32_t)wd) { ty += 1u; rem -= (int32_t)wd; }
        const int cx = cl.x + rem, cy = cl.y + (int)ty;
        // the rectangle inside this super-tile (and the leaf), in its local tiles
        const int bx = ((ltx0 >> sh) + cx) << sh, by = ((lty0 >> sh) + cy) << sh;
        const uint32_t x0 = (uint32_t)(max(r.x, bx) - bx), x1 = (uint32_t)(min(r.z, bx + 8) - bx);
        const uint32_t y0 = (uint32_t)(max(r.y, by) - by), y1 = (uint32_t)(min(r.w, by + 8) - by);
        kq[q] = ((x0 | ((x1 - 1u) << 3) | (y0 << 6) | ((y1 - 1u) << 9)) << kCellBits) | (uint32_t)(cy * SW + cx);
        vq[q] = j;
    }
    const uint32_t o4 = ob + 4u * (uint32_t)tid;
    if (o4 + 3u < oe) {
        *reinterpret_cast<uint4*>(keys + o4) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
        *reinterpret_cast<uint4*>(vals + o4) = make_uint4(vq[0], vq[1], vq[2], vq[3]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (o4 + (uint32_t)q < oe) {
                keys[o4 + q] = kq[q];
                vals[o4 + q] = vq[q];
            }
    }
}

// Fine level.  A super-tile's group (slots in depth order) is cut into
// segments of kSeg entries; a work item is one segment, processed by one
// workgroup whose wavefront w owns tile rows 2w and 2w + 1 of the super-tile
// (8 x 8 tiles at leaf-local tile (sx << 3, sy << 3)).  Three passes keep the
// work balanced however long a group is:
//   count: per item and tile, the entries of the segment that cover the tile;
//   scan:  per tile, those counts become the write positions of the items in
//          segment order, starting at the tile's offset;
//   write: each item appends its covering entries at its positions.
// A segment is walked 64 entries at a time: a ballot per tile over the 64
// entries' rectangles (carried in their sort keys, local to the super-tile)
// gives the covering entries, and the rank of an entry is the number of set
// bits below its lane.
constexpr int kSeg = 512;

struct FineItem {
    int sc;            // super-tile
    uint64_t b, e;     // segment [b, e) of the group array
    int64_t item;      // work item index
};

// item -> (super-tile, segment); false for the surplus items of the grid
__device__ __forceinline__ bool fine_item(const uint64_t* __restrict__ soff, const uint32_t* __restrict__ ioff,
                                          const uint32_t* __restrict__ item_sc, int n_super, FineItem& it)
{
    const uint32_t i = blockIdx.x;
    if (i >= ioff[n_super]) return false;
    const int sc = (int)item_sc[i];
    it.sc = sc;
    it.item = i;
    it.b = soff[sc] + (uint64_t)(i - ioff[sc]) * kSeg;
    it.e = min<uint64_t>(soff[sc + 1], it.b + kSeg);
    return true;
}

template <bool WRITE, bool BUF>
__global__ __launch_bounds__(256) void k_fine(int ltx0, int lty0, int TWL, int THL, int SW, int n_super,
                                              const uint64_t* __restrict__ soff, const uint32_t* __restrict__ ioff,
                                              const uint32_t* __restrict__ item_sc,
                                              const uint32_t* __restrict__ group, const uint32_t* __restrict__ gkey,
                                              uint32_t* __restrict__ pos, uint64_t n_values,
                                              uint32_t* __restrict__ values)
{
    FineItem it;
    if (!fine_item(soff, ioff, item_sc, n_super, it)) return;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    // global tile coordinates of this wave's 2 x 8 tiles of the super-tile;
    // tiles outside the leaf (super-tiles straddling its border) are skipped
    const int gx0 = (((ltx0 >> kSuperShift) + it.sc % SW) << kSuperShift);
    const int gy0 = (((lty0 >> kSuperShift) + it.sc / SW) << kSuperShift) + 2 * wave;
    if (gy0 >= lty0 + THL || gy0 + 2 <= lty0) return;
    (void)gx0;
    uint32_t* wp = pos + it.item * 64 + wave * 16;   // this wave's 16 tiles of the item
    // BUF: the slot array as a raw buffer of n_values u32 (byte offsets are
    // 32-bit: fewer than 2^30 entries), else plain stores
    const __amdgpu_buffer_rsrc_t vbuf =
        __builtin_amdgcn_make_buffer_rsrc(values, (short)0, (int)(uint32_t)(BUF ? n_values * 4u : 0u), 0x00020000);
    // running position (write) or count (count pass) of each tile, uniform
    uint32_t cur[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) cur[q] = WRITE ? __builtin_amdgcn_readfirstlane(wp[q]) : 0u;
    const uint64_t b = it.b, e = it.e;
    const uint32_t row0 = 2u * (uint32_t)wave;
    uint32_t sl_n = 0, key_n = 0;          // the next chunk's entry, loaded one chunk ahead
    if (b + lane < e) {
        sl_n = group[b + lane];
        key_n = gkey[b + lane];
    }
    for (uint64_t k = b; k < e; k += 64) {
        const bool ok = k + lane < e;
        const uint32_t sl = sl_n, lr = key_n >> kCellBits;
        if (k + 64 + lane < e) {
            sl_n = group[k + 64 + lane];
            key_n = gkey[k + 64 + lane];
        }
        // the entry covers tile (c, r) of the super-tile iff x0 <= c < x1 and
        // y0 <= r < y1: bit q of `bits` (q = 8 (r - row0) + c) marks the
        // wave's tiles it covers, and one ballot per tile tests a bit
        const uint32_t x0 = lr & 7u, x1 = ((lr >> 3) & 7u) + 1u;
        const uint32_t y0 = (lr >> 6) & 7u, y1 = ((lr >> 9) & 7u) + 1u;
        const uint32_t cols = (0xFFu >> (8u - x1)) & (0xFFu << x0);
        const bool r0 = ok && y0 <= row0 && row0 < y1;
        const bool r1 = ok && y0 <= row0 + 1u && row0 + 1u < y1;
        const uint32_t bits = (r0 ? cols : 0u) | (r1 ? cols << 8 : 0u);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const bool cov = (bits & (1u << q)) != 0u;
            const uint64_t m = gsd::ballot(cov);
            if (WRITE) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                const uint32_t p = cur[q] + below;
                if (BUF) {
                    // lanes that do not cover the tile get an offset past the
                    // buffer's end, and the hardware drops those stores (so
                    // would it any position >= n_values)
                    __builtin_amdgcn_raw_buffer_store_b32(sl, vbuf, (int)(cov ? p * 4u : 0xFFFFFFFFu), 0, 0);
                } else if (cov && p < n_values) {
                    values[p] = sl;   // always true when the counts agree
                }
            }
            cur[q] += (uint32_t)__builtin_popcountll(m);
        }
    }
    if (!WRITE && lane < 16) {
        uint32_t v = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (lane == q) v = cur[q];
        wp[lane] = v;
    }
}

// One workgroup: segments per super-tile, their exclusive scan ioff
// [n_super + 1] and the item -> super-tile map.
__global__ __launch_bounds__(1024) void k_fine_items(const uint64_t* __restrict__ soff, int n_super,
                                                     uint32_t* __restrict__ ioff, uint32_t* __restrict__ item_sc)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int s0 = 0; s0 < n_super; s0 += 1024) {
        const int s = s0 + tid;
        const uint32_t ns = s < n_super ? (uint32_t)((soff[s + 1] - soff[s] + kSeg - 1) / kSeg) : 0u;
        uint32_t x = ns;                       // inclusive wave scan
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = __shfl_up(x, o, 64);
            if (lane >= o) x += u;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        uint32_t before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const uint32_t first = before + x - ns;
        if (s < n_super) {
            ioff[s] = first;
            for (uint32_t q = 0; q < ns; ++q) item_sc[first + q] = (uint32_t)s;
        }
        __syncthreads();
        if (tid == 1023) carry = first + ns;
        __syncthreads();
    }
    if (tid == 0) ioff[n_super] = carry;
}

// per (super-tile, tile): item counts -> write positions, in item order
// (positions inside the leaf's slot array, < 2^32)
__global__ __launch_bounds__(256) void k_fine_scan(int ltx0, int lty0, int TWL, int THL, int SW, int n_super,
                                                   const uint32_t* __restrict__ ioff,
                                                   const uint64_t* __restrict__ toff, uint32_t* __restrict__ pos)
{
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= (int64_t)n_super * 64) return;
    const int sc = (int)(g >> 6), j = (int)(g & 63);
    const int gx = (((ltx0 >> kSuperShift) + sc % SW) << kSuperShift) + (j & 7);
    const int gy = (((lty0 >> kSuperShift) + sc / SW) << kSuperShift) + (j >> 3);
    if (gx < ltx0 || gx >= ltx0 + TWL || gy < lty0 || gy >= lty0 + THL) return;
    uint32_t p = (uint32_t)toff[(int64_t)(gy - lty0) * TWL + (gx - ltx0)];
    // eight items' counts are loaded before their positions are written, so
    // the loads do not wait on each other
    uint32_t i = ioff[sc];
    const uint32_t ie = ioff[sc + 1];
    for (; i + 8u <= ie; i += 8u) {
        uint32_t c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = pos[(int64_t)(i + u) * 64 + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            pos[(int64_t)(i + u) * 64 + j] = p;
            p += c[u];
        }
    }
    for (; i < ie; ++i) {
        const uint32_t c = pos[(int64_t)i * 64 + j];
        pos[(int64_t)i * 64 + j] = p;
        p += c;
    }
}

// offsets[s] = first position whose key (& kmask) is >= s, for s in
// [0, n_seg]; keys sorted ascending by key & kmask, all < n_seg.  Four keys
// per thread.
__global__ __launch_bounds__(256) void k_seg_offsets(const uint32_t* __restrict__ keys, int64_t n, int64_t n_seg,
                                                     uint32_t kmask, uint64_t* __restrict__ offsets)
{
    const int64_t k0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (k0 > n) return;
    int64_t prev = k0 == 0 ? -1 : (int64_t)(keys[k0 - 1] & kmask);
    uint32_t cur4[4];
    if (k0 + 4 <= n && (k0 & 3) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + k0);
        cur4[0] = v.x & kmask; cur4[1] = v.y & kmask; cur4[2] = v.z & kmask; cur4[3] = v.w & kmask;
    } else {
        for (int q = 0; q < 4; ++q) cur4[q] = k0 + q < n ? keys[k0 + q] & kmask : 0u;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + q;
        if (k > n) break;
        const int64_t cur = k == n ? n_seg : (int64_t)cur4[q];
        for (int64_t s = prev + 1; s <= cur; ++s) offsets[s] = (uint64_t)k;
        prev = cur;
    }
}

// the depth sort's input, from the flag pass: candidate i goes to its slot
// with its depth bits (depth > 0: the bits order like the values)
__global__ __launch_bounds__(256) void k_depth_pairs(int64_t n, const uint32_t* __restrict__ flag,
                                                     const uint32_t* __restrict__ slot,
                                                     const uint32_t* __restrict__ dkey, uint32_t* __restrict__ keys,
                                                     uint32_t* __restrict__ vals)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n || !flag[i]) return;
    const uint32_t s = slot[i];
    keys[s] = dkey[i];
    vals[s] = s;
}

// the rectangles in depth order, packed: what the per-leaf passes over the
// depth order read, contiguously, instead of gathering rect by slot
__global__ __launch_bounds__(256) void k_rect_depth(int64_t n, const uint32_t* __restrict__ order,
                                                    const int4* __restrict__ rect, uint2* __restrict__ rect_d)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    rect_d[k] = gsd::rect_pack(rect[order[k]]);
}

__global__ void k_export_keys(int64_t n_tiles, int ltx0, int lty0, int TWL, int TW, const uint64_t* __restrict__ offsets,
                              const uint32_t* __restrict__ values, const float4* __restrict__ g2,
                              uint64_t* __restrict__ keys)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_tiles) return;
    const int64_t tile = (int64_t)(lty0 + t / TWL) * TW + (ltx0 + t % TWL);
    for (uint64_t k = offsets[t]; k < offsets[t + 1]; ++k)
        keys[k] = ((uint64_t)tile << 32) | (uint64_t)__builtin_bit_cast(uint32_t, g2[values[k]].y);
}

}  // namespace

int super_cols(gs_tile_rect leaf) { return ((leaf.tx1 - 1) >> kSuperShift) - (leaf.tx0 >> kSuperShift) + 1; }
int super_rows(gs_tile_rect leaf) { return ((leaf.ty1 - 1) >> kSuperShift) - (leaf.ty0 >> kSuperShift) + 1; }
int64_t super_cells(gs_tile_rect leaf) { return (int64_t)super_cols(leaf) * super_rows(leaf); }
int super_shift() { return kSuperShift; }
uint32_t super_key_mask() { return (1u << kCellBits) - 1u; }
int64_t super_cells_max() { return (int64_t)1 << kCellBits; }

int bits_for(int64_t n_keys)
{
    int b = 0;
    while (b < 40 && (1ll << b) < n_keys) ++b;
    return b;
}

gs_status launch_rect_diff(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                           int64_t n_list, int32_t* diff)
{
    const int64_t n = list ? n_list : proj->n_cand;
    const int64_t cells = (int64_t)(leaf.tx1 - leaf.tx0) * (leaf.ty1 - leaf.ty0);
    if (n > 0) {
        GsTimerScope ts(ctx, "rect_diff");
        const int TWL = leaf.tx1 - leaf.tx0, THL = leaf.ty1 - leaf.ty0;
        if (cells <= kDiffLds) {
            hipLaunchKernelGGL(k_rect_diff_lds, dim3((unsigned)ceil_div(n, kDiffBlock)), dim3(256),
                               sizeof(int32_t) * cells, ctx->stream, n, list, proj->rect, leaf.tx0, leaf.ty0, leaf.tx1,
                               leaf.ty1, diff);
        } else if (!list && TWL <= kRowCellsMax && THL <= kRowsMax && n < (int64_t)1 << 30) {
            // by rows: every cell of the grid is written
            const int64_t nblk = ceil_div(n, kRowRects);
            const int64_t nh = nblk * THL;
            std::vector<GsAlloc> tmp;
            uint32_t* hist = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nh, GS_MEM_SCRATCH, &tmp);
            uint32_t* off = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * (nh + 1), GS_MEM_SCRATCH, &tmp);
            uint32_t* rec = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * 4 * n, GS_MEM_SCRATCH, &tmp);
            if (!hist || !off || !rec) {
                gs_free_all(ctx, &tmp);
                return GS_ERR_OOM;
            }
            hipLaunchKernelGGL(k_row_hist, dim3((unsigned)nblk), dim3(256), 0, ctx->stream, n, proj->rect, leaf.tx0,
                               leaf.ty0, leaf.tx1, leaf.ty1, hist);
            gs_status st = launch_scan_u32_to_u32(ctx, hist, off, nh);
            if (st == GS_OK) {
                hipLaunchKernelGGL(k_row_scatter, dim3((unsigned)nblk), dim3(256), 0, ctx->stream, n, proj->rect,
                                   leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, off, rec);
                hipLaunchKernelGGL(k_row_sum, dim3((unsigned)THL), dim3(256), sizeof(int32_t) * TWL, ctx->stream, off,
                                   (int)nblk, rec, TWL, diff);
            }
            gs_free_all(ctx, &tmp);
            if (st != GS_OK) return st;
        } else
            hipLaunchKernelGGL(k_rect_diff, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, n, list,
                               proj->rect, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, diff);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_count_cells(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                             int64_t n_list, uint32_t* cnt)
{
    if (n_list > 0) {
        GsTimerScope ts(ctx, "bin_count");
        hipLaunchKernelGGL(k_count_cells, dim3((unsigned)ceil_div(n_list, 256)), dim3(256), 0, ctx->stream, n_list,
                           list, proj->rect_d, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, kSuperShift, cnt);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_leaf_counts(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, uint32_t* out)
{
    const int TWL = leaf.tx1 - leaf.tx0;
    const int64_t n = (int64_t)TWL * (leaf.ty1 - leaf.ty0);
    if (n > 0) {
        GsTimerScope ts(ctx, "bin_count");
        hipLaunchKernelGGL(k_leaf_counts, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream,
                           proj->tile_cnt, proj->TW, leaf.tx0, leaf.ty0, TWL, n, out);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

int64_t emit_blocks(uint64_t total) { return ceil_div((int64_t)total, kEO); }

gs_status launch_emit_cells(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                            int64_t n_list, const uint32_t* eoff, uint32_t ebase, uint64_t total, uint32_t* keys,
                            uint32_t* vals, uint32_t* bst)
{
    if (n_list > 0 && total > 0) {
        GsTimerScope ts(ctx, "emit");
        if (bst)
            hipLaunchKernelGGL(k_emit_starts, dim3((unsigned)ceil_div(n_list, 256)), dim3(256), 0, ctx->stream, n_list,
                               eoff, ebase, bst);
        hipLaunchKernelGGL(k_emit_pairs, dim3((unsigned)emit_blocks(total)), dim3(256), 0, ctx->stream, n_list, list,
                           proj->order, proj->rect_d, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, kSuperShift,
                           super_cols(leaf), eoff, ebase, (uint32_t)total, bst, keys, vals);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

int64_t fine_items_bound(gs_tile_rect leaf, uint64_t n_cells)
{
    return super_cells(leaf) + (int64_t)((n_cells + kSeg - 1) / kSeg);
}

// items, their per-tile counts and the write positions (everything of the
// fine level before the slot array is written)
gs_status launch_fine_prepare(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                              const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint64_t* toff,
                              uint32_t* item_sc, uint32_t* ioff, uint32_t* pos)
{
    (void)proj;
    const int n_super = (int)super_cells(leaf);
    const int64_t items = fine_items_bound(leaf, n_cells);
    if (n_super <= 0 || n_cells == 0) return GS_OK;
    const int TWL = leaf.tx1 - leaf.tx0, THL = leaf.ty1 - leaf.ty0, SW = super_cols(leaf);
    GsTimerScope ts(ctx, "fine");
    hipLaunchKernelGGL(k_fine_items, dim3(1), dim3(1024), 0, ctx->stream, soff, n_super, ioff, item_sc);
    hipLaunchKernelGGL((k_fine<false, false>), dim3((unsigned)items), dim3(256), 0, ctx->stream, leaf.tx0, leaf.ty0,
                       TWL, THL, SW, n_super, soff, ioff, item_sc, group, gkey, pos, 0ull, nullptr);
    hipLaunchKernelGGL(k_fine_scan, dim3((unsigned)ceil_div((int64_t)n_super * 64, 256)), dim3(256), 0, ctx->stream,
                       leaf.tx0, leaf.ty0, TWL, THL, SW, n_super, ioff, toff, pos);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

// the slot array from the prepared items and positions
gs_status launch_fine_write(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                            const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint32_t* item_sc,
                            const uint32_t* ioff, uint32_t* pos, uint64_t n_values, uint32_t* values)
{
    (void)proj;
    const int n_super = (int)super_cells(leaf);
    const int64_t items = fine_items_bound(leaf, n_cells);
    if (n_super <= 0 || n_cells == 0) return GS_OK;
    const int TWL = leaf.tx1 - leaf.tx0, THL = leaf.ty1 - leaf.ty0, SW = super_cols(leaf);
    GsTimerScope ts(ctx, "fine");
    if (n_values < (1ull << 30))
        hipLaunchKernelGGL((k_fine<true, true>), dim3((unsigned)items), dim3(256), 0, ctx->stream, leaf.tx0, leaf.ty0,
                           TWL, THL, SW, n_super, soff, ioff, item_sc, group, gkey, pos, n_values, values);
    else
        hipLaunchKernelGGL((k_fine<true, false>), dim3((unsigned)items), dim3(256), 0, ctx->stream, leaf.tx0,
                           leaf.ty0, TWL, THL, SW, n_super, soff, ioff, item_sc, group, gkey, pos, n_values, values);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_fine_lists(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                            const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint64_t* toff,
                            uint32_t* item_sc, uint32_t* ioff, uint32_t* pos, uint64_t n_values, uint32_t* values)
{
    gs_status st = launch_fine_prepare(ctx, proj, leaf, soff, group, gkey, n_cells, toff, item_sc, ioff, pos);
    if (st != GS_OK) return st;
    return launch_fine_write(ctx, proj, leaf, soff, group, gkey, n_cells, item_sc, ioff, pos, n_values, values);
}

gs_status launch_seg_offsets(gs_ctx* ctx, const uint32_t* sorted_keys, int64_t n, int64_t n_seg, uint32_t kmask,
                             uint64_t* offsets)
{
    GsTimerScope ts(ctx, "seg_offsets");
    hipLaunchKernelGGL(k_seg_offsets, dim3((unsigned)ceil_div(ceil_div(n + 1, 4), 256)), dim3(256), 0, ctx->stream,
                       sorted_keys, n, n_seg, kmask, offsets);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_depth_pairs(gs_ctx* ctx, int64_t n, const uint32_t* flag, const uint32_t* slot, const uint32_t* dkey,
                             uint32_t* keys, uint32_t* vals)
{
    if (n > 0)
        hipLaunchKernelGGL(k_depth_pairs, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, n, flag, slot,
                           dkey, keys, vals);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_rect_depth(gs_ctx* ctx, const gs_proj* proj, const uint32_t* order, uint2* rect_d)
{
    if (proj->n_cand > 0)
        hipLaunchKernelGGL(k_rect_depth, dim3((unsigned)ceil_div(proj->n_cand, 256)), dim3(256), 0, ctx->stream,
                           proj->n_cand, order, proj->rect, rect_d);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_export_keys(gs_ctx* ctx, const gs_bins* b, uint64_t* keys)
{
    if (b->n_tiles > 0)
        hipLaunchKernelGGL(k_export_keys, dim3((unsigned)ceil_div(b->n_tiles, 256)), dim3(256), 0, ctx->stream,
                           b->n_tiles, b->leaf.tx0, b->leaf.ty0, b->TWL, b->proj->TW, b->offsets, b->values,
                           b->proj->g2, keys);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
