// planner.hip -- load-budgeted leaf planning.
//
// BoundedGS page, "01": regions are sized by their actual load, estimated
// from the overlap count, the pixels and the buffer layout, so dense regions
// become small and sparse ones large; Fig. 3 B->C: regions over the budget
// are subdivided further.  Reading: starting from the whole tile grid, a
// region is kept when est <= budget or it is a single tile; otherwise its
// longer side (ties: x) is halved at floor(len/2) and both halves are planned
// in order (depth-first order of the leaves).
//
// Reading of the load estimate (the library's own allocation bounds):
//   est = bI I + bC Cb + bP P + bT T + b0
// with I the region's Gaussian-tile overlaps and Cb the (candidate,
// super-cell) pairs over the image-aligned 8 x 8-tile super-cells the region
// meets -- an upper bound of the coarse pairs its binning sorts.  Per-tile
// and per-super-cell counts come from 2D difference arrays; summed-area
// tables make every region's I and Cb O(1).  The split
// recursion runs in one workgroup, level by level: the frontier is kept in
// depth-first order, and each level replaces every region to be split by its
// two halves (a workgroup scan gives the output positions), so the final
// frontier is the depth-first list of leaves.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

__global__ void k_counts_to_sat(const int32_t* __restrict__ cnt, int TW, int TH, uint64_t* __restrict__ sat)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t S = TW + 1;
    if (k >= S * (TH + 1)) return;
    const int64_t y = k / S, x = k % S;
    sat[k] = (x == 0 || y == 0) ? 0ull : (uint64_t)(uint32_t)cnt[(y - 1) * TW + (x - 1)];
}

struct PlanArgs {
    int W, H, TW, TH, SW;
    uint64_t budget, bI, bP, bT, b0, bC;
    const uint64_t* sat;     // (TH + 1) x (TW + 1), tile counts (NULL when bI = 0)
    const uint64_t* sat8;    // (SH + 1) x (SW + 1), super-cell counts
    const uint64_t* isum;    // the whole grid's intersections (when sat is NULL)
};

__device__ __forceinline__ uint64_t sat_rect(const uint64_t* __restrict__ sat, int64_t S, int x0, int y0, int x1,
                                             int y1)
{
    return sat[(int64_t)y1 * S + x1] - sat[(int64_t)y0 * S + x1] - sat[(int64_t)y1 * S + x0] +
           sat[(int64_t)y0 * S + x0];
}

__device__ __forceinline__ uint64_t region_est(const PlanArgs& a, int4 r)
{
    const uint64_t I = a.bI ? sat_rect(a.sat, a.TW + 1, r.x, r.y, r.z, r.w) : 0ull;
    const uint64_t Cb = sat_rect(a.sat8, a.SW + 1, r.x >> 3, r.y >> 3, ((r.z - 1) >> 3) + 1, ((r.w - 1) >> 3) + 1);
    const int64_t x1 = min<int64_t>((int64_t)r.z * 16, a.W), y1 = min<int64_t>((int64_t)r.w * 16, a.H);
    const uint64_t P = (uint64_t)(x1 - (int64_t)r.x * 16) * (uint64_t)(y1 - (int64_t)r.y * 16);
    const uint64_t T = (uint64_t)(r.z - r.x) * (uint64_t)(r.w - r.y);
    return a.bI * I + a.bC * Cb + a.bP * P + a.bT * T + a.b0;
}

__device__ __forceinline__ bool region_split(const PlanArgs& a, int4 r)
{
    const bool single = (r.z - r.x) == 1 && (r.w - r.y) == 1;
    return !single && region_est(a, r) > a.budget;
}

// Difference array of the candidates' super-cell rectangles on the
// [SH][SW] grid (add its 2D prefix for the counts).  A block takes
// kCellBlock candidates into an LDS copy of the grid, then adds its nonzero
// cells to the global grid: far fewer global atomics on the few cells.
// isum (optional): the candidates' tile rectangle areas are added to it (the
// grid's intersections, one atomic per block).
constexpr int kCellBlock = 8192;
constexpr int kCellLds = 16384;    // cells of the LDS copy (64 KB)

__global__ __launch_bounds__(256) void k_cell_diff(int64_t n, const int4* __restrict__ rect, int SW, int SH,
                                                   int32_t* __restrict__ diff, unsigned long long* __restrict__ isum)
{
    __shared__ uint64_t ws[4];
    uint64_t area = 0;
    extern __shared__ int32_t hd[];
    const int64_t cells = (int64_t)SW * SH;
    const bool lds = cells <= kCellLds;
    if (lds) {
        for (int64_t k = threadIdx.x; k < cells; k += blockDim.x) hd[k] = 0;
        __syncthreads();
    }
    const int64_t c0 = (int64_t)blockIdx.x * kCellBlock;
    for (int64_t k = c0 + threadIdx.x; k < min<int64_t>(n, c0 + kCellBlock); k += blockDim.x) {
        const int4 r = rect[k];
        if (!(r.x < r.z && r.y < r.w)) continue;
        area += (uint64_t)(r.z - r.x) * (uint64_t)(r.w - r.y);
        const int x0 = r.x >> 3, y0 = r.y >> 3, x1 = ((r.z - 1) >> 3) + 1, y1 = ((r.w - 1) >> 3) + 1;
        auto add = [&](int y, int x, int v) {
            if (lds) atomicAdd(&hd[(int64_t)y * SW + x], v);
            else atomicAdd(&diff[(int64_t)y * SW + x], v);
        };
        add(y0, x0, 1);
        if (x1 < SW) add(y0, x1, -1);
        if (y1 < SH) add(y1, x0, -1);
        if (x1 < SW && y1 < SH) add(y1, x1, 1);
    }
    if (lds) {
        __syncthreads();
        for (int64_t k = threadIdx.x; k < cells; k += blockDim.x)
            if (hd[k]) atomicAdd(&diff[k], hd[k]);
    }
    if (isum) {
        area = gsd::wave_sum_u64(area);
        if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = area;
        __syncthreads();
        if (threadIdx.x == 0) atomicAdd(isum, (unsigned long long)(ws[0] + ws[1] + ws[2] + ws[3]));
    }
}

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* tot, uint32_t* sh)
{
    // sh: kPlanThreads / 64 entries
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        if (w < wave) before += sh[w];
        all += sh[w];
    }
    __syncthreads();
    *tot = all;
    return before + x - v;
}

// frontier ping-pong in global memory; cap >= number of tiles.  The frontier
// starts as the whole grid, or as the given roots (a cached layout to
// re-check, in order); each level splits every region over the budget in
// place, so the leaves come out depth-first per root, roots in order.
__global__ __launch_bounds__(kPlanThreads) void k_plan(PlanArgs a,
                                                       int4* __restrict__ fa, int4* __restrict__ fb, int64_t cap,
                                                       const gs_leaf* __restrict__ roots, int32_t n_roots,
                                                       gs_leaf* __restrict__ leaves, int32_t max_leaves,
                                                       int32_t* __restrict__ count_out,
                                                       int32_t* __restrict__ over_out,
                                                       uint64_t* __restrict__ totals_out)
{
    __shared__ uint32_t sh[kPlanThreads / 64];
    __shared__ uint32_t s_total, s_any;
    // the whole grid's intersections and (candidate, super-cell) pairs
    if (totals_out && threadIdx.x == 0) {
        totals_out[0] = a.sat ? sat_rect(a.sat, a.TW + 1, 0, 0, a.TW, a.TH) : *a.isum;
        totals_out[1] = sat_rect(a.sat8, a.SW + 1, 0, 0, a.SW, (a.TH + 7) >> 3);
    }
    int4* cur = fa;
    int4* nxt = fb;
    uint32_t n = 1;
    if (n_roots > 0) {
        for (int32_t i = threadIdx.x; i < n_roots; i += kPlanThreads)
            cur[i] = make_int4(roots[i].tx0, roots[i].ty0, roots[i].tx1, roots[i].ty1);
        n = (uint32_t)n_roots;
    } else if (threadIdx.x == 0) {
        cur[0] = make_int4(0, 0, a.TW, a.TH);
    }
    __syncthreads();
    for (;;) {
        // one level: every region to split becomes two, in order
        uint32_t carry = 0;
        if (threadIdx.x == 0) s_any = 0;
        __syncthreads();
        for (uint32_t c0 = 0; c0 < n; c0 += kPlanThreads) {
            const uint32_t i = c0 + threadIdx.x;
            int4 r = make_int4(0, 0, 0, 0);
            bool sp = false;
            if (i < n) {
                r = cur[i];
                sp = region_split(a, r);
            }
            const uint32_t w = i < n ? (sp ? 2u : 1u) : 0u;
            uint32_t tot;
            const uint32_t pos = carry + block_excl_scan_u32(w, &tot, sh);
            if (i < n && pos + w <= cap) {
                if (!sp) {
                    nxt[pos] = r;
                } else {
                    int4 lo = r, hi = r;
                    const int wdt = r.z - r.x, hgt = r.w - r.y;
                    if (wdt >= hgt) { lo.z = r.x + wdt / 2; hi.x = lo.z; }
                    else { lo.w = r.y + hgt / 2; hi.y = lo.w; }
                    nxt[pos] = lo;
                    nxt[pos + 1] = hi;
                    s_any = 1;
                }
            }
            carry += tot;
            __syncthreads();
        }
        const uint32_t any = s_any;
        n = carry < cap ? carry : (uint32_t)cap;
        int4* t = cur;
        cur = nxt;
        nxt = t;
        __syncthreads();
        if (!any) break;
    }
    // cur holds the leaves in depth-first order
    uint32_t over = 0;
    for (uint32_t i = threadIdx.x; i < n; i += kPlanThreads) {
        const int4 r = cur[i];
        const uint64_t e = region_est(a, r);
        if (e > a.budget) over = 1;
        if ((int32_t)i < max_leaves) {
            gs_leaf L;
            L.tx0 = r.x; L.ty0 = r.y; L.tx1 = r.z; L.ty1 = r.w;
            L.est_bytes = e;
            L.over_budget = e > a.budget ? 1 : 0;
            L.pad = 0;
            leaves[i] = L;
        }
    }
    if (over) atomicOr(over_out, 1);
    if (threadIdx.x == 0) *count_out = (int32_t)n;
}

}  // namespace

gs_status launch_tile_counts(gs_ctx* ctx, const gs_proj* proj, int32_t* grid)
{
    const int TW = proj->TW, TH = proj->TH;
    gs_status st = launch_fill_u32(ctx, (uint32_t*)grid, 0u, (int64_t)TW * TH);
    if (st != GS_OK) return st;
    gs_tile_rect all{0, 0, TW, TH};
    if ((st = launch_rect_diff(ctx, proj, all, nullptr, 0, grid)) != GS_OK) return st;
    return launch_prefix2d_i32(ctx, grid, TH, TW);
}

gs_status launch_plan(gs_ctx* ctx, const gs_proj* proj, uint64_t* sat, uint64_t budget, const gs_cost_model* cost,
                      const gs_leaf* roots_dev, int32_t n_roots, gs_leaf* leaves_dev, int32_t max_leaves,
                      int32_t* count_dev, int32_t* over_dev, uint64_t* totals_dev)
{
    const int TW = proj->TW, TH = proj->TH;
    const int SW = (TW + 7) >> 3, SH = (TH + 7) >> 3;
    const int64_t T = (int64_t)TW * TH;
    // the tile counts' table only when the model prices intersections (sat
    // given); otherwise the grid's total comes from the super-cell pass
    gs_status st = GS_OK;
    if (sat) {
        const int64_t S = (int64_t)(TW + 1) * (TH + 1);
        hipLaunchKernelGGL(k_counts_to_sat, dim3((unsigned)ceil_div(S, 256)), dim3(256), 0, ctx->stream,
                           proj->tile_cnt, TW, TH, sat);
        if ((st = launch_prefix2d_u64(ctx, sat, TH + 1, TW + 1)) != GS_OK) return st;
    } else if (cost->b_isect != 0) {
        return gs_fail(ctx, GS_ERR_STATE, "the cost model prices intersections: the tile counts are needed");
    }

    std::vector<GsAlloc> tmp;
    int4* fa = (int4*)gs_malloc(ctx, sizeof(int4) * T, GS_MEM_SCRATCH, &tmp);
    int4* fb = (int4*)gs_malloc(ctx, sizeof(int4) * T, GS_MEM_SCRATCH, &tmp);
    int32_t* cgrid = (int32_t*)gs_malloc(ctx, sizeof(int32_t) * SW * SH, GS_MEM_SCRATCH, &tmp);
    uint64_t* sat8 = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (SW + 1) * (SH + 1), GS_MEM_SCRATCH, &tmp);
    uint64_t* isum = sat ? nullptr : (uint64_t*)gs_malloc(ctx, sizeof(uint64_t), GS_MEM_SCRATCH, &tmp);
    if (!fa || !fb || !cgrid || !sat8 || (!sat && !isum)) {
        gs_free_all(ctx, &tmp);
        return GS_ERR_OOM;
    }
    if (isum && (st = launch_fill_u32(ctx, (uint32_t*)isum, 0u, 2)) != GS_OK) {
        gs_free_all(ctx, &tmp);
        return st;
    }
    // candidates per image-aligned super-cell of 8 x 8 tiles, and their table
    if ((st = launch_fill_u32(ctx, (uint32_t*)cgrid, 0u, (int64_t)SW * SH)) != GS_OK) {
        gs_free_all(ctx, &tmp);
        return st;
    }
    if (proj->n_cand > 0) {
        GsTimerScope ts(ctx, "rect_diff");
        const size_t lds = (int64_t)SW * SH <= kCellLds ? sizeof(int32_t) * SW * SH : 0;
        hipLaunchKernelGGL(k_cell_diff, dim3((unsigned)ceil_div(proj->n_cand, kCellBlock)), dim3(256), lds,
                           ctx->stream, proj->n_cand, proj->rect, SW, SH, cgrid, (unsigned long long*)isum);
    }
    if ((st = launch_prefix2d_i32(ctx, cgrid, SH, SW)) != GS_OK) {
        gs_free_all(ctx, &tmp);
        return st;
    }
    const int64_t S8 = (int64_t)(SW + 1) * (SH + 1);
    hipLaunchKernelGGL(k_counts_to_sat, dim3((unsigned)ceil_div(S8, 256)), dim3(256), 0, ctx->stream, cgrid, SW, SH,
                       sat8);
    if ((st = launch_prefix2d_u64(ctx, sat8, SH + 1, SW + 1)) != GS_OK) {
        gs_free_all(ctx, &tmp);
        return st;
    }
    PlanArgs a;
    a.W = proj->W; a.H = proj->H; a.TW = TW; a.TH = TH; a.SW = SW;
    a.budget = budget;
    a.bI = cost->b_isect; a.bP = cost->b_pixel; a.bT = cost->b_tile; a.b0 = cost->b_const; a.bC = cost->b_cell;
    a.sat = sat;
    a.sat8 = sat8;
    a.isum = isum;
    GS_HIP(ctx, hipMemsetAsync(over_dev, 0, sizeof(int32_t), ctx->stream));
    {
        GsTimerScope ts(ctx, "plan_split");
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, ctx->stream, a, fa, fb, T, roots_dev, n_roots,
                           leaves_dev, max_leaves, count_dev, over_dev, totals_dev);
    }
    gs_free_all(ctx, &tmp);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

// ---------------------------------------------------------------------------
// leaf -> candidate groups.  Binning a leaf only needs the candidates whose
// rectangle meets it, in depth order.  The candidates are visited in depth
// order (their packed rectangles, rect_d, contiguous); each emits (leaf,
// depth position) for every leaf it meets -- one leaf when its four rectangle
// corners share a leaf (leaves are rectangles), otherwise every leaf its
// rectangle meets -- and a stable radix sort on the leaf id groups them with
// the depth order kept inside each group.

namespace {

// Per-leaf passes over a leaf's tiles run on a grid of (chunk, leaf): block
// (c, L) takes tiles [c kLeafChunk, (c + 1) kLeafChunk) of leaf L in its
// leaf-local row-major order (blocks past the leaf's end return), so that a
// view's leaves keep the whole GPU busy whatever their number.
constexpr int kLeafChunk = 4096;

__global__ __launch_bounds__(256) void k_leaf_map(const gs_leaf* __restrict__ leaves, int TW,
                                                  int32_t* __restrict__ lot)
{
    const gs_leaf L = leaves[blockIdx.y];
    const int w = L.tx1 - L.tx0;
    const int64_t tot = (int64_t)w * (L.ty1 - L.ty0);
    const int64_t k0 = (int64_t)blockIdx.x * kLeafChunk, k1 = min(tot, k0 + kLeafChunk);
    for (int64_t k = k0 + threadIdx.x; k < k1; k += 256)
        lot[(int64_t)(L.ty0 + k / w) * TW + (L.tx0 + k % w)] = (int32_t)blockIdx.y;
}

__device__ __forceinline__ bool rect_meets(int4 r, const gs_leaf& L)
{
    return r.x < L.tx1 && L.tx0 < r.z && r.y < L.ty1 && L.ty0 < r.w;
}

// Up to this many leaves, a candidate tests every leaf rectangle (from LDS)
// instead of looking its corners up in the tile -> leaf map.
constexpr int kLeafDirect = 64;

// EMIT = false: number of leaves met; true: write the (leaf, depth position)
// pairs, leaves in ascending order
template <bool EMIT>
__global__ __launch_bounds__(256) void k_leaf_pairs(int64_t n, const uint2* __restrict__ rect_d,
                                                    const gs_leaf* __restrict__ leaves, int nl,
                                                    const int32_t* __restrict__ lot, int TW,
                                                    uint32_t* __restrict__ cnt, const uint64_t* __restrict__ off,
                                                    uint32_t* __restrict__ keys, uint32_t* __restrict__ vals)
{
    __shared__ int4 sl[kLeafDirect];
    const bool direct = nl <= kLeafDirect;
    if (direct) {
        for (int L = threadIdx.x; L < nl; L += blockDim.x)
            sl[L] = make_int4(leaves[L].tx0, leaves[L].ty0, leaves[L].tx1, leaves[L].ty1);
        __syncthreads();
    }
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const uint32_t j = (uint32_t)k;   // the depth position
    const int4 r = gsd::rect_unpack(rect_d[k]);
    if (direct) {
        uint64_t o = EMIT ? off[k] : 0;
        uint32_t m = 0;
        for (int L = 0; L < nl; ++L) {
            const int4 q = sl[L];
            if (r.x < q.z && q.x < r.z && r.y < q.w && q.y < r.w) {
                if (EMIT) {
                    keys[o] = (uint32_t)L;
                    vals[o] = j;
                    ++o;
                }
                ++m;
            }
        }
        if (!EMIT) cnt[k] = m;
        return;
    }
    const int a = lot[(int64_t)r.y * TW + r.x], b = lot[(int64_t)r.y * TW + r.z - 1];
    const int c = lot[(int64_t)(r.w - 1) * TW + r.x], d = lot[(int64_t)(r.w - 1) * TW + r.z - 1];
    if (a >= 0 && a == b && a == c && a == d) {   // the four corners in one leaf: the rectangle inside it
        if (EMIT) {
            keys[off[k]] = (uint32_t)a;
            vals[off[k]] = j;
        } else {
            cnt[k] = 1u;
        }
        return;
    }
    uint64_t o = EMIT ? off[k] : 0;
    uint32_t m = 0;
    for (int L = 0; L < nl; ++L)
        if (rect_meets(r, leaves[L])) {
            if (EMIT) {
                keys[o] = (uint32_t)L;
                vals[o] = j;
                ++o;
            }
            ++m;
        }
    if (!EMIT) cnt[k] = m;
}

// per grouped (leaf, depth position) entry: the super-tiles of its leaf that
// the rectangle meets (the entry's coarse pairs)
__global__ __launch_bounds__(256) void k_group_cells(int64_t n, const uint32_t* __restrict__ leaf_of,
                                                     const uint32_t* __restrict__ pos, const uint2* __restrict__ rect_d,
                                                     const gs_leaf* __restrict__ leaves, int sh,
                                                     uint32_t* __restrict__ cnt)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const gs_leaf lf = leaves[leaf_of[k]];
    const int4 r = gsd::rect_unpack(rect_d[pos[k]]);
    // image-aligned super-cells that the rectangle meets inside the leaf
    const int x0 = max(r.x, lf.tx0), x1 = min(r.z, lf.tx1);
    const int y0 = max(r.y, lf.ty0), y1 = min(r.w, lf.ty1);
    uint32_t c = 0;
    if (x0 < x1 && y0 < y1)
        c = (uint32_t)((((x1 - 1) >> sh) - (x0 >> sh) + 1) * (((y1 - 1) >> sh) - (y0 >> sh) + 1));
    cnt[k] = c;
}

// per leaf: the scan value at its first entry and its number of coarse pairs
// (u32 arithmetic modulo 2^32: exact for any leaf with fewer than 2^32
// pairs), and its intersections (the last of its tile offsets)
__global__ void k_leaf_cell_bounds(int nl, const uint64_t* __restrict__ goff, const uint32_t* __restrict__ coff,
                                   const gs_leaf* __restrict__ leaves, const uint64_t* __restrict__ toff_base,
                                   const uint64_t* __restrict__ toff, uint32_t* __restrict__ out,
                                   uint64_t* __restrict__ isect)
{
    const int L = blockIdx.x * blockDim.x + threadIdx.x;
    if (L >= nl) return;
    const uint32_t a = coff[goff[L]], b = coff[goff[L + 1]];
    out[2 * L] = a;
    out[2 * L + 1] = b - a;
    const gs_leaf lf = leaves[L];
    isect[L] = toff[toff_base[L] + (uint64_t)(lf.tx1 - lf.tx0) * (uint64_t)(lf.ty1 - lf.ty0)];
}

// Per leaf, the exclusive scan of its tiles' candidate counts in leaf-local
// row-major order, written at out + base[L] (T_L + 1 entries, the last the
// leaf's total), in three steps over the (chunk, leaf) grid: each block sums
// its chunk; one thread per leaf scans its chunk sums (in place) and writes
// the total; each block scans its chunk (256 tiles per round: a wavefront
// scan, the four wavefront totals through LDS, a running carry) from its
// chunk's offset.
__device__ __forceinline__ uint64_t leaf_tile_count(const int32_t* __restrict__ tile_cnt, int TW, const gs_leaf& lf,
                                                    int TWL, int64_t t, int64_t t1)
{
    return t < t1 ? (uint64_t)tile_cnt[(int64_t)(lf.ty0 + t / TWL) * TW + lf.tx0 + t % TWL] : 0ull;
}

__global__ __launch_bounds__(256) void k_toff_sums(const gs_leaf* __restrict__ leaves,
                                                   const int32_t* __restrict__ tile_cnt, int TW,
                                                   uint64_t* __restrict__ csum)
{
    __shared__ uint64_t ws[4];
    const gs_leaf lf = leaves[blockIdx.y];
    const int TWL = lf.tx1 - lf.tx0;
    const int64_t n = (int64_t)TWL * (lf.ty1 - lf.ty0);
    const int64_t t0 = (int64_t)blockIdx.x * kLeafChunk, t1 = min(n, t0 + kLeafChunk);
    uint64_t s = 0;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) s += leaf_tile_count(tile_cnt, TW, lf, TWL, t, t1);
    s = gsd::wave_sum_u64(s);
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) csum[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

__global__ __launch_bounds__(256) void k_toff_chunk_scan(int nl, int nchunk, const gs_leaf* __restrict__ leaves,
                                                         uint64_t* __restrict__ csum,
                                                         const uint64_t* __restrict__ base, uint64_t* __restrict__ out)
{
    for (int L = blockIdx.x * 256 + threadIdx.x; L < nl; L += gridDim.x * 256) {
        const gs_leaf lf = leaves[L];
        const int64_t n = (int64_t)(lf.tx1 - lf.tx0) * (lf.ty1 - lf.ty0);
        uint64_t run = 0;
        for (int c = 0; c < nchunk; ++c) {
            uint64_t& x = csum[(int64_t)L * nchunk + c];
            const uint64_t v = x;
            x = run;
            run += v;
        }
        out[base[L] + n] = run;
    }
}

__global__ __launch_bounds__(256) void k_toff_write(const gs_leaf* __restrict__ leaves,
                                                    const int32_t* __restrict__ tile_cnt, int TW,
                                                    const uint64_t* __restrict__ csum,
                                                    const uint64_t* __restrict__ base, uint64_t* __restrict__ out)
{
    __shared__ uint64_t ws[4];
    const gs_leaf lf = leaves[blockIdx.y];
    const int TWL = lf.tx1 - lf.tx0;
    const int64_t n = (int64_t)TWL * (lf.ty1 - lf.ty0);
    const int64_t t0 = (int64_t)blockIdx.x * kLeafChunk, t1 = min(n, t0 + kLeafChunk);
    if (t0 >= t1) return;
    uint64_t* o = out + base[blockIdx.y];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t carry = csum[(int64_t)blockIdx.y * gridDim.x + blockIdx.x];
    for (int64_t c = t0; c < t1; c += 256) {
        const int64_t t = c + threadIdx.x;
        const uint64_t v = leaf_tile_count(tile_cnt, TW, lf, TWL, t, t1);
        uint64_t x = v;
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t u = __shfl_up((unsigned long long)x, d, 64);
            if (lane >= d) x += u;
        }
        if (lane == 63) ws[wave] = x;
        __syncthreads();
        uint64_t before = 0;
        for (int w = 0; w < wave; ++w) before += ws[w];
        if (t < t1) o[t] = carry + before + x - v;
        carry += ws[0] + ws[1] + ws[2] + ws[3];
        __syncthreads();
    }
}

}  // namespace

// chunks of kLeafChunk tiles of the largest leaf (host leaves)
static int leaf_chunks(const gs_leaf* hleaves, int32_t n_leaves)
{
    int64_t m = 1;
    for (int32_t L = 0; L < n_leaves; ++L)
        m = std::max<int64_t>(m, ceil_div((int64_t)(hleaves[L].tx1 - hleaves[L].tx0) * (hleaves[L].ty1 - hleaves[L].ty0),
                                          kLeafChunk));
    return (int)m;
}

namespace {

// base[L] = sum over the leaves before L of (their tiles + 1): where each
// leaf's tile offsets (T_L + 1 entries) and launch order start.  One block:
// thread t sums a run of consecutive leaves, the runs are scanned across the
// block, and each thread writes its run's bases.
constexpr int kBaseThreads = 1024;

__device__ __forceinline__ uint64_t leaf_slots(const gs_leaf& L)
{
    return (uint64_t)(L.tx1 - L.tx0) * (uint64_t)(L.ty1 - L.ty0) + 1;
}

__global__ __launch_bounds__(kBaseThreads) void k_tile_bases(const gs_leaf* __restrict__ leaves, int nl,
                                                             uint64_t* __restrict__ base)
{
    __shared__ uint64_t ws[kBaseThreads / 64];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int per = (nl + kBaseThreads - 1) / kBaseThreads;
    const int l0 = min(nl, t * per), l1 = min(nl, l0 + per);
    uint64_t s = 0;
    for (int L = l0; L < l1; ++L) s += leaf_slots(leaves[L]);
    uint64_t x = s;   // inclusive scan over the wavefront
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    if (lane == 63) ws[w] = x;
    __syncthreads();
    uint64_t run = x - s;
    for (int v = 0; v < w; ++v) run += ws[v];
    if (t == 0) base[0] = 0;
    for (int L = l0; L < l1; ++L) {
        run += leaf_slots(leaves[L]);
        base[L + 1] = run;
    }
}

}  // namespace

gs_status launch_tile_bases(gs_ctx* ctx, const gs_leaf* leaves_dev, int32_t n_leaves, uint64_t* base)
{
    hipLaunchKernelGGL(k_tile_bases, dim3(1), dim3(kBaseThreads), 0, ctx->stream, leaves_dev, (int)n_leaves, base);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_leaf_toff(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, const gs_leaf* hleaves,
                           int32_t n_leaves, const uint64_t* toff_base, uint64_t* toff)
{
    if (n_leaves > 0) {
        GsTimerScope ts(ctx, "leaf_groups");
        const int nch = leaf_chunks(hleaves, n_leaves);
        std::vector<GsAlloc> tmp;
        uint64_t* csum = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (size_t)nch * n_leaves, GS_MEM_SCRATCH, &tmp);
        if (!csum) return GS_ERR_OOM;
        const dim3 grid((unsigned)nch, (unsigned)n_leaves);
        hipLaunchKernelGGL(k_toff_sums, grid, dim3(256), 0, ctx->stream, leaves_dev, proj->tile_cnt, proj->TW, csum);
        hipLaunchKernelGGL(k_toff_chunk_scan, dim3((unsigned)ceil_div(n_leaves, 256)), dim3(256), 0, ctx->stream,
                           n_leaves, nch, leaves_dev, csum, toff_base, toff);
        hipLaunchKernelGGL(k_toff_write, grid, dim3(256), 0, ctx->stream, leaves_dev, proj->tile_cnt, proj->TW, csum,
                           toff_base, toff);
        gs_free_all(ctx, &tmp);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_plan_offsets(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, int64_t n_entries,
                              const uint32_t* leaf_of, const uint32_t* slot, uint32_t* cell_cnt, uint32_t* cell_off)
{
    GsTimerScope ts(ctx, "leaf_groups");
    if (n_entries > 0)
        hipLaunchKernelGGL(k_group_cells, dim3((unsigned)ceil_div(n_entries, 256)), dim3(256), 0, ctx->stream,
                           n_entries, leaf_of, slot, proj->rect_d, leaves_dev, super_shift(), cell_cnt);
    gs_status st = launch_scan_u32_to_u32(ctx, cell_cnt, cell_off, n_entries);
    if (st != GS_OK) return st;
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_leaf_bounds(gs_ctx* ctx, const gs_leaf* leaves_dev, int32_t n_leaves, const uint64_t* group_off,
                             const uint32_t* cell_off, const uint64_t* toff_base, const uint64_t* toff,
                             uint32_t* leaf_cells, uint64_t* leaf_isect)
{
    if (n_leaves > 0) {
        GsTimerScope ts(ctx, "leaf_groups");
        hipLaunchKernelGGL(k_leaf_cell_bounds, dim3((unsigned)ceil_div(n_leaves, 256)), dim3(256), 0, ctx->stream,
                           n_leaves, group_off, cell_off, leaves_dev, toff_base, toff, leaf_cells, leaf_isect);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_leaf_map(gs_ctx* ctx, const gs_leaf* leaves_dev, const gs_leaf* hleaves, int32_t n_leaves, int TW,
                          int TH, int32_t* lot)
{
    // k_leaf_pairs reads the map only for more than kLeafDirect leaves
    if (n_leaves <= kLeafDirect) return GS_OK;
    // -1 on tiles no leaf covers (a layout that renders part of the view)
    gs_status st = launch_fill_u32(ctx, (uint32_t*)lot, 0xFFFFFFFFu, (int64_t)TW * TH);
    if (st != GS_OK) return st;
    if (n_leaves > 0)
        hipLaunchKernelGGL(k_leaf_map, dim3((unsigned)leaf_chunks(hleaves, n_leaves), (unsigned)n_leaves), dim3(256), 0,
                           ctx->stream, leaves_dev, TW, lot);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_leaf_pairs(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, int32_t n_leaves,
                            const int32_t* lot, uint32_t* cnt, const uint64_t* off, uint32_t* keys, uint32_t* vals)
{
    const int64_t n = proj->n_cand;
    if (n > 0) {
        GsTimerScope ts(ctx, "leaf_groups");
        if (!off)
            hipLaunchKernelGGL(k_leaf_pairs<false>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, n,
                               proj->rect_d, leaves_dev, n_leaves, lot, proj->TW, cnt, off, keys, vals);
        else
            hipLaunchKernelGGL(k_leaf_pairs<true>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, n,
                               proj->rect_d, leaves_dev, n_leaves, lot, proj->TW, cnt, off, keys, vals);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
