// binning.hip -- tile-intersection counting, (tile, depth, slot) ordering of
// one leaf's intersections, and the candidate orders they start from.
//
// BoundedGS page, "01": raster buffers grow with the overlaps of Gaussians
// and image tiles.  Design (MI355X):
//   - once per view the candidates are sorted by depth (stable LSD radix on
//     the f32 depth bits over slots in ascending order), giving the order
//     (depth, slot) that every tile list must follow;
//   - a leaf's candidates are visited in that order; each writes one
//     (leaf-local tile id, slot) pair per tile of its rectangle inside the
//     leaf at an offset from an exclusive scan of the per-candidate tile
//     counts (no atomics; a wavefront shares a wide rectangle so that the
//     writes stay coalesced);
//   - a stable radix sort on the tile id alone (ceil(log2 T_L) bits, two
//     passes for most leaves) then yields each tile's list in (depth, slot)
//     order, and tile offsets come from the key boundaries.
// The per-tile counts of a whole grid (for the planner) come from a 2D
// difference array: four integer atomics per rectangle and a 2D prefix; the
// cells of the first row and column, which every rectangle clamped at the
// image border hits, are aggregated in LDS first.
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

// tiles of each listed candidate's rectangle inside the leaf
__global__ __launch_bounds__(256) void k_count_tiles(int64_t n, const uint32_t* __restrict__ list,
                                                     const int4* __restrict__ rect, int ltx0, int lty0, int ltx1,
                                                     int lty1, uint32_t* __restrict__ cnt)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const int4 r = rect[list[k]];
    const int w = min(r.z, ltx1) - max(r.x, ltx0), h = min(r.w, lty1) - max(r.y, lty0);
    cnt[k] = (w > 0 && h > 0) ? (uint32_t)(w * h) : 0u;
}

constexpr int kOB = 256;     // threads of an emission block
constexpr int kOE = 4096;    // outputs of an emission block

__device__ __forceinline__ int64_t last_le(const uint64_t* __restrict__ a, int64_t n, uint64_t v)
{
    // largest k in [0, n) with a[k] <= v (a non-decreasing, a[0] <= v)
    int64_t lo = 0, hi = n - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (a[mid] <= v) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// (leaf-local tile, slot) pairs of the listed candidates, in list order and
// row-major tile order within a rectangle.  eoff is the exclusive scan of the
// per-candidate tile counts (n + 1 entries).  Each block writes a fixed range
// of kOE consecutive outputs, so the writes are coalesced whatever the
// rectangle sizes; the candidate of an output is found by binary search in an
// LDS copy of the block's part of eoff (or in eoff itself when that part is
// too long, which only long runs of empty candidates cause).
__global__ __launch_bounds__(kOB) void k_emit_pairs(int64_t n, const uint32_t* __restrict__ list,
                                                    const int4* __restrict__ rect, int ltx0, int lty0, int ltx1,
                                                    int lty1, const uint64_t* __restrict__ eoff, uint64_t total,
                                                    uint32_t* __restrict__ keys, uint32_t* __restrict__ vals)
{
    __shared__ uint64_t se[kOE + 1];
    __shared__ int64_t s_c0, s_m;
    const uint64_t o0 = (uint64_t)blockIdx.x * kOE;
    const uint64_t o1 = min<uint64_t>(total, o0 + kOE);
    if (o0 >= o1) return;
    if (threadIdx.x == 0) {
        const int64_t c0 = last_le(eoff, n + 1, o0);
        const int64_t c1 = last_le(eoff, n + 1, o1 - 1);
        s_c0 = c0;
        s_m = c1 - c0 + 1;
    }
    __syncthreads();
    const int64_t c0 = s_c0, m = s_m;
    const bool in_lds = m <= kOE + 1;
    if (in_lds)
        for (int64_t k = threadIdx.x; k < m; k += kOB) se[k] = eoff[c0 + k];
    __syncthreads();
    const int TWL = ltx1 - ltx0;
    for (uint64_t o = o0 + threadIdx.x; o < o1; o += kOB) {
        int64_t c;
        uint64_t start;
        if (in_lds) {
            const int64_t k = last_le(se, m, o);
            c = c0 + k;
            start = se[k];
        } else {
            c = c0 + last_le(eoff + c0, m, o);
            start = eoff[c];
        }
        const uint32_t j = list[c];
        const int4 r = rect[j];
        const int x0 = max(r.x, ltx0) - ltx0, y0 = max(r.y, lty0) - lty0;
        const int w = min(r.z, ltx1) - ltx0 - x0;
        const uint32_t t = (uint32_t)(o - start);
        keys[o] = (uint32_t)((y0 + (int)(t / (uint32_t)w)) * TWL + x0 + (int)(t % (uint32_t)w));
        vals[o] = j;
    }
}

// offsets[s] = first position whose key is >= s, for s in [0, n_seg]; keys
// sorted ascending, all < n_seg.  Four keys per thread.
__global__ __launch_bounds__(256) void k_seg_offsets(const uint32_t* __restrict__ keys, int64_t n, int64_t n_seg,
                                                     uint64_t* __restrict__ offsets)
{
    const int64_t k0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (k0 > n) return;
    int64_t prev = k0 == 0 ? -1 : (int64_t)keys[k0 - 1];
    uint32_t cur4[4];
    if (k0 + 4 <= n && (k0 & 3) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + k0);
        cur4[0] = v.x; cur4[1] = v.y; cur4[2] = v.z; cur4[3] = v.w;
    } else {
        for (int q = 0; q < 4; ++q) cur4[q] = k0 + q < n ? keys[k0 + q] : 0u;
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

__global__ __launch_bounds__(256) void k_depth_pairs(int64_t n, const float4* __restrict__ g2,
                                                     uint32_t* __restrict__ keys, uint32_t* __restrict__ vals)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    keys[j] = __builtin_bit_cast(uint32_t, g2[j].y);   // depth > 0: the bits order like the values
    vals[j] = (uint32_t)j;
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
    if (n > 0) {
        GsTimerScope ts(ctx, "rect_diff");
        hipLaunchKernelGGL(k_rect_diff, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, n, list,
                           proj->rect, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, diff);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_count_tiles(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                             int64_t n_list, uint32_t* cnt)
{
    if (n_list > 0) {
        GsTimerScope ts(ctx, "bin_count");
        hipLaunchKernelGGL(k_count_tiles, dim3((unsigned)ceil_div(n_list, 256)), dim3(256), 0, ctx->stream, n_list,
                           list, proj->rect, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, cnt);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_emit_pairs(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                            int64_t n_list, const uint64_t* eoff, uint64_t total, uint32_t* keys, uint32_t* vals)
{
    if (n_list > 0 && total > 0) {
        GsTimerScope ts(ctx, "emit");
        hipLaunchKernelGGL(k_emit_pairs, dim3((unsigned)ceil_div((int64_t)total, kOE)), dim3(kOB), 0, ctx->stream,
                           n_list, list, proj->rect, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, eoff, total, keys, vals);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_seg_offsets(gs_ctx* ctx, const uint32_t* sorted_keys, int64_t n, int64_t n_seg, uint64_t* offsets)
{
    GsTimerScope ts(ctx, "seg_offsets");
    hipLaunchKernelGGL(k_seg_offsets, dim3((unsigned)ceil_div(ceil_div(n + 1, 4), 256)), dim3(256), 0, ctx->stream,
                       sorted_keys, n, n_seg, offsets);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_depth_pairs(gs_ctx* ctx, const gs_proj* proj, uint32_t* keys, uint32_t* vals)
{
    if (proj->n_cand > 0)
        hipLaunchKernelGGL(k_depth_pairs, dim3((unsigned)ceil_div(proj->n_cand, 256)), dim3(256), 0, ctx->stream,
                           proj->n_cand, proj->g2, keys, vals);
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
