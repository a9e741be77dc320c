// binning.hip -- per-leaf tile-intersection counting, key emission and the
// (tile, depth, slot) sort.
//
// BoundedGS page, "01": raster buffers grow with the overlaps of Gaussians
// and image tiles.  Design (MI355X):
//   1. counts per tile from a 2D difference array: four integer atomics per
//      candidate rectangle, then a 2D inclusive prefix (O(N_c + T), exact);
//   2. exclusive scan of the counts -> u64 tile offsets;
//   3. emission: every (candidate, tile) pair is bucketed into its tile's
//      segment through a per-tile atomic cursor, as the 64-bit composite
//      (depth bits << 32 | slot); candidates whose rectangle covers many tiles
//      are emitted by a whole wavefront so that one thread never carries a
//      large rectangle alone;
//   4. each tile's segment is sorted by the composite (depth, then slot --
//      unique, so the result does not depend on the emission order): bitonic
//      networks in LDS for segments that fit, chunk sorts plus merge-path
//      merges in HBM for longer ones.
// This replaces a global LSD radix sort over (tile << 32 | depth) keys (6-7
// passes over all entries) with about two passes.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

__global__ __launch_bounds__(256) void k_rect_diff(int64_t n, const int4* __restrict__ rect, int ltx0, int lty0,
                                                   int ltx1, int lty1, int32_t* __restrict__ diff)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    const int4 r = rect[j];
    const int TWL = ltx1 - ltx0, THL = lty1 - lty0;
    const int x0 = max(r.x, ltx0) - ltx0, x1 = min(r.z, ltx1) - ltx0;
    const int y0 = max(r.y, lty0) - lty0, y1 = min(r.w, lty1) - lty0;
    if (x0 >= x1 || y0 >= y1) return;
    atomicAdd(&diff[(int64_t)y0 * TWL + x0], 1);
    if (x1 < TWL) atomicAdd(&diff[(int64_t)y0 * TWL + x1], -1);
    if (y1 < THL) atomicAdd(&diff[(int64_t)y1 * TWL + x0], -1);
    if (x1 < TWL && y1 < THL) atomicAdd(&diff[(int64_t)y1 * TWL + x1], 1);
}

constexpr int kWideRect = 32;   // rectangles with more tiles are emitted by a whole wave

__device__ __forceinline__ void emit_one(int64_t t, uint64_t comp, const uint64_t* __restrict__ offsets,
                                         uint32_t* __restrict__ cursor, uint64_t* __restrict__ out)
{
    const uint32_t k = atomicAdd(&cursor[t], 1u);
    out[offsets[t] + k] = comp;
}

__global__ __launch_bounds__(256) void k_emit(int64_t n, const int4* __restrict__ rect,
                                              const float4* __restrict__ g2, int ltx0, int lty0, int ltx1,
                                              int lty1, const uint64_t* __restrict__ offsets,
                                              uint32_t* __restrict__ cursor, uint64_t* __restrict__ out)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = gsd::lane_id();
    const int TWL = ltx1 - ltx0;
    int x0 = 0, x1 = 0, y0 = 0, y1 = 0;
    uint64_t comp = 0;
    if (j < n) {
        const int4 r = rect[j];
        x0 = max(r.x, ltx0) - ltx0; x1 = min(r.z, ltx1) - ltx0;
        y0 = max(r.y, lty0) - lty0; y1 = min(r.w, lty1) - lty0;
        if (x0 >= x1 || y0 >= y1) { x0 = x1 = y0 = y1 = 0; }
        comp = ((uint64_t)__builtin_bit_cast(uint32_t, g2[j].y) << 32) | (uint64_t)(uint32_t)j;
    }
    const int w = x1 - x0, h = y1 - y0;
    const bool wide = w * h > kWideRect;
    if (!wide) {
        for (int ty = y0; ty < y1; ++ty)
            for (int tx = x0; tx < x1; ++tx) emit_one((int64_t)ty * TWL + tx, comp, offsets, cursor, out);
    }
    // wide rectangles: the wave takes them one at a time, lanes stride the tiles
    uint64_t pending = gsd::ballot(wide);
    while (pending) {
        const int src = __builtin_ctzll(pending);
        pending &= pending - 1;
        const int sx0 = __shfl(x0, src, 64), sy0 = __shfl(y0, src, 64);
        const int sw = __shfl(w, src, 64), sh = __shfl(h, src, 64);
        const uint64_t scomp = __shfl(comp, src, 64);
        const int tot = sw * sh;
        for (int k = lane; k < tot; k += 64) {
            const int ty = sy0 + k / sw, tx = sx0 + k % sw;
            emit_one((int64_t)ty * TWL + tx, scomp, offsets, cursor, out);
        }
    }
}

// ---------------------------------------------------------------------------
// per-tile segment sort

template <int CAP>
__device__ __forceinline__ void bitonic_lds(uint64_t* s, int n2)
{
    for (int k = 2; k <= n2; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = threadIdx.x; i < n2; i += blockDim.x) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const uint64_t a = s[i], b = s[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        s[i] = b;
                        s[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int next_pow2(int v)
{
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// segments with lo < len <= CAP: one block, bitonic sort in LDS
template <int CAP>
__global__ __launch_bounds__(1024) void k_sort_lds(int64_t n_tiles, const uint64_t* __restrict__ offsets, const uint64_t* __restrict__ comp,
                           uint32_t* __restrict__ values, int lo)
{
    __shared__ uint64_t s[CAP];
    const int64_t t = blockIdx.x;
    if (t >= n_tiles) return;
    const uint64_t start = offsets[t];
    const int64_t len = (int64_t)(offsets[t + 1] - start);
    if (len <= lo || len > CAP) return;
    if (len == 1) {
        if (threadIdx.x == 0) values[start] = (uint32_t)comp[start];
        return;
    }
    const int n2 = next_pow2((int)len);
    for (int i = threadIdx.x; i < n2; i += blockDim.x) s[i] = i < len ? comp[start + i] : ~0ull;
    __syncthreads();
    bitonic_lds<CAP>(s, n2);
    for (int i = threadIdx.x; i < len; i += blockDim.x) values[start + i] = (uint32_t)s[i];
}

constexpr int kChunk = 8192;

// segments longer than kChunk: one block sorts kChunk chunks in LDS, then
// merges runs pairwise (merge path) between comp and scratch
__global__ __launch_bounds__(1024) void k_sort_big(int64_t n_tiles, const uint64_t* __restrict__ offsets,
                                                   uint64_t* __restrict__ comp, uint64_t* __restrict__ scratch,
                                                   uint32_t* __restrict__ values)
{
    __shared__ uint64_t s[kChunk];
    const int64_t t = blockIdx.x;
    if (t >= n_tiles) return;
    const uint64_t start = offsets[t];
    const int64_t len = (int64_t)(offsets[t + 1] - start);
    if (len <= kChunk) return;
    uint64_t* src = comp + start;
    uint64_t* dst = scratch + start;
    for (int64_t c0 = 0; c0 < len; c0 += kChunk) {
        const int m = (int)min<int64_t>(kChunk, len - c0);
        const int n2 = next_pow2(m);
        for (int i = threadIdx.x; i < n2; i += blockDim.x) s[i] = i < m ? src[c0 + i] : ~0ull;
        __syncthreads();
        bitonic_lds<kChunk>(s, n2);
        for (int i = threadIdx.x; i < m; i += blockDim.x) src[c0 + i] = s[i];
        __syncthreads();
    }
    for (int64_t w = kChunk; w < len; w *= 2) {
        for (int64_t p0 = 0; p0 < len; p0 += 2 * w) {
            const uint64_t* A = src + p0;
            const int64_t la = min<int64_t>(w, len - p0);
            const uint64_t* B = A + la;
            const int64_t lb = min<int64_t>(w, len - p0 - la);
            const int64_t m = la + lb;
            const int64_t per = (m + blockDim.x - 1) / blockDim.x;
            const int64_t k0 = (int64_t)threadIdx.x * per;
            const int64_t k1 = min<int64_t>(m, k0 + per);
            if (k0 < m) {
                int64_t lo = max<int64_t>(0, k0 - lb), hi = min<int64_t>(k0, la);
                while (lo < hi) {
                    const int64_t mid = (lo + hi) >> 1;
                    if (A[mid] < B[k0 - 1 - mid]) lo = mid + 1;
                    else hi = mid;
                }
                int64_t i = lo, j = k0 - lo;
                for (int64_t k = k0; k < k1; ++k) {
                    const bool takeA = i < la && (j >= lb || A[i] < B[j]);
                    dst[p0 + k] = takeA ? A[i++] : B[j++];
                }
            }
        }
        __syncthreads();
        uint64_t* tmp = src;
        src = dst;
        dst = tmp;
    }
    for (int64_t i = threadIdx.x; i < len; i += blockDim.x) values[start + i] = (uint32_t)src[i];
}

__global__ void k_max_segment(const uint64_t* __restrict__ offsets, int64_t n_tiles, uint64_t* __restrict__ out)
{
    uint64_t m = 0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n_tiles; t += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t len = offsets[t + 1] - offsets[t];
        m = len > m ? len : m;
    }
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t v = __shfl_xor(m, o, 64);
        m = v > m ? v : m;
    }
    if (gsd::lane_id() == 0) atomicMax((unsigned long long*)out, (unsigned long long)m);
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

gs_status launch_rect_diff(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, int32_t* diff)
{
    if (proj->n_cand > 0) {
        GsTimerScope ts(ctx, "rect_diff");
        hipLaunchKernelGGL(k_rect_diff, dim3((unsigned)ceil_div(proj->n_cand, 256)), dim3(256), 0, ctx->stream,
                           proj->n_cand, proj->rect, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, diff);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_emit(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* offsets,
                      uint32_t* cursor, uint64_t* comp)
{
    if (proj->n_cand > 0) {
        GsTimerScope ts(ctx, "emit");
        hipLaunchKernelGGL(k_emit, dim3((unsigned)ceil_div(proj->n_cand, 256)), dim3(256), 0, ctx->stream,
                           proj->n_cand, proj->rect, proj->g2, leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, offsets,
                           cursor, comp);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_sort_tiles(gs_ctx* ctx, int64_t n_tiles, const uint64_t* offsets, uint64_t* comp,
                            uint64_t* scratch, uint32_t* values, int64_t max_len)
{
    if (n_tiles <= 0 || max_len <= 0) return GS_OK;
    GsTimerScope ts(ctx, "sort_tiles");
    const dim3 grid((unsigned)n_tiles);
    hipLaunchKernelGGL(k_sort_lds<256>, grid, dim3(64), 0, ctx->stream, n_tiles, offsets, comp, values, 0);
    if (max_len > 256)
        hipLaunchKernelGGL(k_sort_lds<2048>, grid, dim3(256), 0, ctx->stream, n_tiles, offsets, comp, values, 256);
    if (max_len > 2048)
        hipLaunchKernelGGL(k_sort_lds<8192>, grid, dim3(1024), 0, ctx->stream, n_tiles, offsets, comp, values, 2048);
    if (max_len > kChunk)
        hipLaunchKernelGGL(k_sort_big, grid, dim3(1024), 0, ctx->stream, n_tiles, offsets, comp, scratch, values);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_max_segment(gs_ctx* ctx, const uint64_t* offsets, int64_t n_tiles, uint64_t* out)
{
    GS_HIP(ctx, hipMemsetAsync(out, 0, sizeof(uint64_t), ctx->stream));
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>(ceil_div(n_tiles, 256), 1), 1024);
    hipLaunchKernelGGL(k_max_segment, dim3((unsigned)blocks), dim3(256), 0, ctx->stream, offsets, n_tiles, out);
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
