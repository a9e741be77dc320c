// scan.hip -- device-wide exclusive scans, fills and 2D inclusive prefix sums
// (reduce-then-scan over 2048-element tiles; block sums scanned by one block).
#include "gs_device.h"
#include "gs_internal.h"

namespace {

constexpr int kBlock = 256;
constexpr int kItems = 8;
constexpr int kTile = kBlock * kItems;

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane)
{
    for (int o = 1; o < 64; o <<= 1) {
        const T u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// exclusive scan of one value per thread over a 256-thread block; returns the
// block total through *total
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* total)
{
    __shared__ T wsum[kBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T incl = wave_incl_scan(v, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    T before = 0, tot = 0;
    for (int w = 0; w < kBlock / 64; ++w) {
        if (w < wave) before += wsum[w];
        tot += wsum[w];
    }
    __syncthreads();
    *total = tot;
    return before + incl - v;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kBlock) void k_scan_reduce(const TI* __restrict__ in, int64_t n, TO* __restrict__ sums)
{
    const int64_t base = (int64_t)blockIdx.x * kTile;
    TO s = 0;
    for (int k = threadIdx.x; k < kTile; k += kBlock) {
        const int64_t i = base + k;
        if (i < n) s += (TO)in[i];
    }
    TO tot;
    block_excl_scan<TO>(s, &tot);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// one block: exclusive scan of sums[0..nb) in place; total -> *total_out
template <typename TO>
__global__ __launch_bounds__(kBlock) void k_scan_sums(TO* __restrict__ sums, int64_t nb, TO* __restrict__ total_out)
{
    TO carry = 0;
    for (int64_t c = 0; c < nb; c += kTile) {
        TO v[kItems];
        TO loc = 0;
        for (int k = 0; k < kItems; ++k) {
            const int64_t i = c + (int64_t)threadIdx.x * kItems + k;
            v[k] = i < nb ? sums[i] : 0;
            loc += v[k];
        }
        TO tot;
        TO pre = block_excl_scan<TO>(loc, &tot) + carry;
        for (int k = 0; k < kItems; ++k) {
            const int64_t i = c + (int64_t)threadIdx.x * kItems + k;
            if (i < nb) sums[i] = pre;
            pre += v[k];
        }
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) *total_out = carry;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kBlock) void k_scan_apply(const TI* __restrict__ in, int64_t n,
                                                       const TO* __restrict__ block_off, TO* __restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
    TO v[kItems];
    TO loc = 0;
    for (int k = 0; k < kItems; ++k) {
        const int64_t i = base + k;
        v[k] = i < n ? (TO)in[i] : 0;
        loc += v[k];
    }
    TO tot;
    TO pre = block_excl_scan<TO>(loc, &tot) + block_off[blockIdx.x];
    for (int k = 0; k < kItems; ++k) {
        const int64_t i = base + k;
        if (i < n) out[i] = pre;
        pre += v[k];
    }
}

template <typename TI, typename TO>
gs_status scan_impl(gs_ctx* ctx, const TI* in, TO* out, int64_t n, const char* name)
{
    const int64_t nb = n > 0 ? ceil_div(n, kTile) : 0;
    std::vector<GsAlloc> tmp;
    TO* sums = nullptr;
    if (nb > 0) {
        sums = (TO*)gs_malloc(ctx, sizeof(TO) * nb, GS_MEM_SCRATCH, &tmp);
        if (!sums) return GS_ERR_OOM;
        GsTimerScope ts(ctx, name);
        hipLaunchKernelGGL((k_scan_reduce<TI, TO>), dim3((unsigned)nb), dim3(kBlock), 0, ctx->stream, in, n, sums);
    }
    {
        GsTimerScope ts(ctx, name);
        hipLaunchKernelGGL((k_scan_sums<TO>), dim3(1), dim3(kBlock), 0, ctx->stream, sums, nb, out + n);
        if (nb > 0)
            hipLaunchKernelGGL((k_scan_apply<TI, TO>), dim3((unsigned)nb), dim3(kBlock), 0, ctx->stream, in, n,
                               sums, out);
    }
    gs_free_all(ctx, &tmp);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

template <typename T>
__global__ void k_fill(T* __restrict__ p, T v, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

template <typename T>
gs_status fill_impl(gs_ctx* ctx, T* p, T v, int64_t n)
{
    if (n <= 0) return GS_OK;
    const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 8192);
    hipLaunchKernelGGL((k_fill<T>), dim3((unsigned)blocks), dim3(256), 0, ctx->stream, p, v, n);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

// inclusive prefix along each row: one wave per row, 64-wide chunks
template <typename T>
__global__ __launch_bounds__(256) void k_row_prefix(T* __restrict__ g, int rows, int cols)
{
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= rows) return;
    T* row = g + (int64_t)wave * cols;
    T carry = 0;
    for (int c = 0; c < cols; c += 64) {
        const int i = c + lane;
        T v = i < cols ? row[i] : 0;
        v = wave_incl_scan(v, lane) + carry;
        if (i < cols) row[i] = v;
        carry = __shfl(v, 63, 64);
    }
}

// inclusive prefix down each column: a block takes 32 columns, its 32
// wavefront-halves each a chunk of rows (consecutive lanes on consecutive
// columns); chunk sums, then each chunk re-walked with the sums above it
template <typename T>
__global__ __launch_bounds__(1024) void k_col_prefix(T* __restrict__ g, int rows, int cols)
{
    __shared__ T part[32][33];
    const int cx = threadIdx.x & 31, ck = threadIdx.x >> 5;
    const int c = blockIdx.x * 32 + cx;
    const int R = (rows + 31) / 32;
    const int r0 = min(rows, ck * R), r1 = min(rows, r0 + R);
    T s = 0;
    if (c < cols)
        for (int r = r0; r < r1; ++r) s += g[(int64_t)r * cols + c];
    part[ck][cx] = s;
    __syncthreads();
    T acc = 0;
    for (int k = 0; k < ck; ++k) acc += part[k][cx];
    if (c < cols)
        for (int r = r0; r < r1; ++r) {
            acc += g[(int64_t)r * cols + c];
            g[(int64_t)r * cols + c] = acc;
        }
}

template <typename T>
gs_status prefix2d_impl(gs_ctx* ctx, T* g, int rows, int cols)
{
    if (rows <= 0 || cols <= 0) return GS_OK;
    GsTimerScope ts(ctx, "prefix2d");
    hipLaunchKernelGGL((k_row_prefix<T>), dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, ctx->stream, g, rows,
                       cols);
    hipLaunchKernelGGL((k_col_prefix<T>), dim3((unsigned)ceil_div(cols, 32)), dim3(1024), 0, ctx->stream, g, rows,
                       cols);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

}  // namespace

gs_status launch_scan_u32_to_u64(gs_ctx* ctx, const uint32_t* in, uint64_t* out, int64_t n)
{
    return scan_impl<uint32_t, uint64_t>(ctx, in, out, n, "scan");
}

gs_status launch_scan_u32_to_u32(gs_ctx* ctx, const uint32_t* in, uint32_t* out, int64_t n)
{
    return scan_impl<uint32_t, uint32_t>(ctx, in, out, n, "scan");
}

gs_status launch_fill_u32(gs_ctx* ctx, uint32_t* p, uint32_t v, int64_t n) { return fill_impl(ctx, p, v, n); }
gs_status launch_fill_f32(gs_ctx* ctx, float* p, float v, int64_t n) { return fill_impl(ctx, p, v, n); }

gs_status launch_prefix2d_i32(gs_ctx* ctx, int32_t* grid, int rows, int cols)
{
    return prefix2d_impl(ctx, grid, rows, cols);
}

gs_status launch_prefix2d_u64(gs_ctx* ctx, uint64_t* grid, int rows, int cols)
{
    return prefix2d_impl(ctx, grid, rows, cols);
}
