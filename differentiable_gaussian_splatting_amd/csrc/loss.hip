// loss.hip -- deterministic f64 sums and the L1 + SSIM loss with its
// gradient, over the whole image or over a leaf's rectangle with a halo.
//
// SkipGS notes, "loss function": L = (1 - lambda) L1 + lambda (1 - SSIM),
// lambda = 0.2.  SSIM reading: 11x11 Gaussian window (sigma 1.5, weights
// summing to 1), K1 = 0.01, K2 = 0.03 on a [0, 1] range, zero padding, mean
// over channels and pixels.  The window is separable, so each windowed
// statistic is a horizontal then a vertical 11-tap pass; the gradient pushes
// the per-pixel partials of SSIM back through the same (symmetric, hence
// self-adjoint) zero-padded filter.
//
// Per leaf (the BoundedGS page, "02 / method", notes that windows computed
// inside a leaf differ from the whole image's at its edges): the buffer is
// the leaf's pixel rectangle grown by at least 10 pixels on each side
// (clipped to the image).  A window centred within 5 pixels of the leaf reads
// only pixels within 10 pixels of it, so every centre whose window reaches a
// leaf pixel sees the whole image's values; zero padding at the buffer's
// edges is the image's own where they meet the image border and elsewhere
// only touches centres further than 5 pixels from the leaf, which neither an
// owned term nor an owned pixel's gradient uses.  Each centre's SSIM term is
// summed by the leaf that owns it, so the leaves' sums and gradients are
// those of the whole image.
#include <mutex>

#include "gs_device.h"
#include "gs_internal.h"

namespace {

// one block: out = (accumulate ? out : 0) + sum(in[k * stride]) in a fixed order
__global__ __launch_bounds__(256) void k_sum_f64(const double* __restrict__ in, int64_t n, int stride,
                                                 double* __restrict__ out, int accumulate)
{
    __shared__ double sh[256];
    double s = 0.0;
    for (int64_t k = threadIdx.x; k < n; k += 256) s += in[k * stride];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = (accumulate ? *out : 0.0) + sh[0];
}

// block b: part[b] = sum of in[k * stride] for k in [b * per, (b + 1) * per)
__global__ __launch_bounds__(256) void k_sum_chunks(const double* __restrict__ in, int64_t n, int stride, int64_t per,
                                                    double* __restrict__ part)
{
    __shared__ double sh[256];
    const int64_t k0 = (int64_t)blockIdx.x * per, k1 = min<int64_t>(n, k0 + per);
    double s = 0.0;
    for (int64_t k = k0 + threadIdx.x; k < k1; k += 256) s += in[k * stride];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

struct Win {
    float w[11];
};

// Owned rectangle of the buffer: the centres whose SSIM terms (and pixels
// whose L1 terms) are summed, and the pixels whose gradient is written.
struct Owned {
    int x0, y0, x1, y1;
    __device__ bool has(int x, int y) const { return x >= x0 && x < x1 && y >= y0 && y < y1; }
};

constexpr int kSB = 256;

// Tiles of the two SSIM kernels: 32 x 16 outputs of one channel per
// workgroup, read with a 5-pixel apron (zero outside the buffer) into LDS, so
// that each separable pass reads its taps from LDS and each image or map is
// read from memory about once.  A tap outside the buffer reads the apron's
// zero and adds a zero product: the zero padding, with no compare per tap.
constexpr int kTX = 32, kTY = 16, kR = 5, kIX = kTX + 2 * kR, kIY = kTY + 2 * kR;

__device__ __forceinline__ int64_t ssim_block_id()
{
    return ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
}

// Five windowed statistics of channel ch (horizontal 11-tap pass into LDS,
// then the vertical pass), the SSIM map and the per-pixel partials
// dS/d(mu_x) - 2 mu_x dS/d(sigma_xx) - mu_y dS/d(sigma_xy), dS/d(sigma_xx),
// dS/d(sigma_xy) into grad[(s * 3 + ch) * P + p]; the block's sums of S and
// |x - y| over the owned rectangle into part[2 * block], part[2 * block + 1].
// Each pass adds its 11 taps in order.
__global__ __launch_bounds__(kSB) void k_ssim_stats(int W, int H, Win win, Owned own, const float* __restrict__ x,
                                                    const float* __restrict__ y, float* __restrict__ grad,
                                                    double* __restrict__ part)
{
    __shared__ float sx[kIY][kIX], sy[kIY][kIX];
    __shared__ float hs[5][kIY][kTX];
    const int ch = blockIdx.z;
    const int64_t P = (int64_t)W * H;
    const int x0 = blockIdx.x * kTX, y0 = blockIdx.y * kTY;
    const float* xc = x + ch * P;
    const float* yc = y + ch * P;
    for (int i = threadIdx.x; i < kIX * kIY; i += kSB) {
        const int ly = i / kIX, lx = i % kIX;
        const int gx = x0 + lx - kR, gy = y0 + ly - kR;
        const bool in = gx >= 0 && gx < W && gy >= 0 && gy < H;
        sx[ly][lx] = in ? xc[(int64_t)gy * W + gx] : 0.0f;
        sy[ly][lx] = in ? yc[(int64_t)gy * W + gx] : 0.0f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kIY * kTX; i += kSB) {
        const int ly = i / kTX, lx = i % kTX;
        float a = 0.f, b = 0.f, c = 0.f, d = 0.f, e = 0.f;
#pragma unroll
        for (int t = 0; t < 11; ++t) {
            const float wv = win.w[t], xv = sx[ly][lx + t], yv = sy[ly][lx + t];
            a += wv * xv;
            b += wv * yv;
            c += wv * xv * xv;
            d += wv * yv * yv;
            e += wv * xv * yv;
        }
        hs[0][ly][lx] = a;
        hs[1][ly][lx] = b;
        hs[2][ly][lx] = c;
        hs[3][ly][lx] = d;
        hs[4][ly][lx] = e;
    }
    __syncthreads();
    double s_sum = 0.0, l1_sum = 0.0;
    for (int i = threadIdx.x; i < kTY * kTX; i += kSB) {
        const int ly = i / kTX, lx = i % kTX;
        const int px = x0 + lx, py = y0 + ly;
        if (px >= W || py >= H) continue;
        float st[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 11; ++t) {
            const float wv = win.w[t];
#pragma unroll
            for (int s = 0; s < 5; ++s) st[s] += wv * hs[s][ly + t][lx];
        }
        const float C1 = 0.0001f, C2 = 0.0009f;
        const float mx = st[0], my = st[1];
        const float sxx = st[2] - mx * mx, syy = st[3] - my * my, sxy = st[4] - mx * my;
        const float N1 = 2.f * mx * my + C1, N2 = 2.f * sxy + C2;
        const float D1 = mx * mx + my * my + C1, D2 = sxx + syy + C2;
        const float iD = 1.0f / (D1 * D2);
        const float S = N1 * N2 * iD;
        const float dS_dmx = 2.f * my * N2 * iD - S * 2.f * mx / D1;
        const float dS_dsxx = -S / D2;
        const float dS_dsxy = 2.f * N1 * iD;
        const int64_t p = (int64_t)py * W + px;
        grad[(0 * 3 + ch) * P + p] = dS_dmx - 2.f * mx * dS_dsxx - my * dS_dsxy;
        grad[(1 * 3 + ch) * P + p] = dS_dsxx;
        grad[(2 * 3 + ch) * P + p] = dS_dsxy;
        if (own.has(px, py)) {
            s_sum += (double)S;
            l1_sum += fabs((double)sx[ly + kR][lx + kR] - (double)sy[ly + kR][lx + kR]);
        }
    }
    s_sum = gsd::wave_sum_d(s_sum);
    l1_sum = gsd::wave_sum_d(l1_sum);
    __shared__ double sh[2][kSB / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sh[0][wave] = s_sum;
        sh[1][wave] = l1_sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0, b = 0.0;
        for (int w = 0; w < kSB / 64; ++w) {
            a += sh[0][w];
            b += sh[1][w];
        }
        const int64_t bid = ssim_block_id();
        part[2 * bid] = a;
        part[2 * bid + 1] = b;
    }
}

// The three partial maps of channel ch through the same filter (horizontal
// pass into LDS, then vertical), and the gradient of the loss w.r.t. the
// image (zero outside the owned rectangle).
__global__ __launch_bounds__(kSB) void k_ssim_grad(int W, int H, Win win, Owned own, const float* __restrict__ gm,
                                                   const float* __restrict__ x, const float* __restrict__ y,
                                                   float lambda, float inv, float* __restrict__ dl)
{
    __shared__ float sm[3][kIY][kIX];
    __shared__ float hs[3][kIY][kTX];
    const int ch = blockIdx.z;
    const int64_t P = (int64_t)W * H;
    const int x0 = blockIdx.x * kTX, y0 = blockIdx.y * kTY;
    for (int i = threadIdx.x; i < kIX * kIY; i += kSB) {
        const int ly = i / kIX, lx = i % kIX;
        const int gx = x0 + lx - kR, gy = y0 + ly - kR;
        const bool in = gx >= 0 && gx < W && gy >= 0 && gy < H;
        const int64_t g = (int64_t)gy * W + gx;
#pragma unroll
        for (int s = 0; s < 3; ++s) sm[s][ly][lx] = in ? gm[(s * 3 + ch) * P + g] : 0.0f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kIY * kTX; i += kSB) {
        const int ly = i / kTX, lx = i % kTX;
        float a[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 11; ++t) {
#pragma unroll
            for (int s = 0; s < 3; ++s) a[s] += win.w[t] * sm[s][ly][lx + t];
        }
#pragma unroll
        for (int s = 0; s < 3; ++s) hs[s][ly][lx] = a[s];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTY * kTX; i += kSB) {
        const int ly = i / kTX, lx = i % kTX;
        const int px = x0 + lx, py = y0 + ly;
        if (px >= W || py >= H) continue;
        const int64_t k = ch * P + (int64_t)py * W + px;
        if (!own.has(px, py)) {
            dl[k] = 0.0f;
            continue;
        }
        float f[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 11; ++t) {
            const float wv = win.w[t];
#pragma unroll
            for (int s = 0; s < 3; ++s) f[s] += wv * hs[s][ly + t][lx];
        }
        const float xv = x[k], yv = y[k];
        const float dssim = f[0] + 2.f * xv * f[1] + yv * f[2];
        const float d = xv - yv;
        const float sg = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
        dl[k] = (1.0f - lambda) * sg * inv - lambda * dssim * inv;
    }
}

}  // namespace

namespace {

__global__ void k_view_loss(int kind, const double* __restrict__ sums, double P3, double lambda,
                            double* __restrict__ out)
{
    if (threadIdx.x != 0) return;
    if (kind == 0) {
        out[0] = sums[0] / P3;
    } else {
        const double ssim = sums[0] / P3, l1 = sums[1] / P3;
        out[0] = (1.0 - lambda) * l1 + lambda * (1.0 - ssim);
    }
}

}  // namespace

gs_status launch_view_loss(gs_ctx* ctx, int kind, const double* sums, int64_t P, double lambda, double* out)
{
    hipLaunchKernelGGL(k_view_loss, dim3(1), dim3(64), 0, ctx->stream, kind, sums, 3.0 * (double)P, lambda, out);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_sum_f64(gs_ctx* ctx, const double* in, int64_t n, int stride, double* out, int accumulate,
                         double* chunk_sums)
{
    // two stages for long inputs: up to 256 blocks each sum a contiguous
    // chunk (fixed order), then one block sums the chunk sums
    constexpr int64_t kChunk = 4096;
    if (n <= kChunk) {
        hipLaunchKernelGGL(k_sum_f64, dim3(1), dim3(256), 0, ctx->stream, in, n, stride, out, accumulate);
        GS_HIP(ctx, hipGetLastError());
        return GS_OK;
    }
    const int64_t nb = std::min<int64_t>(256, ceil_div(n, kChunk));
    const int64_t per = ceil_div(n, nb);
    std::vector<GsAlloc> tmp;
    double* part = chunk_sums ? chunk_sums : (double*)gs_malloc(ctx, sizeof(double) * nb, GS_MEM_SCRATCH, &tmp);
    if (!part) return GS_ERR_OOM;
    hipLaunchKernelGGL(k_sum_chunks, dim3((unsigned)nb), dim3(256), 0, ctx->stream, in, n, stride, per, part);
    hipLaunchKernelGGL(k_sum_f64, dim3(1), dim3(256), 0, ctx->stream, part, nb, 1, out, accumulate);
    gs_free_all(ctx, &tmp);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

int64_t ssim_partial_blocks(int W, int H) { return 3 * ceil_div(W, kTX) * ceil_div(H, kTY); }

gs_status launch_ssim(gs_ctx* ctx, int W, int H, int ox0, int oy0, int ox1, int oy1, float inv, const float* image,
                      const float* target, float lambda, float* dl_dimage, double* partials, int64_t n_blocks,
                      float* scratch)
{
    Win win;
    double g[11], s = 0.0;
    for (int i = 0; i < 11; ++i) {
        g[i] = std::exp(-((i - 5) * (i - 5)) / (2.0 * 1.5 * 1.5));
        s += g[i];
    }
    for (int i = 0; i < 11; ++i) win.w[i] = (float)(g[i] / s);
    (void)n_blocks;   // = ssim_partial_blocks(W, H), one pair of sums per workgroup
    const Owned own{ox0, oy0, ox1, oy1};
    const dim3 grid((unsigned)ceil_div(W, kTX), (unsigned)ceil_div(H, kTY), 3);
    GsTimerScope ts(ctx, "ssim");
    hipLaunchKernelGGL(k_ssim_stats, grid, dim3(kSB), 0, ctx->stream, W, H, win, own, image, target, scratch,
                       partials);
    hipLaunchKernelGGL(k_ssim_grad, grid, dim3(kSB), 0, ctx->stream, W, H, win, own, scratch, image, target, lambda,
                       inv, dl_dimage);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

// ---------------------------------------------------------------------------
// Work buffers of gs_loss_ssim_static: one static device array per device the
// library runs on (held until the process ends), so that the SSIM loss can
// run without allocating.  Layout: the 9 per-pixel partial maps of an image
// of up to GS_SSIM_STATIC_MAX_PIXELS pixels, then the two sums of every
// workgroup of the largest grid such an image can take (3 x ceil(W / 32) x
// ceil(H / 16) <= 3 x 131072 for W H <= 2^21), 256 chunk sums and the two
// totals.  Nothing in it accumulates across calls: every value a call reads
// was written earlier in the same call.
namespace {
constexpr int64_t kStaticPixels = GS_SSIM_STATIC_MAX_PIXELS;
constexpr int64_t kStaticBlocks = 3 * (kStaticPixels / kTY);
constexpr size_t kStaticMapBytes = sizeof(float) * 9 * (size_t)kStaticPixels;
constexpr size_t kStaticBytes = kStaticMapBytes + sizeof(double) * (2 * (size_t)kStaticBlocks + 256 + 2);
static_assert(kStaticMapBytes % 256 == 0, "block sums start 256-byte aligned");
constexpr int kStaticDevices = 64;

static __device__ __align__(256) unsigned char ssim_scratch[kStaticBytes];

std::mutex g_static_mu;
unsigned char* g_static_ptr[kStaticDevices] = {};
}  // namespace

gs_status ssim_static_init(gs_ctx* ctx)
{
    if (ctx->device < 0 || ctx->device >= kStaticDevices)
        return gs_fail(ctx, GS_ERR_DEVICE, "device %d beyond the static SSIM buffers' table", ctx->device);
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (g_static_ptr[ctx->device]) return GS_OK;
    // the array's device address on the current device (each device holds
    // its own copy); host code uses this address, never the symbol itself
    void* p = nullptr;
    GS_HIP(ctx, hipGetSymbolAddress(&p, HIP_SYMBOL(ssim_scratch)));
    if (!p) return gs_fail(ctx, GS_ERR_DEVICE, "no device address for the static SSIM buffers");
    g_static_ptr[ctx->device] = (unsigned char*)p;
    return GS_OK;
}

gs_status ssim_static_buffers(gs_ctx* ctx, int W, int H, SsimStatic* out)
{
    if ((int64_t)W * H > kStaticPixels || ssim_partial_blocks(W, H) > kStaticBlocks)
        return gs_fail(ctx, GS_ERR_OVERFLOW, "%d x %d image: the static SSIM buffers hold at most %lld pixels", W,
                       H, (long long)kStaticPixels);
    unsigned char* base = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        if (ctx->device >= 0 && ctx->device < kStaticDevices) base = g_static_ptr[ctx->device];
    }
    if (!base) return gs_fail(ctx, GS_ERR_STATE, "static SSIM buffers not set up on device %d", ctx->device);
    out->maps = (float*)base;
    out->part = (double*)(base + kStaticMapBytes);
    out->chunk = out->part + 2 * kStaticBlocks;
    out->sums = out->chunk + 256;
    return GS_OK;
}
