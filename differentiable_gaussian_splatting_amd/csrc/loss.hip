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

constexpr int kSB = 256;

// horizontal pass of the five statistics of each channel:
// out[(s * 3 + ch) * P + p], s = x, y, x^2, y^2, xy
__global__ __launch_bounds__(kSB) void k_ssim_h(int W, int H, Win win, const float* __restrict__ x,
                                                const float* __restrict__ y, float* __restrict__ out)
{
    const int64_t P = (int64_t)W * H;
    const int64_t k = (int64_t)blockIdx.x * kSB + threadIdx.x;
    if (k >= 3 * P) return;
    const int ch = (int)(k / P);
    const int64_t p = k % P;
    const int py = (int)(p / W), px = (int)(p % W);
    const float* xr = x + ch * P + (int64_t)py * W;
    const float* yr = y + ch * P + (int64_t)py * W;
    float a = 0.f, b = 0.f, c = 0.f, d = 0.f, e = 0.f;
#pragma unroll
    for (int t = 0; t < 11; ++t) {
        const int q = px + t - 5;
        if (q < 0 || q >= W) continue;
        const float wv = win.w[t], xv = xr[q], yv = yr[q];
        a += wv * xv;
        b += wv * yv;
        c += wv * xv * xv;
        d += wv * yv * yv;
        e += wv * xv * yv;
    }
    out[(0 * 3 + ch) * P + p] = a;
    out[(1 * 3 + ch) * P + p] = b;
    out[(2 * 3 + ch) * P + p] = c;
    out[(3 * 3 + ch) * P + p] = d;
    out[(4 * 3 + ch) * P + p] = e;
}

// Owned rectangle of the buffer: the centres whose SSIM terms (and pixels
// whose L1 terms) are summed, and the pixels whose gradient is written.
struct Owned {
    int x0, y0, x1, y1;
    __device__ bool has(int x, int y) const { return x >= x0 && x < x1 && y >= y0 && y < y1; }
};

// vertical pass + SSIM map + per-pixel partials dS/d(mu_x), dS/d(E[x^2]),
// dS/d(E[xy]) into grad[(s * 3 + ch) * P + p]; block partial sums of S and
// |x - y| over the owned rectangle into part[2 * block], part[2 * block + 1]
__global__ __launch_bounds__(kSB) void k_ssim_v(int W, int H, Win win, Owned own, const float* __restrict__ hs,
                                                const float* __restrict__ x, const float* __restrict__ y,
                                                float* __restrict__ grad, double* __restrict__ part)
{
    const int64_t P = (int64_t)W * H;
    const int64_t k = (int64_t)blockIdx.x * kSB + threadIdx.x;
    double s_sum = 0.0, l1_sum = 0.0;
    if (k < 3 * P) {
        const int ch = (int)(k / P);
        const int64_t p = k % P;
        const int py = (int)(p / W), px = (int)(p % W);
        float st[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 11; ++t) {
            const int q = py + t - 5;
            if (q < 0 || q >= H) continue;
            const float wv = win.w[t];
#pragma unroll
            for (int s = 0; s < 5; ++s) st[s] += wv * hs[(s * 3 + ch) * P + (int64_t)q * W + px];
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
        grad[(0 * 3 + ch) * P + p] = dS_dmx - 2.f * mx * dS_dsxx - my * dS_dsxy;
        grad[(1 * 3 + ch) * P + p] = dS_dsxx;
        grad[(2 * 3 + ch) * P + p] = dS_dsxy;
        if (own.has(px, py)) {
            s_sum = (double)S;
            l1_sum = fabs((double)x[k] - (double)y[k]);
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
        part[2 * blockIdx.x] = a;
        part[2 * blockIdx.x + 1] = b;
    }
}

// horizontal pass of the three partial maps (9 maps)
__global__ __launch_bounds__(kSB) void k_ssim_h2(int W, int H, Win win, const float* __restrict__ in,
                                                 float* __restrict__ out)
{
    const int64_t P = (int64_t)W * H;
    const int64_t k = (int64_t)blockIdx.x * kSB + threadIdx.x;
    if (k >= 9 * P) return;
    const int64_t m = k / P, p = k % P;
    const int py = (int)(p / W), px = (int)(p % W);
    const float* r = in + m * P + (int64_t)py * W;
    float a = 0.f;
#pragma unroll
    for (int t = 0; t < 11; ++t) {
        const int q = px + t - 5;
        if (q >= 0 && q < W) a += win.w[t] * r[q];
    }
    out[k] = a;
}

// vertical pass + gradient of the loss w.r.t. the image (zero outside the
// owned rectangle)
__global__ __launch_bounds__(kSB) void k_ssim_v2(int W, int H, Win win, Owned own, const float* __restrict__ hs,
                                                 const float* __restrict__ x, const float* __restrict__ y,
                                                 float lambda, float inv, float* __restrict__ dl)
{
    const int64_t P = (int64_t)W * H;
    const int64_t k = (int64_t)blockIdx.x * kSB + threadIdx.x;
    if (k >= 3 * P) return;
    const int ch = (int)(k / P);
    const int64_t p = k % P;
    const int py = (int)(p / W), px = (int)(p % W);
    if (!own.has(px, py)) {
        dl[k] = 0.0f;
        return;
    }
    float f[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 11; ++t) {
        const int q = py + t - 5;
        if (q < 0 || q >= H) continue;
        const float wv = win.w[t];
#pragma unroll
        for (int s = 0; s < 3; ++s) f[s] += wv * hs[(s * 3 + ch) * P + (int64_t)q * W + px];
    }
    const float xv = x[k], yv = y[k];
    const float dssim = f[0] + 2.f * xv * f[1] + yv * f[2];
    const float d = xv - yv;
    const float sg = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
    dl[k] = (1.0f - lambda) * sg * inv - lambda * dssim * inv;
}

}  // namespace

gs_status launch_sum_f64(gs_ctx* ctx, const double* in, int64_t n, int stride, double* out, int accumulate)
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
    double* part = (double*)gs_malloc(ctx, sizeof(double) * nb, GS_MEM_SCRATCH, &tmp);
    if (!part) return GS_ERR_OOM;
    hipLaunchKernelGGL(k_sum_chunks, dim3((unsigned)nb), dim3(256), 0, ctx->stream, in, n, stride, per, part);
    hipLaunchKernelGGL(k_sum_f64, dim3(1), dim3(256), 0, ctx->stream, part, nb, 1, out, accumulate);
    gs_free_all(ctx, &tmp);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

int64_t ssim_partial_blocks(int W, int H) { return ceil_div(3 * (int64_t)W * H, kSB); }

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
    const int64_t P = (int64_t)W * H;
    float* bufA = scratch;            // 15 maps
    float* bufB = scratch + 15 * P;   // 9 maps
    const Owned own{ox0, oy0, ox1, oy1};
    GsTimerScope ts(ctx, "ssim");
    hipLaunchKernelGGL(k_ssim_h, dim3((unsigned)ceil_div(3 * P, kSB)), dim3(kSB), 0, ctx->stream, W, H, win, image,
                       target, bufA);
    hipLaunchKernelGGL(k_ssim_v, dim3((unsigned)n_blocks), dim3(kSB), 0, ctx->stream, W, H, win, own, bufA, image,
                       target, bufB, partials);
    hipLaunchKernelGGL(k_ssim_h2, dim3((unsigned)ceil_div(9 * P, kSB)), dim3(kSB), 0, ctx->stream, W, H, win, bufB,
                       bufA);
    hipLaunchKernelGGL(k_ssim_v2, dim3((unsigned)ceil_div(3 * P, kSB)), dim3(kSB), 0, ctx->stream, W, H, win, own,
                       bufA, image, target, lambda, inv, dl_dimage);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
