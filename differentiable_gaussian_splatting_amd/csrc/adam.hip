// adam.hip -- one Adam step over all N x F parameters from the compact
// per-candidate gradients, and the compact -> dense gradient scatter.
//
// BoundedGS page, "01": the gradient of the whole view is summed before one
// parameter update; SkipGS notes, "loss function": Adam.  Gaussians that are
// not candidates of the view get a zero gradient (their moments still decay,
// as in a dense Adam step over the whole model).  One pass per parameter
// group keeps the parameter and moment streams coalesced.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

using gsd::AdamArgs;
using gsd::adam_one;

// The five parameter groups in one launch: blocks [bend[q-1], bend[q]) update
// group q (means, log-scales, quaternions, opacity logits, SH; W values per
// Gaussian, W a compile-time constant).  Each group covers the Gaussians
// [g0, g1) whose candidates are exactly the slots [s0, s1) of the compact
// gradient rows (row s - s0 of grad3d, the group's values from column col0):
// g0 = 0 or the Gaussian of slot s0, g1 = N or the Gaussian of slot s1 (slots
// are in ascending Gaussian order), read on the device, hence grid-stride
// loops.  The flat value range [g0 W, g1 W) is walked as aligned float4s
// (arrays 16-byte aligned, checked by the launcher; otherwise one value per
// thread), with at most three single values at each end.  Indices are 32-bit
// (N W < 2^32, checked by the launcher).
struct AdamGroup {
    float* p;
    float* m;
    float* v;
    int col0;
    bool vec;
};

struct AdamJob {
    AdamGroup grp[5];
    int bend[5];   // cumulative block counts
};

template <int W>
__device__ __forceinline__ void adam_group(const AdamGroup& gr, int blk, int nblk, uint32_t g0, uint32_t g1,
                                           int64_t s0, int F, const int32_t* __restrict__ slot_of,
                                           const float* __restrict__ grad3d, const AdamArgs& a)
{
    const uint32_t e0 = g0 * (uint32_t)W, e1 = g1 * (uint32_t)W;
    const uint32_t t = (uint32_t)blk * blockDim.x + threadIdx.x;
    const uint32_t stride = (uint32_t)nblk * blockDim.x;
    auto grad = [&](uint32_t k) {
        const uint32_t i = k / (uint32_t)W;
        const int32_t s = slot_of[i];
        return s >= 0 ? grad3d[(int64_t)(s - s0) * F + gr.col0 + (k - i * (uint32_t)W)] : 0.0f;
    };
    auto one = [&](uint32_t k) {
        float p = gr.p[k], m = gr.m[k], v = gr.v[k];
        adam_one(grad(k), p, m, v, a);
        gr.p[k] = p;
        gr.m[k] = m;
        gr.v[k] = v;
    };
    if (!gr.vec) {
        for (uint32_t k = e0 + t; k < e1; k += stride) one(k);
        return;
    }
    const uint32_t a0 = min((e0 + 3u) & ~3u, e1);
    const uint32_t a1 = max(a0, e1 & ~3u);
    if (t < a0 - e0) one(e0 + t);
    if (t < e1 - a1) one(a1 + t);
    for (uint32_t k = a0 + 4u * t; k < a1; k += 4u * stride) {
        float4 pp = *reinterpret_cast<const float4*>(gr.p + k);
        float4 mm = *reinterpret_cast<const float4*>(gr.m + k);
        float4 vv = *reinterpret_cast<const float4*>(gr.v + k);
        const float q0 = grad(k), q1 = grad(k + 1), q2 = grad(k + 2), q3 = grad(k + 3);
        adam_one(q0, pp.x, mm.x, vv.x, a);
        adam_one(q1, pp.y, mm.y, vv.y, a);
        adam_one(q2, pp.z, mm.z, vv.z, a);
        adam_one(q3, pp.w, mm.w, vv.w, a);
        *reinterpret_cast<float4*>(gr.p + k) = pp;
        *reinterpret_cast<float4*>(gr.m + k) = mm;
        *reinterpret_cast<float4*>(gr.v + k) = vv;
    }
}

template <int DEG>
__global__ __launch_bounds__(256) void k_adam(uint32_t n, int64_t n_cand, const uint32_t* __restrict__ ids,
                                              int64_t s0, int64_t s1, const int32_t* __restrict__ slot_of,
                                              const float* __restrict__ grad3d, AdamJob job, AdamArgs a)
{
    constexpr int F = 11 + 3 * (DEG + 1) * (DEG + 1);
    const uint32_t g0 = s0 == 0 ? 0u : ids[s0];
    const uint32_t g1 = s1 >= n_cand ? n : ids[s1];
    const int b = blockIdx.x;
    int q = 0;
    while (q < 4 && b >= job.bend[q]) ++q;
    const int lo = q == 0 ? 0 : job.bend[q - 1];
    const int blk = b - lo, nblk = job.bend[q] - lo;
    switch (q) {
    case 0: adam_group<3>(job.grp[0], blk, nblk, g0, g1, s0, F, slot_of, grad3d, a); break;
    case 1: adam_group<3>(job.grp[1], blk, nblk, g0, g1, s0, F, slot_of, grad3d, a); break;
    case 2: adam_group<4>(job.grp[2], blk, nblk, g0, g1, s0, F, slot_of, grad3d, a); break;
    case 3: adam_group<1>(job.grp[3], blk, nblk, g0, g1, s0, F, slot_of, grad3d, a); break;
    default: adam_group<F - 11>(job.grp[4], blk, nblk, g0, g1, s0, F, slot_of, grad3d, a); break;
    }
}

__global__ __launch_bounds__(256) void k_scatter(int64_t n, int F, const int32_t* __restrict__ slot_of,
                                                 const float* __restrict__ grad3d, float* __restrict__ dense)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n * F) return;
    const int64_t i = k / F;
    const int c = (int)(k - i * F);
    const int32_t s = slot_of[i];
    dense[k] = s >= 0 ? grad3d[(int64_t)s * F + c] : 0.0f;
}

}  // namespace

gs_status launch_adam(gs_ctx* ctx, const gs_proj* proj, int64_t n, int sh_degree, const gs_param_ptrs* p,
                      const gs_param_ptrs* m, const gs_param_ptrs* v, const float* grad3d, int64_t s0, int64_t s1,
                      int32_t step, float lr, float b1, float b2, float eps)
{
    const int K = (sh_degree + 1) * (sh_degree + 1);
    const AdamArgs a = gsd::adam_args(step, lr, b1, b2, eps);
    const int width[5] = {3, 3, 4, 1, 3 * K};
    float* const pp[5] = {p->means, p->log_scales, p->quats, p->opacity_logits, p->sh};
    float* const mp[5] = {m->means, m->log_scales, m->quats, m->opacity_logits, m->sh};
    float* const vp[5] = {v->means, v->log_scales, v->quats, v->opacity_logits, v->sh};
    const int col0[5] = {0, 3, 6, 10, 11};
    if (n <= 0) return GS_OK;
    if ((uint64_t)n * (uint64_t)(3 * K) >= (1ull << 32))
        return gs_fail(ctx, GS_ERR_OVERFLOW, "Adam over %lld Gaussians x %d values exceeds 2^32", (long long)n, 3 * K);
    GsTimerScope ts(ctx, "adam");
    // blocks per group for the Gaussians of the slot range (about its share
    // of all Gaussians): about four float4s per thread, at most 4096 blocks
    const int64_t share = proj->n_cand > 0 ? ceil_div(n * (s1 - s0), proj->n_cand) : n;
    AdamJob job;
    int total = 0;
    for (int q = 0; q < 5; ++q) {
        job.grp[q] = AdamGroup{pp[q], mp[q], vp[q], col0[q],
                               (((uintptr_t)pp[q] | (uintptr_t)mp[q] | (uintptr_t)vp[q]) & 15u) == 0};
        total += (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(share * width[q], 4 * 4 * 256), 4096));
        job.bend[q] = total;
    }
#define GS_ADAM(D) hipLaunchKernelGGL(k_adam<D>, dim3((unsigned)total), dim3(256), 0, ctx->stream, (uint32_t)n, \
                                      proj->n_cand, proj->ids, s0, s1, proj->slot_of, grad3d, job, a)
    switch (sh_degree) {
    case 0: GS_ADAM(0); break;
    case 1: GS_ADAM(1); break;
    case 2: GS_ADAM(2); break;
    default: GS_ADAM(3); break;
    }
#undef GS_ADAM
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_scatter_grad3d(gs_ctx* ctx, const gs_proj* proj, int F, const float* grad3d, float* dense)
{
    if (proj->n > 0)
        hipLaunchKernelGGL(k_scatter, dim3((unsigned)ceil_div(proj->n * F, 256)), dim3(256), 0, ctx->stream, proj->n,
                           F, proj->slot_of, grad3d, dense);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
