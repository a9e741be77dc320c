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

struct AdamArgs {
    float lr, b1, b2, eps, bc1, bc2;
};

// Group of `width` consecutive values per Gaussian at column `col0` of the
// compact gradient rows of slots [s0, s1) (row s - s0 in grad3d).  Covers the
// Gaussians [g0, g1) whose candidates are exactly those slots: g0 = 0 or the
// Gaussian of slot s0, g1 = N or the Gaussian of slot s1 (slots are in
// ascending Gaussian order).  Grid-stride, since g0 and g1 are read here.
__global__ __launch_bounds__(256) void k_adam_group(int64_t n, int64_t n_cand, const uint32_t* __restrict__ ids,
                                                    int64_t s0, int64_t s1, int width, int col0, int F,
                                                    const int32_t* __restrict__ slot_of,
                                                    const float* __restrict__ grad3d, float* __restrict__ p,
                                                    float* __restrict__ m, float* __restrict__ v, AdamArgs a)
{
    const int64_t g0 = s0 == 0 ? 0 : (int64_t)ids[s0];
    const int64_t g1 = s1 >= n_cand ? n : (int64_t)ids[s1];
    for (int64_t k = g0 * width + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < g1 * width;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = k / width;
        const int c = (int)(k - i * width);
        const int32_t s = slot_of[i];
        const float g = s >= 0 ? grad3d[(int64_t)(s - s0) * F + col0 + c] : 0.0f;
        const float mk = a.b1 * m[k] + (1.0f - a.b1) * g;
        const float vk = a.b2 * v[k] + (1.0f - a.b2) * g * g;
        m[k] = mk;
        v[k] = vk;
        const float mh = mk / a.bc1, vh = vk / a.bc2;
        p[k] = p[k] - a.lr * mh / (sqrtf(vh) + a.eps);
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
    const int F = 11 + 3 * K;
    AdamArgs a;
    a.lr = lr; a.b1 = b1; a.b2 = b2; a.eps = eps;
    a.bc1 = (float)(1.0 - std::pow((double)b1, (double)step));
    a.bc2 = (float)(1.0 - std::pow((double)b2, (double)step));
    struct G { float* p; float* m; float* v; int width, col0; } groups[5] = {
        {p->means, m->means, v->means, 3, 0},
        {p->log_scales, m->log_scales, v->log_scales, 3, 3},
        {p->quats, m->quats, v->quats, 4, 6},
        {p->opacity_logits, m->opacity_logits, v->opacity_logits, 1, 10},
        {p->sh, m->sh, v->sh, 3 * K, 11}};
    if (n <= 0) return GS_OK;
    GsTimerScope ts(ctx, "adam");
    // enough threads for the Gaussians of the slot range (about its share of
    // all Gaussians), at most 8 per compute unit and wavefront slot
    const int64_t share = proj->n_cand > 0 ? ceil_div(n * (s1 - s0), proj->n_cand) : n;
    for (const G& g : groups) {
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(share * g.width, 256), 8192));
        hipLaunchKernelGGL(k_adam_group, dim3((unsigned)blocks), dim3(256), 0, ctx->stream, n, proj->n_cand,
                           proj->ids, s0, s1, g.width, g.col0, F, proj->slot_of, grad3d, g.p, g.m, g.v, a);
    }
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
