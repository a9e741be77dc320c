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
    float lr_t, b1, b2, eps, inv_bc2;   // lr_t = lr / (1 - b1^t), inv_bc2 = 1 / (1 - b2^t)
};

// m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
// p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// (hardware reciprocal and square root, 1 ulp)
__device__ __forceinline__ void adam_one(float g, float& p, float& m, float& v, const AdamArgs& a)
{
    m = a.b1 * m + (1.0f - a.b1) * g;
    v = a.b2 * v + (1.0f - a.b2) * g * g;
    p = p - a.lr_t * m * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(v * a.inv_bc2) + a.eps);
}

// Group of `width` consecutive values per Gaussian at column `col0` of the
// compact gradient rows of slots [s0, s1) (row s - s0 in grad3d).  Covers the
// Gaussians [g0, g1) whose candidates are exactly those slots: g0 = 0 or the
// Gaussian of slot s0, g1 = N or the Gaussian of slot s1 (slots are in
// ascending Gaussian order).  Grid-stride, since g0 and g1 are read here.
// Indices are 32-bit (n * width < 2^32, checked by the launcher).  vec: the
// arrays are 16-byte aligned and width is a multiple of 4, so each thread
// takes an aligned float4 of one Gaussian's values.
__global__ __launch_bounds__(256) void k_adam_group(uint32_t n, int64_t n_cand, const uint32_t* __restrict__ ids,
                                                    int64_t s0, int64_t s1, uint32_t width, int col0, int F,
                                                    const int32_t* __restrict__ slot_of,
                                                    const float* __restrict__ grad3d, float* __restrict__ p,
                                                    float* __restrict__ m, float* __restrict__ v, AdamArgs a,
                                                    bool vec)
{
    const uint32_t g0 = s0 == 0 ? 0u : ids[s0];
    const uint32_t g1 = s1 >= n_cand ? n : ids[s1];
    const uint32_t e0 = g0 * width, e1 = g1 * width;
    const uint32_t stride = gridDim.x * blockDim.x;
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (!vec) {
        for (uint32_t k = e0 + t; k < e1; k += stride) {
            const uint32_t i = k / width;
            const int32_t s = slot_of[i];
            const float g = s >= 0 ? grad3d[(int64_t)(s - s0) * F + col0 + (k - i * width)] : 0.0f;
            adam_one(g, p[k], m[k], v[k], a);
        }
        return;
    }
    for (uint32_t k = e0 + 4 * t; k < e1; k += 4 * stride) {
        const uint32_t i = k / width;
        const int32_t s = slot_of[i];
        float4 gg = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (s >= 0) {
            const float* gr = grad3d + (int64_t)(s - s0) * F + col0 + (k - i * width);
            gg = make_float4(gr[0], gr[1], gr[2], gr[3]);
        }
        float4 pp = *reinterpret_cast<const float4*>(p + k);
        float4 mm = *reinterpret_cast<const float4*>(m + k);
        float4 vv = *reinterpret_cast<const float4*>(v + k);
        adam_one(gg.x, pp.x, mm.x, vv.x, a);
        adam_one(gg.y, pp.y, mm.y, vv.y, a);
        adam_one(gg.z, pp.z, mm.z, vv.z, a);
        adam_one(gg.w, pp.w, mm.w, vv.w, a);
        *reinterpret_cast<float4*>(p + k) = pp;
        *reinterpret_cast<float4*>(m + k) = mm;
        *reinterpret_cast<float4*>(v + k) = vv;
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
    a.b1 = b1; a.b2 = b2; a.eps = eps;
    a.lr_t = (float)((double)lr / (1.0 - std::pow((double)b1, (double)step)));
    a.inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)b2, (double)step)));
    struct G { float* p; float* m; float* v; int width, col0; } groups[5] = {
        {p->means, m->means, v->means, 3, 0},
        {p->log_scales, m->log_scales, v->log_scales, 3, 3},
        {p->quats, m->quats, v->quats, 4, 6},
        {p->opacity_logits, m->opacity_logits, v->opacity_logits, 1, 10},
        {p->sh, m->sh, v->sh, 3 * K, 11}};
    if (n <= 0) return GS_OK;
    if ((uint64_t)n * (uint64_t)(3 * K) >= (1ull << 32))
        return gs_fail(ctx, GS_ERR_OVERFLOW, "Adam over %lld Gaussians x %d values exceeds 2^32", (long long)n, 3 * K);
    GsTimerScope ts(ctx, "adam");
    // enough threads for the Gaussians of the slot range (about its share of
    // all Gaussians), at most 8 per compute unit and wavefront slot
    const int64_t share = proj->n_cand > 0 ? ceil_div(n * (s1 - s0), proj->n_cand) : n;
    for (const G& g : groups) {
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(share * g.width, 1024), 8192));
        const bool vec = g.width % 4 == 0 && (((uintptr_t)g.p | (uintptr_t)g.m | (uintptr_t)g.v) & 15u) == 0;
        hipLaunchKernelGGL(k_adam_group, dim3((unsigned)blocks), dim3(256), 0, ctx->stream, (uint32_t)n,
                           proj->n_cand, proj->ids, s0, s1, (uint32_t)g.width, g.col0, F, proj->slot_of, grad3d,
                           g.p, g.m, g.v, a, vec);
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
