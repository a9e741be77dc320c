// gs_device.h -- device-side helpers for the gfx950 kernels of libgsmi.
//
// Float discipline.  Everything on the forward path (projection, binning
// keys, compositing) is f32 with a fixed operation order: the library is
// built with -ffp-contract=off, correctly rounded f32 division and square
// root, and IEEE denormals; an fma is used only where fmaf() is written.
// This makes every threshold decision (candidate culling, tile rectangles,
// alpha < 1/255, T < 1e-4) reproducible bit for bit by an independent
// implementation of the same specification.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <stdint.h>

namespace gsd {

// ---------------------------------------------------------------------------
// exp by Cody & Waite argument reduction ("Software Manual for the Elementary
// Functions", 1980) with a degree-7 Taylor polynomial:
//   k = rint(x log2 e); r = (x - k ln2_hi) - k ln2_lo; e^r = sum_{n<=7} r^n/n!
//   (Horner, fma); result = ldexp(p, k).
// ln2_hi is ln 2 rounded to f32 with its 12 low significand bits cleared, so
// that k * ln2_hi is exact for |k| < 2^12; ln2_lo = f32(ln 2 - ln2_hi).
// Within 2 ulp of exp over [-87, 88].
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2Hi = __builtin_bit_cast(
    float, __builtin_bit_cast(uint32_t, 0.693147180559945309417232121458f) & 0xFFFFF000u);
constexpr float kLn2Lo = (float)(0.693147180559945309417232121458 - (double)kLn2Hi);
constexpr float kInvFact2 = 1.0f / 2.0f;
constexpr float kInvFact3 = 1.0f / 6.0f;
constexpr float kInvFact4 = 1.0f / 24.0f;
constexpr float kInvFact5 = 1.0f / 120.0f;
constexpr float kInvFact6 = 1.0f / 720.0f;
constexpr float kInvFact7 = 1.0f / 5040.0f;

// core: valid for -87 <= x <= 88.7
__device__ __forceinline__ float exp_cw_core(float x)
{
    const float k = __builtin_rintf(x * kLog2e);
    float r = __builtin_fmaf(-k, kLn2Hi, x);
    r = __builtin_fmaf(-k, kLn2Lo, r);
    float p = kInvFact7;
    p = __builtin_fmaf(p, r, kInvFact6);
    p = __builtin_fmaf(p, r, kInvFact5);
    p = __builtin_fmaf(p, r, kInvFact4);
    p = __builtin_fmaf(p, r, kInvFact3);
    p = __builtin_fmaf(p, r, kInvFact2);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)k);
}

// exp of the Gaussian falloff, for the rasterizer's alpha.  The argument is
// clamped into [-6, 0] first: an entry is included only where
// o exp(power) >= 1/255 with o <= 1, i.e. power > -ln 255 = -5.54, so below -6
// every lane skips the entry whatever value is returned, and above 0 the
// caller skips it too.  On [-6, 0], k is in [-9, 0], which allows
//   t = fma(x, log2 e, 1.5 2^23)   (the sum's ulp is 1: t - 1.5 2^23 is x log2 e
//                                  rounded to the nearest integer k, ties to even)
//   r = fma(-k, ln2, x)            (one f32 ln 2: |k (ln2 - ln2_f32)| < 2e-8)
//   e^r = 1 + r + r^2 (c2 + c3 r + ... + c6 r^4) (Horner, fma), the degree-6
//         polynomial with the least maximum relative error on |r| <= ln2 / 2
//         (4.9e-9 with the f32 coefficients below, under a tenth of an ulp)
//   result = p 2^k, formed by adding k to p's exponent field: the low 9 bits of
//   t's pattern above the significand are those of 1.5 2^23, so (bits(t) << 23)
//   is k << 23 modulo 2^32, and p 2^k stays normal.
// Within 1 ulp of exp over [-6, 0] (every f32 there checked against libm).
// The rasterizer tests the range itself (falloff_in_range) and calls the core
// unclamped: lanes outside the range skip the entry, so their value is unused.
constexpr float kLn2F = 0.693147180559945309417232121458f;
constexpr float kRoundMagic = 12582912.0f;   // 1.5 * 2^23
constexpr float kFall2 = __builtin_bit_cast(float, 0x3efffffeu);   // 0.49999994
constexpr float kFall3 = __builtin_bit_cast(float, 0x3e2aaa2du);   // 0.16666479
constexpr float kFall4 = __builtin_bit_cast(float, 0x3d2aabbeu);   // 0.041667692
constexpr float kFall5 = __builtin_bit_cast(float, 0x3c092e32u);   // 0.0083728302
constexpr float kFall6 = __builtin_bit_cast(float, 0x3ab5dcf3u);   // 0.0013875052
__device__ __forceinline__ float exp_falloff_core(float x)
{
    const float t = __builtin_fmaf(x, kLog2e, kRoundMagic);
    const float k = t - kRoundMagic;
    const float r = __builtin_fmaf(-k, kLn2F, x);
    float p = kFall6;
    p = __builtin_fmaf(p, r, kFall5);
    p = __builtin_fmaf(p, r, kFall4);
    p = __builtin_fmaf(p, r, kFall3);
    p = __builtin_fmaf(p, r, kFall2);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, t) << 23) + __builtin_bit_cast(uint32_t, p));
}

__device__ __forceinline__ float exp_falloff(float x)
{
    return exp_falloff_core(__builtin_amdgcn_fmed3f(x, -6.0f, 0.0f));
}

// -6 <= x <= 0 (NaN: false) in one unsigned compare: 0 - x maps both zeros to
// +0 and keeps the order, and the patterns of +0 .. 6 are 0 .. 0x40C00000
// while negative numbers and NaN lie above.  An entry at power < -6 has
// alpha <= exp(-6) < 1/255 and is skipped, as at power > 0.
__device__ __forceinline__ bool falloff_in_range(float x)
{
    return __builtin_bit_cast(uint32_t, 0.0f - x) <= 0x40C00000u;
}

// exp_cw_core of x inside [-87, 88.7]; 0 below, inf above, NaN kept.  The
// special cases are selects, not branches, so that loads around a call are
// not held back by control flow.
__device__ __forceinline__ float exp_cw(float x)
{
    float r = exp_cw_core(__builtin_amdgcn_fmed3f(x, -87.0f, 88.7f));
    r = x < -87.0f ? 0.0f : r;
    r = x > 88.7f ? __builtin_inff() : r;
    return x != x ? x : r;
}

// compositing constants
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTMin = 0.0001f;

// ---------------------------------------------------------------------------
// Real orthonormal SH basis, degree <= 3, no Condon-Shortley phase, order l
// then m = -l..l, as polynomials in the unit direction (x, y, z).
__device__ __forceinline__ void sh_basis(int deg, float x, float y, float z, float* Y)
{
    Y[0] = 0.282094791773878143f;
    if (deg < 1) return;
    Y[1] = 0.488602511902919921f * y;
    Y[2] = 0.488602511902919921f * z;
    Y[3] = 0.488602511902919921f * x;
    if (deg < 2) return;
    const float xx = x * x, yy = y * y, zz = z * z;
    const float xy = x * y, yz = y * z, xz = x * z;
    Y[4] = 1.09254843059207907f * xy;
    Y[5] = 1.09254843059207907f * yz;
    Y[6] = 0.315391565252520050f * ((2.0f * zz - xx) - yy);
    Y[7] = 1.09254843059207907f * xz;
    Y[8] = 0.546274215296039535f * (xx - yy);
    if (deg < 3) return;
    Y[9] = 0.590043589926643510f * (y * (3.0f * xx - yy));
    Y[10] = 2.89061144264055405f * (xy * z);
    Y[11] = 0.457045799464465739f * (y * ((4.0f * zz - xx) - yy));
    Y[12] = 0.373176332590115391f * (z * ((2.0f * zz - 3.0f * xx) - 3.0f * yy));
    Y[13] = 0.457045799464465739f * (x * ((4.0f * zz - xx) - yy));
    Y[14] = 1.44530572132027703f * (z * (xx - yy));
    Y[15] = 0.590043589926643510f * (x * (xx - 3.0f * yy));
}

// d Y_k / d(x, y, z) of the polynomials above (k = 0..K-1), D[k][3]
__device__ __forceinline__ void sh_basis_grad(int deg, float x, float y, float z, float (*D)[3])
{
    constexpr float c1 = 0.488602511902919921f, c2a = 1.09254843059207907f,
                    c2b = 0.315391565252520050f, c2c = 0.546274215296039535f,
                    c3a = 0.590043589926643510f, c3b = 2.89061144264055405f,
                    c3c = 0.457045799464465739f, c3d = 0.373176332590115391f,
                    c3e = 1.44530572132027703f;
    D[0][0] = D[0][1] = D[0][2] = 0.0f;
    if (deg < 1) return;
    D[1][0] = 0.0f; D[1][1] = c1; D[1][2] = 0.0f;
    D[2][0] = 0.0f; D[2][1] = 0.0f; D[2][2] = c1;
    D[3][0] = c1; D[3][1] = 0.0f; D[3][2] = 0.0f;
    if (deg < 2) return;
    const float xx = x * x, yy = y * y, zz = z * z;
    D[4][0] = c2a * y; D[4][1] = c2a * x; D[4][2] = 0.0f;
    D[5][0] = 0.0f; D[5][1] = c2a * z; D[5][2] = c2a * y;
    D[6][0] = -2.0f * c2b * x; D[6][1] = -2.0f * c2b * y; D[6][2] = 4.0f * c2b * z;
    D[7][0] = c2a * z; D[7][1] = 0.0f; D[7][2] = c2a * x;
    D[8][0] = 2.0f * c2c * x; D[8][1] = -2.0f * c2c * y; D[8][2] = 0.0f;
    if (deg < 3) return;
    D[9][0] = 6.0f * c3a * x * y; D[9][1] = 3.0f * c3a * (xx - yy); D[9][2] = 0.0f;
    D[10][0] = c3b * y * z; D[10][1] = c3b * x * z; D[10][2] = c3b * x * y;
    D[11][0] = -2.0f * c3c * x * y; D[11][1] = c3c * (4.0f * zz - xx - 3.0f * yy); D[11][2] = 8.0f * c3c * y * z;
    D[12][0] = -6.0f * c3d * x * z; D[12][1] = -6.0f * c3d * y * z; D[12][2] = c3d * (6.0f * zz - 3.0f * xx - 3.0f * yy);
    D[13][0] = c3c * (4.0f * zz - 3.0f * xx - yy); D[13][1] = -2.0f * c3c * x * y; D[13][2] = 8.0f * c3c * x * z;
    D[14][0] = 2.0f * c3e * x * z; D[14][1] = -2.0f * c3e * y * z; D[14][2] = c3e * (xx - yy);
    D[15][0] = 3.0f * c3a * (xx - yy); D[15][1] = -6.0f * c3a * x * y; D[15][2] = 0.0f;
}

// ---------------------------------------------------------------------------
// LDS staging of the rows of W floats of a wavefront's mw (<= 64) consecutive
// items (src: the first item's row) into rows of stride RS.  With `aligned`
// (src 16-byte aligned) every lane issues all of its float4 loads before the
// first LDS store, so the loads are in flight together.  need: bit r set for
// the rows that are read later; the others are left unloaded (their LDS
// values are unspecified).
template <int W, int RS>
__device__ __forceinline__ void stage_rows(float* S, const float* __restrict__ src, int mw, int lane, bool aligned,
                                           uint64_t need = ~0ull)
{
    const int nv = mw * W;
    if (!aligned) {
        for (int q = lane; q < nv; q += 64)
            if ((need >> (q / W)) & 1ull) S[(q / W) * RS + q % W] = src[q];
        return;
    }
    constexpr int NQ = (16 * W + 63) / 64;   // float4s per lane
    float t[NQ][4];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const int q = 4 * (lane + 64 * r);
        // the rows the float4 touches (indices clamped into the wavefront's rows)
        const int qa = q < nv ? q : nv - 1, qb = q + 3 < nv ? q + 3 : nv - 1;
        const bool wanted = ((need >> (qa / W)) | (need >> (qb / W))) & 1ull;
        if (!wanted) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t[r][e] = 0.0f;
        } else if (q + 3 < nv) {
            const float4 v = *reinterpret_cast<const float4*>(src + q);
            t[r][0] = v.x;
            t[r][1] = v.y;
            t[r][2] = v.z;
            t[r][3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) t[r][e] = q + e < nv ? src[q + e] : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const int q = 4 * (lane + 64 * r);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (q + e < nv) S[((q + e) / W) * RS + (q + e) % W] = t[r][e];
    }
}

// ---------------------------------------------------------------------------
// Adam (SkipGS notes, "loss function"): one step of one value.
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

// the step-t constants (bias corrections in f64, rounded once)
inline AdamArgs adam_args(int32_t step, float lr, float b1, float b2, float eps)
{
    AdamArgs a;
    a.b1 = b1;
    a.b2 = b2;
    a.eps = eps;
    a.lr_t = (float)((double)lr / (1.0 - std::pow((double)b1, (double)step)));
    a.inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)b2, (double)step)));
    return a;
}

// ---------------------------------------------------------------------------
// wave64 helpers
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The compiler may reorder LDS accesses of one wavefront that it believes do
// not alias; this fence orders them (the hardware keeps a wave's LDS ops in
// order) without a workgroup barrier.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                  BANK_MASK, BOUND));
}

// Sum over the 64 lanes; the total is valid in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v)
{
    v += dpp_f<0xB1>(v);              // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);              // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);             // row_ror:4
    v += dpp_f<0x128>(v);             // row_ror:8
    v += dpp_f<0x142, 0xA>(v);        // row_bcast:15 into rows 1, 3
    v += dpp_f<0x143, 0xC>(v);        // row_bcast:31 into rows 2, 3
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_to_lane63(v)), 63));
}

__device__ __forceinline__ double wave_sum_d(double v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
    for (int o = 32; o > 0; o >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, o, 64);
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// A candidate's tile rectangle [x0, x1) x [y0, y1) in 8 bytes: x0 | y0 << 16
// and (x1 - 1) | (y1 - 1) << 16.  Exact for non-empty rectangles of a grid
// at most 2^16 tiles wide and high (every candidate's, for images up to 2^20
// pixels a side).
__device__ __forceinline__ uint2 rect_pack(int4 r)
{
    return make_uint2((uint32_t)r.x | ((uint32_t)r.y << 16), (uint32_t)(r.z - 1) | ((uint32_t)(r.w - 1) << 16));
}

__device__ __forceinline__ int4 rect_unpack(uint2 p)
{
    return make_int4((int)(p.x & 0xFFFFu), (int)(p.x >> 16), (int)(p.y & 0xFFFFu) + 1, (int)(p.y >> 16) + 1);
}

}  // namespace gsd
