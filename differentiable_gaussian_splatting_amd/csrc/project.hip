// project.hip -- EWA projection with candidate compaction, its backward, and
// inspection exports.
//
// BoundedGS page, Fig. 3 C->D->E: projected state and gradients are kept only
// for candidate Gaussians (those that may take part in the view).  Two passes:
// (1) per Gaussian, decide candidacy; (2) after an exclusive scan of the
// decisions (stable, ascending Gaussian id), recompute and write the compact
// state of each candidate at its slot.  Pass 2 recomputes the geometry rather
// than staging it for all N Gaussians, so only candidates cost HBM writes.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

struct CamDev {
    float R[9], t[3], cc[3];
    float fx, fy, cx, cy, near_z, limx, limy;
    int W, H, TW, TH;
};

CamDev make_cam(const gs_camera* c)
{
    CamDev d;
    for (int k = 0; k < 9; ++k) d.R[k] = c->R[k];
    for (int k = 0; k < 3; ++k) d.t[k] = c->t[k];
    // camera centre -R^T t, summed in row order
    for (int k = 0; k < 3; ++k) d.cc[k] = -((d.R[k] * d.t[0] + d.R[3 + k] * d.t[1]) + d.R[6 + k] * d.t[2]);
    d.fx = c->fx; d.fy = c->fy; d.cx = c->cx; d.cy = c->cy; d.near_z = c->near_z;
    d.limx = 1.3f * ((0.5f * (float)c->width) / c->fx);
    d.limy = 1.3f * ((0.5f * (float)c->height) / c->fy);
    d.W = c->width; d.H = c->height;
    d.TW = (c->width + 15) / 16; d.TH = (c->height + 15) / 16;
    return d;
}

struct Proj2D {
    bool ok;
    float x, y, A, B, C, r, depth;
    int tx0, ty0, tx1, ty1;
    uint32_t flags;
    float vx, vy, vz;   // mean - camera centre (for the colour direction)
};

__device__ __forceinline__ float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The inputs of one Gaussian's projection, loaded together (no load waits on
// an earlier decision).
struct GaussIn {
    float mx, my, mz, l0, l1, l2;
    float4 q;
};

__device__ __forceinline__ GaussIn load_gauss(const float* __restrict__ means, const float* __restrict__ log_scales,
                                              const float* __restrict__ quats, int64_t i)
{
    GaussIn g;
    g.mx = means[3 * i];
    g.my = means[3 * i + 1];
    g.mz = means[3 * i + 2];
    g.l0 = log_scales[3 * i];
    g.l1 = log_scales[3 * i + 1];
    g.l2 = log_scales[3 * i + 2];
    g.q = *reinterpret_cast<const float4*>(quats + 4 * i);
    return g;
}

// Geometry of one Gaussian in the specified f32 operation order.
__device__ __forceinline__ Proj2D project_geom(const CamDev& cam, const GaussIn& gi)
{
    Proj2D o;
    o.ok = true;
    o.flags = 0;
    const float mx = gi.mx, my = gi.my, mz = gi.mz;
    const float px = ((cam.R[0] * mx + cam.R[1] * my) + cam.R[2] * mz) + cam.t[0];
    const float py = ((cam.R[3] * mx + cam.R[4] * my) + cam.R[5] * mz) + cam.t[1];
    const float pz = ((cam.R[6] * mx + cam.R[7] * my) + cam.R[8] * mz) + cam.t[2];
    o.depth = pz;
    o.vx = mx - cam.cc[0];
    o.vy = my - cam.cc[1];
    o.vz = mz - cam.cc[2];
    if (!(pz > cam.near_z)) { o.ok = false; return o; }

    const float s0 = gsd::exp_cw(gi.l0);
    const float s1 = gsd::exp_cw(gi.l1);
    const float s2 = gsd::exp_cw(gi.l2);
    const float4 q = gi.q;
    const float qn = sqrtf(((q.x * q.x + q.y * q.y) + q.z * q.z) + q.w * q.w);
    const float w = q.x / qn, x = q.y / qn, y = q.z / qn, z = q.w / qn;
    float Rq[3][3];
    Rq[0][0] = 1.0f - 2.0f * (y * y + z * z);
    Rq[0][1] = 2.0f * (x * y - w * z);
    Rq[0][2] = 2.0f * (x * z + w * y);
    Rq[1][0] = 2.0f * (x * y + w * z);
    Rq[1][1] = 1.0f - 2.0f * (x * x + z * z);
    Rq[1][2] = 2.0f * (y * z - w * x);
    Rq[2][0] = 2.0f * (x * z - w * y);
    Rq[2][1] = 2.0f * (y * z + w * x);
    Rq[2][2] = 1.0f - 2.0f * (x * x + y * y);
    const float s[3] = {s0, s1, s2};
    float M[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) M[r][c] = Rq[r][c] * s[c];
    float Sg[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = r; c < 3; ++c) {
            Sg[r][c] = (M[r][0] * M[c][0] + M[r][1] * M[c][1]) + M[r][2] * M[c][2];
            Sg[c][r] = Sg[r][c];
        }
    const float u = px / pz, v = py / pz;
    float ux = u, uy = v;
    if (ux < -cam.limx) { ux = -cam.limx; o.flags |= 8u; }
    else if (ux > cam.limx) { ux = cam.limx; o.flags |= 8u; }
    if (uy < -cam.limy) { uy = -cam.limy; o.flags |= 16u; }
    else if (uy > cam.limy) { uy = cam.limy; o.flags |= 16u; }
    const float J00 = cam.fx / pz, J02 = -((cam.fx * ux) / pz);
    const float J11 = cam.fy / pz, J12 = -((cam.fy * uy) / pz);
    float T[2][3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        T[0][c] = J00 * cam.R[c] + J02 * cam.R[6 + c];
        T[1][c] = J11 * cam.R[3 + c] + J12 * cam.R[6 + c];
    }
    float U[2][3];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 3; ++c) U[a][c] = (T[a][0] * Sg[0][c] + T[a][1] * Sg[1][c]) + T[a][2] * Sg[2][c];
    const float s00 = (U[0][0] * T[0][0] + U[0][1] * T[0][1]) + U[0][2] * T[0][2];
    const float s01 = (U[0][0] * T[1][0] + U[0][1] * T[1][1]) + U[0][2] * T[1][2];
    const float s11 = (U[1][0] * T[1][0] + U[1][1] * T[1][1]) + U[1][2] * T[1][2];
    const float a = s00 + 0.3f, b = s01, c = s11 + 0.3f;
    const float det = a * c - b * b;
    if (!(det > 0.0f)) { o.ok = false; return o; }
    o.A = c / det;
    o.B = -(b / det);
    o.C = a / det;
    const float mid = 0.5f * (a + c);
    float disc = mid * mid - det;
    disc = disc > 0.1f ? disc : 0.1f;
    const float lam = mid + sqrtf(disc);
    o.r = ceilf(3.0f * sqrtf(lam));
    o.x = cam.fx * u + cam.cx;
    o.y = cam.fy * v + cam.cy;
    if (!(isfinite(o.x) && isfinite(o.y) && isfinite(o.A) && isfinite(o.B) && isfinite(o.C) && isfinite(o.r))) {
        o.ok = false;
        return o;
    }
    o.tx0 = (int)clampf(floorf((o.x - o.r) * 0.0625f), 0.0f, (float)cam.TW);
    o.tx1 = (int)clampf(floorf((o.x + o.r) * 0.0625f) + 1.0f, 0.0f, (float)cam.TW);
    o.ty0 = (int)clampf(floorf((o.y - o.r) * 0.0625f), 0.0f, (float)cam.TH);
    o.ty1 = (int)clampf(floorf((o.y + o.r) * 0.0625f) + 1.0f, 0.0f, (float)cam.TH);
    if (o.tx0 >= o.tx1 || o.ty0 >= o.ty1) o.ok = false;
    return o;
}

// dkey (optional): each Gaussian's depth bits (the depth sort's key; the
// same value the compact state's depth gets)
__global__ __launch_bounds__(256) void k_project_flags(CamDev cam, int64_t n, const float* __restrict__ means,
                                                       const float* __restrict__ log_scales,
                                                       const float* __restrict__ quats, uint32_t* __restrict__ flag,
                                                       uint32_t* __restrict__ dkey)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const auto g = project_geom(cam, load_gauss(means, log_scales, quats, i));
    flag[i] = g.ok ? 1u : 0u;
    if (dkey) dkey[i] = __builtin_bit_cast(uint32_t, g.depth);
}

// Compact state of every candidate.  A wavefront covers 64 consecutive
// Gaussians; their SH rows are contiguous, so the wave stages them in LDS with
// coalesced loads (row stride 3K + 1 floats keeps the per-lane row reads free
// of bank conflicts) before each lane evaluates its colour.
template <int DEG>
__global__ __launch_bounds__(256) void k_project_write(CamDev cam, int64_t n, const float* __restrict__ means,
                                                       const float* __restrict__ log_scales,
                                                       const float* __restrict__ quats,
                                                       const float* __restrict__ logits,
                                                       const float* __restrict__ sh, bool sh_aligned,
                                                       const uint32_t* __restrict__ flag,
                                                       const uint32_t* __restrict__ slot, uint32_t* __restrict__ ids,
                                                       int4* __restrict__ rect, float4* __restrict__ g0,
                                                       float4* __restrict__ g1, float4* __restrict__ g2,
                                                       int32_t* __restrict__ slot_of)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    constexpr int RS = 3 * K + 1;
    __shared__ float shs[4][64 * RS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w0 = (int64_t)blockIdx.x * blockDim.x + wave * 64;
    const int64_t i = w0 + lane;
    float* S = shs[wave];
    // every input of the lane's Gaussian is requested before the SH rows are
    // staged, so that all loads of the wavefront are in flight together
    const bool live = i < n;
    GaussIn gi{};
    uint32_t cand = 0, j = 0;
    float logit = 0.0f;
    if (live) {
        gi = load_gauss(means, log_scales, quats, i);
        cand = flag[i];
        j = slot[i];
        logit = logits[i];
    }
    // only the candidates' SH rows are read (a wavefront's rows are contiguous:
    // a row beside a candidate's shares its cache lines, the others are
    // skipped)
    const uint64_t need = gsd::ballot(cand != 0);
    if (w0 < n)
        gsd::stage_rows<3 * K, RS>(S, sh + w0 * 3 * K, (int)(n - w0 < 64 ? n - w0 : 64), lane, sh_aligned, need);
    gsd::wave_sync();
    if (!live) return;
    if (!cand) {
        slot_of[i] = -1;
        return;
    }
    slot_of[i] = (int32_t)j;
    const Proj2D p = project_geom(cam, gi);
    const float o = 1.0f / (1.0f + gsd::exp_cw(-logit));
    const float vn = sqrtf((p.vx * p.vx + p.vy * p.vy) + p.vz * p.vz);
    const float dx = p.vx / vn, dy = p.vy / vn, dz = p.vz / vn;
    float Y[16];
    gsd::sh_basis(DEG, dx, dy, dz, Y);
    const float* shi = S + lane * RS;
    float rgb[3];
    uint32_t fl = p.flags;
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) {
        float acc = Y[0] * shi[ch];
#pragma unroll
        for (int k = 1; k < K; ++k) acc = acc + Y[k] * shi[3 * k + ch];
        acc = acc + 0.5f;
        if (acc < 0.0f) {
            acc = 0.0f;
            fl |= (1u << ch);
        }
        rgb[ch] = acc;
    }
    ids[j] = (uint32_t)i;
    rect[j] = make_int4(p.tx0, p.ty0, p.tx1, p.ty1);
    g0[j] = make_float4(p.x, p.y, -0.5f * p.A, -p.B);
    g1[j] = make_float4(-0.5f * p.C, o, rgb[0], rgb[1]);
    g2[j] = make_float4(rgb[2], p.depth, p.r, __builtin_bit_cast(float, fl));
}

// ---------------------------------------------------------------------------
// Projection backward of one candidate, Gaussian i (f32): the chain rule
// through each step of the projection, with the forward's clamp decisions
// (flags fl).  g: the candidate's 9 screen-space partials (mean2d, conic,
// opacity, colour).  shi: its 3K SH coefficients (device memory or LDS).
// Out: geo[0..10] = dL/d(mean, log-scale, quaternion, opacity logit), Y[0..K-1]
// = the SH basis at the view direction and grm[3] = dL/drgb, zero where the
// forward clamped the channel; dL/dsh[k][c] = Y[k] grm[c].
template <int DEG>
__device__ __forceinline__ void proj_bwd_one(const CamDev& cam, const GaussIn& gi, float logit, uint32_t fl,
                                             const float* g, const float* shi, float* geo, float* Y, float* grm)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    // forward recomputation
    const float mu[3] = {gi.mx, gi.my, gi.mz};
    float p[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) p[r] = cam.R[3 * r] * mu[0] + cam.R[3 * r + 1] * mu[1] + cam.R[3 * r + 2] * mu[2] + cam.t[r];
    const float pz = p[2];
    float s[3];
    s[0] = gsd::exp_cw(gi.l0);
    s[1] = gsd::exp_cw(gi.l1);
    s[2] = gsd::exp_cw(gi.l2);
    const float4 q = gi.q;
    const float qn = sqrtf(q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w);
    const float w = q.x / qn, x = q.y / qn, y = q.z / qn, z = q.w / qn;
    float Rq[3][3];
    Rq[0][0] = 1.0f - 2.0f * (y * y + z * z); Rq[0][1] = 2.0f * (x * y - w * z); Rq[0][2] = 2.0f * (x * z + w * y);
    Rq[1][0] = 2.0f * (x * y + w * z); Rq[1][1] = 1.0f - 2.0f * (x * x + z * z); Rq[1][2] = 2.0f * (y * z - w * x);
    Rq[2][0] = 2.0f * (x * z - w * y); Rq[2][1] = 2.0f * (y * z + w * x); Rq[2][2] = 1.0f - 2.0f * (x * x + y * y);
    float M[3][3], Sg[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) M[r][c] = Rq[r][c] * s[c];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int c = 0; c < 3; ++c) Sg[r][c] = M[r][0] * M[c][0] + M[r][1] * M[c][1] + M[r][2] * M[c][2];
    const float u = p[0] / pz, v = p[1] / pz;
    const bool clx = (fl & 8u) != 0, cly = (fl & 16u) != 0;
    const float ux = clx ? (u < 0.0f ? -cam.limx : cam.limx) : u;
    const float uy = cly ? (v < 0.0f ? -cam.limy : cam.limy) : v;
    const float iz = 1.0f / pz;
    const float J00 = cam.fx * iz, J02 = -cam.fx * ux * iz, J11 = cam.fy * iz, J12 = -cam.fy * uy * iz;
    float T[2][3], U[2][3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        T[0][c] = J00 * cam.R[c] + J02 * cam.R[6 + c];
        T[1][c] = J11 * cam.R[3 + c] + J12 * cam.R[6 + c];
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 3; ++c) U[a][c] = T[a][0] * Sg[0][c] + T[a][1] * Sg[1][c] + T[a][2] * Sg[2][c];
    const float a = U[0][0] * T[0][0] + U[0][1] * T[0][1] + U[0][2] * T[0][2] + 0.3f;
    const float b = U[0][0] * T[1][0] + U[0][1] * T[1][1] + U[0][2] * T[1][2];
    const float c = U[1][0] * T[1][0] + U[1][1] * T[1][1] + U[1][2] * T[1][2] + 0.3f;
    const float det = a * c - b * b;
    const float o = 1.0f / (1.0f + gsd::exp_cw(-logit));
    const float vx = mu[0] - cam.cc[0], vy = mu[1] - cam.cc[1], vz = mu[2] - cam.cc[2];
    const float vn = sqrtf(vx * vx + vy * vy + vz * vz);
    const float d[3] = {vx / vn, vy / vn, vz / vn};

    // mean2d = (fx u + cx, fy v + cy)
    float dp[3];
    const float du = cam.fx * g[0], dv = cam.fy * g[1];
    dp[0] = du * iz;
    dp[1] = dv * iz;
    dp[2] = -(du * u + dv * v) * iz;
    // conic = (c, -b, a) / det
    const float dA = g[2], dB = g[3], dC = g[4];
    const float idet2 = 1.0f / (det * det);
    const float da = (-c * c * dA + b * c * dB - b * b * dC) * idet2;
    const float db = (2.0f * b * c * dA - (a * c + b * b) * dB + 2.0f * a * b * dC) * idet2;
    const float dc = (-b * b * dA + a * b * dB - a * a * dC) * idet2;
    // Sigma2 entries (0,0), (0,1), (1,1) = U T^T
    float dU[2][3], dT[2][3], dSg[3][3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        dU[0][k] = da * T[0][k] + db * T[1][k];
        dU[1][k] = dc * T[1][k];
        dT[0][k] = da * U[0][k];
        dT[1][k] = db * U[0][k] + dc * U[1][k];
    }
    // U = T Sigma
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) dSg[k][cc] = T[0][k] * dU[0][cc] + T[1][k] * dU[1][cc];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            dT[aa][k] += dU[aa][0] * Sg[k][0] + dU[aa][1] * Sg[k][1] + dU[aa][2] * Sg[k][2];
    // T = J R
    float dJ00 = 0.0f, dJ02 = 0.0f, dJ11 = 0.0f, dJ12 = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        dJ00 += dT[0][k] * cam.R[k];
        dJ02 += dT[0][k] * cam.R[6 + k];
        dJ11 += dT[1][k] * cam.R[3 + k];
        dJ12 += dT[1][k] * cam.R[6 + k];
    }
    const float iz2 = iz * iz;
    dp[2] += -cam.fx * iz2 * dJ00 + cam.fx * ux * iz2 * dJ02 - cam.fy * iz2 * dJ11 + cam.fy * uy * iz2 * dJ12;
    const float dux = -cam.fx * iz * dJ02, duy = -cam.fy * iz * dJ12;
    if (!clx) { dp[0] += dux * iz; dp[2] -= dux * u * iz; }
    if (!cly) { dp[1] += duy * iz; dp[2] -= duy * v * iz; }
    // Sigma = M M^T
    float dM[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc)
            dM[r][cc] = (dSg[r][0] + dSg[0][r]) * M[0][cc] + (dSg[r][1] + dSg[1][r]) * M[1][cc] +
                        (dSg[r][2] + dSg[2][r]) * M[2][cc];
    float dRq[3][3], ds[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) {
            dRq[r][cc] = dM[r][cc] * s[cc];
            ds[cc] += dM[r][cc] * Rq[r][cc];
        }
    geo[3] = ds[0] * s[0];
    geo[4] = ds[1] * s[1];
    geo[5] = ds[2] * s[2];
    // rotation of the unit quaternion (w, x, y, z)
    float gw = 0.0f, gx = 0.0f, gy = 0.0f, gz = 0.0f;
    gy += -4.0f * y * dRq[0][0]; gz += -4.0f * z * dRq[0][0];
    gx += 2.0f * y * dRq[0][1]; gy += 2.0f * x * dRq[0][1]; gw += -2.0f * z * dRq[0][1]; gz += -2.0f * w * dRq[0][1];
    gx += 2.0f * z * dRq[0][2]; gz += 2.0f * x * dRq[0][2]; gw += 2.0f * y * dRq[0][2]; gy += 2.0f * w * dRq[0][2];
    gx += 2.0f * y * dRq[1][0]; gy += 2.0f * x * dRq[1][0]; gw += 2.0f * z * dRq[1][0]; gz += 2.0f * w * dRq[1][0];
    gx += -4.0f * x * dRq[1][1]; gz += -4.0f * z * dRq[1][1];
    gy += 2.0f * z * dRq[1][2]; gz += 2.0f * y * dRq[1][2]; gw += -2.0f * x * dRq[1][2]; gx += -2.0f * w * dRq[1][2];
    gx += 2.0f * z * dRq[2][0]; gz += 2.0f * x * dRq[2][0]; gw += -2.0f * y * dRq[2][0]; gy += -2.0f * w * dRq[2][0];
    gy += 2.0f * z * dRq[2][1]; gz += 2.0f * y * dRq[2][1]; gw += 2.0f * x * dRq[2][1]; gx += 2.0f * w * dRq[2][1];
    gx += -4.0f * x * dRq[2][2]; gy += -4.0f * y * dRq[2][2];
    const float dot = w * gw + x * gx + y * gy + z * gz;
    const float iqn = 1.0f / qn;
    geo[6] = (gw - w * dot) * iqn;
    geo[7] = (gx - x * dot) * iqn;
    geo[8] = (gy - y * dot) * iqn;
    geo[9] = (gz - z * dot) * iqn;
    geo[10] = g[5] * o * (1.0f - o);
    // colour: rgb = 0.5 + sum_k Y_k(d) sh_k, masked where clamped
    float D[16][3];
    gsd::sh_basis(DEG, d[0], d[1], d[2], Y);
    gsd::sh_basis_grad(DEG, d[0], d[1], d[2], D);
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) grm[ch] = (fl & (1u << ch)) ? 0.0f : g[6 + ch];
    float dd0 = 0.0f, dd1 = 0.0f, dd2 = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float t = 0.0f;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) t += shi[3 * k + ch] * grm[ch];
        dd0 += t * D[k][0];
        dd1 += t * D[k][1];
        dd2 += t * D[k][2];
    }
    const float ddot = d[0] * dd0 + d[1] * dd1 + d[2] * dd2;
    const float ivn = 1.0f / vn;
    float dmu[3] = {(dd0 - d[0] * ddot) * ivn, (dd1 - d[1] * ddot) * ivn, (dd2 - d[2] * ddot) * ivn};
#pragma unroll
    for (int e = 0; e < 3; ++e) dmu[e] += cam.R[e] * dp[0] + cam.R[3 + e] * dp[1] + cam.R[6 + e] * dp[2];
    geo[0] = dmu[0];
    geo[1] = dmu[1];
    geo[2] = dmu[2];
}

// Projection backward, one thread per candidate slot in [s0, s_end); row
// j - s0 of grad3d gets the candidate's F partials.
template <int DEG>
__global__ __launch_bounds__(256) void k_project_bwd(CamDev cam, int64_t s0, int64_t s_end,
                                                     const float* __restrict__ means,
                                                     const float* __restrict__ log_scales,
                                                     const float* __restrict__ quats,
                                                     const float* __restrict__ logits, const float* __restrict__ sh,
                                                     const uint32_t* __restrict__ ids,
                                                     const float4* __restrict__ g2s,
                                                     const float* __restrict__ grad2d, float* __restrict__ grad3d)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    constexpr int F = 11 + 3 * K;
    // the wave's 64 output rows are contiguous in grad3d: stage them in LDS
    // (odd row stride) and write them out coalesced at the end
    constexpr int RS = F | 1;
    __shared__ float outs[4][64 * RS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w0 = s0 + (int64_t)blockIdx.x * blockDim.x + wave * 64;   // slots [s0, s_end)
    const int64_t j = w0 + lane;
    float* out = outs[wave] + lane * RS;
    if (j < s_end) {
        const int64_t i = ids[j];
        const uint32_t fl = __builtin_bit_cast(uint32_t, g2s[j].w);
        float Y[16], grm[3];
        proj_bwd_one<DEG>(cam, load_gauss(means, log_scales, quats, i), logits[i], fl, grad2d + 9 * j,
                          sh + (int64_t)3 * K * i, out, Y, grm);
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) out[11 + 3 * k + ch] = Y[k] * grm[ch];
    }
    gsd::wave_sync();
    const int64_t rows = s_end - w0 < 64 ? s_end - w0 : 64;
    if (rows > 0) {
        float* dst = grad3d + (w0 - s0) * F;   // row j - s0
        const float* src = outs[wave];
        for (int q = lane; q < rows * F; q += 64) dst[q] = src[(q / F) * RS + q % F];
    }
}

// ---------------------------------------------------------------------------
// Projection backward fused with the Adam step, over all N Gaussians (one
// Adam step per view over the summed gradient, BoundedGS page, "01"; SkipGS
// notes, "loss function": Adam; Gaussians that are not candidates of the view
// get a zero gradient).  A wavefront takes 64 consecutive Gaussians:
//   1. their SH rows are staged in LDS with coalesced loads;
//   2. each lane runs the projection backward of its Gaussian if it is a
//      candidate (SH coefficients from LDS), giving its 11 geometric partials
//      and the factors Y[k], dL/drgb[c] of its SH partials Y[k] dL/drgb[c];
//   3. the factors replace the staged rows in LDS, and the lane updates its
//      Gaussian's 11 geometric values;
//   4. the wavefront updates its 64 SH rows as aligned float4s (the rows of
//      64 Gaussians start on a 256-byte boundary), each value's partial
//      formed from the two LDS factors.
// No gradient array is written, and each parameter and moment crosses HBM
// once each way.  The backward reads the parameters through `means` ... `sh`
// and Adam updates `pw`; the two may be the same arrays (a Gaussian's values
// are read by its own wavefront before that wavefront writes them).
struct AdamPtrs {
    float* p[5];   // means, log-scales, quaternions, opacity logits, SH
    float* m[5];
    float* v[5];
    bool vec;      // every array 16-byte aligned
};

template <int DEG>
__global__ __launch_bounds__(256) void k_bwd_adam(CamDev cam, int64_t n, const float* __restrict__ means,
                                                  const float* __restrict__ log_scales,
                                                  const float* __restrict__ quats, const float* __restrict__ logits,
                                                  const float* __restrict__ sh, bool sh_aligned,
                                                  const int32_t* __restrict__ slot_of,
                                                  const float4* __restrict__ g2s, const float* __restrict__ grad2d,
                                                  AdamPtrs pw, gsd::AdamArgs a)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    constexpr int W = 3 * K;    // SH values per Gaussian
    constexpr int RS = W + 1;   // LDS row of a staged SH row (odd stride: per-lane rows without bank conflicts)
    constexpr int RT = K + 3;   // LDS row of the SH partial factors: Y[0..K-1], dL/drgb[0..2]
    __shared__ float shs[4][64 * RS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
    if (w0 >= n) return;
    const int mw = (int)(n - w0 < 64 ? n - w0 : 64);   // Gaussians of this wavefront
    const int64_t i = w0 + lane;
    const bool live = lane < mw;
    float* S = shs[wave];
    // the lane's slot and projection inputs are requested before the SH rows
    // are staged, so that these loads are in flight together
    GaussIn gi{};
    float logit = 0.0f;
    const int32_t s = live ? slot_of[i] : -1;
    if (live) {
        gi = load_gauss(means, log_scales, quats, i);
        logit = logits[i];
    }
    // only the candidates' SH rows are staged (the projection backward reads
    // them; the update below reads every row from memory)
    gsd::stage_rows<W, RS>(S, sh + w0 * W, mw, lane, sh_aligned, gsd::ballot(s >= 0));
    gsd::wave_sync();
    float geo[11], Y[16], grm[3];
#pragma unroll
    for (int k = 0; k < 11; ++k) geo[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) Y[k] = 0.0f;
    grm[0] = grm[1] = grm[2] = 0.0f;
    if (s >= 0) {
        const uint32_t fl = __builtin_bit_cast(uint32_t, g2s[s].w);
        proj_bwd_one<DEG>(cam, gi, logit, fl, grad2d + 9 * (int64_t)s, S + lane * RS, geo, Y, grm);
    }
    gsd::wave_sync();   // every lane has read its staged row
    float* Tf = S;
#pragma unroll
    for (int k = 0; k < K; ++k) Tf[lane * RT + k] = Y[k];
#pragma unroll
    for (int c = 0; c < 3; ++c) Tf[lane * RT + K + c] = grm[c];
    gsd::wave_sync();
    if (live) {
        // the 11 geometric values: all loads, then the updates, then the stores
        constexpr int off[11] = {0, 1, 2, 0, 1, 2, 0, 1, 2, 3, 0};
        constexpr int grp[11] = {0, 0, 0, 1, 1, 1, 2, 2, 2, 2, 3};
        constexpr int wid[4] = {3, 3, 4, 1};
        float pp[11], mm[11], vv[11];
#pragma unroll
        for (int k = 0; k < 11; ++k) {
            const int64_t e = wid[grp[k]] * i + off[k];
            pp[k] = pw.p[grp[k]][e];
            mm[k] = pw.m[grp[k]][e];
            vv[k] = pw.v[grp[k]][e];
        }
#pragma unroll
        for (int k = 0; k < 11; ++k) gsd::adam_one(geo[k], pp[k], mm[k], vv[k], a);
#pragma unroll
        for (int k = 0; k < 11; ++k) {
            const int64_t e = wid[grp[k]] * i + off[k];
            pw.p[grp[k]][e] = pp[k];
            pw.m[grp[k]][e] = mm[k];
            pw.v[grp[k]][e] = vv[k];
        }
    }
    // SH values [w0 W, (w0 + mw) W) of the wavefront
    const int nv = mw * W;
    float* P = pw.p[4] + w0 * W;
    float* M = pw.m[4] + w0 * W;
    float* V = pw.v[4] + w0 * W;
    auto shg = [&](int q) {   // partial of value q of the wavefront's rows
        const int gl = q / W, r = q - gl * W;
        const int k = r / 3, c = r - 3 * k;
        return Tf[gl * RT + k] * Tf[gl * RT + K + c];
    };
    if (!pw.vec) {
        for (int q = lane; q < nv; q += 64) {
            float p1 = P[q], m1 = M[q], v1 = V[q];
            gsd::adam_one(shg(q), p1, m1, v1, a);
            P[q] = p1;
            M[q] = m1;
            V[q] = v1;
        }
        return;
    }
    // float4 q4 = lane + 64 r of the rows (16-byte aligned: 64 rows start on a
    // 256-byte boundary), B of them loaded before any is updated
    constexpr int NQ = (16 * W + 63) / 64;
    constexpr int B = 4;
#pragma unroll
    for (int r0 = 0; r0 < NQ; r0 += B) {
        float4 p4[B], m4[B], v4[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int q = 4 * (lane + 64 * (r0 + b));
            if (r0 + b < NQ && q + 3 < nv) {
                p4[b] = *reinterpret_cast<const float4*>(P + q);
                m4[b] = *reinterpret_cast<const float4*>(M + q);
                v4[b] = *reinterpret_cast<const float4*>(V + q);
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int q = 4 * (lane + 64 * (r0 + b));
            if (r0 + b < NQ && q + 3 < nv) {
                gsd::adam_one(shg(q), p4[b].x, m4[b].x, v4[b].x, a);
                gsd::adam_one(shg(q + 1), p4[b].y, m4[b].y, v4[b].y, a);
                gsd::adam_one(shg(q + 2), p4[b].z, m4[b].z, v4[b].z, a);
                gsd::adam_one(shg(q + 3), p4[b].w, m4[b].w, v4[b].w, a);
                *reinterpret_cast<float4*>(P + q) = p4[b];
                *reinterpret_cast<float4*>(M + q) = m4[b];
                *reinterpret_cast<float4*>(V + q) = v4[b];
            }
        }
    }
    // a last partial float4 (rows of a ragged last wavefront)
    const int q0 = nv & ~3;
    if (lane < nv - q0) {
        const int q = q0 + lane;
        float p1 = P[q], m1 = M[q], v1 = V[q];
        gsd::adam_one(shg(q), p1, m1, v1, a);
        P[q] = p1;
        M[q] = m1;
        V[q] = v1;
    }
}

// ---------------------------------------------------------------------------
__global__ void k_export_proj(int64_t n, int field, const uint32_t* __restrict__ ids, const int4* __restrict__ rect,
                              const float4* __restrict__ g0, const float4* __restrict__ g1,
                              const float4* __restrict__ g2, void* __restrict__ dst)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    switch (field) {
    case GS_PROJ_IDS: ((uint32_t*)dst)[j] = ids[j]; break;
    case GS_PROJ_RECT: ((int4*)dst)[j] = rect[j]; break;
    case GS_PROJ_XY: ((float*)dst)[2 * j] = g0[j].x; ((float*)dst)[2 * j + 1] = g0[j].y; break;
    case GS_PROJ_CONIC:   // stored as -A/2, -B, -C/2: exact rescaling
        ((float*)dst)[3 * j] = -2.0f * g0[j].z;
        ((float*)dst)[3 * j + 1] = -g0[j].w;
        ((float*)dst)[3 * j + 2] = -2.0f * g1[j].x;
        break;
    case GS_PROJ_DEPTH: ((float*)dst)[j] = g2[j].y; break;
    case GS_PROJ_RADIUS: ((float*)dst)[j] = g2[j].z; break;
    case GS_PROJ_OPACITY: ((float*)dst)[j] = g1[j].y; break;
    case GS_PROJ_RGB:
        ((float*)dst)[3 * j] = g1[j].z;
        ((float*)dst)[3 * j + 1] = g1[j].w;
        ((float*)dst)[3 * j + 2] = g2[j].x;
        break;
    case GS_PROJ_FLAGS: ((uint32_t*)dst)[j] = __builtin_bit_cast(uint32_t, g2[j].w); break;
    default: break;
    }
}

__global__ void k_copy_i32(int64_t n, const int32_t* __restrict__ src, int32_t* __restrict__ dst)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) dst[j] = src[j];
}

__global__ void k_exp(int64_t n, const float* __restrict__ x, float* __restrict__ y)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) y[j] = gsd::exp_cw(x[j]);
}

__global__ void k_exp_falloff(int64_t n, const float* __restrict__ x, float* __restrict__ y)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) y[j] = gsd::exp_falloff(x[j]);
}

}  // namespace

gs_status launch_project(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, gs_proj* proj,
                         uint32_t* flag, uint32_t* slot, uint32_t* dkey)
{
    const CamDev cd = make_cam(cam);
    const int64_t n = p->n;
    if (n > 0) {
        GsTimerScope ts(ctx, "project_flags");
        hipLaunchKernelGGL(k_project_flags, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, ctx->stream, cd, n,
                           p->means, p->log_scales, p->quats, flag, dkey);
    }
    GS_HIP(ctx, hipGetLastError());
    return launch_scan_u32_to_u32(ctx, flag, slot, n);
}

// second half of the projection (after the host read the candidate count)
gs_status launch_project_write(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, gs_proj* proj,
                               const uint32_t* flag, const uint32_t* slot)
{
    const CamDev cd = make_cam(cam);
    const int64_t n = p->n;
    if (n > 0) {
        GsTimerScope ts(ctx, "project_write");
        const dim3 grid((unsigned)ceil_div(n, 256));
        const bool sh_aligned = ((uintptr_t)p->sh & 15u) == 0;
#define GS_PW(D) hipLaunchKernelGGL(k_project_write<D>, grid, dim3(256), 0, ctx->stream, cd, n, p->means, \
                                    p->log_scales, p->quats, p->opacity_logits, p->sh, sh_aligned, flag, slot, proj->ids, \
                                    proj->rect, proj->g0, proj->g1, proj->g2, proj->slot_of)
        switch (p->sh_degree) {
        case 0: GS_PW(0); break;
        case 1: GS_PW(1); break;
        case 2: GS_PW(2); break;
        default: GS_PW(3); break;
        }
#undef GS_PW
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_bwd_adam(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, const gs_proj* proj,
                          const float* grad2d, const gs_param_ptrs* pr, const gs_param_ptrs* m, const gs_param_ptrs* v,
                          int32_t step, float lr, float b1, float b2, float eps)
{
    const CamDev cd = make_cam(cam);
    const int64_t n = p->n;
    if (n <= 0) return GS_OK;
    AdamPtrs pw;
    const gs_param_ptrs* src[3] = {pr, m, v};
    float** dst[3] = {pw.p, pw.m, pw.v};
    uintptr_t bits = 0;
    for (int t = 0; t < 3; ++t) {
        dst[t][0] = src[t]->means;
        dst[t][1] = src[t]->log_scales;
        dst[t][2] = src[t]->quats;
        dst[t][3] = src[t]->opacity_logits;
        dst[t][4] = src[t]->sh;
        for (int q = 0; q < 5; ++q) bits |= (uintptr_t)dst[t][q];
    }
    pw.vec = (bits & 15u) == 0;
    const gsd::AdamArgs a = gsd::adam_args(step, lr, b1, b2, eps);
    GsTimerScope ts(ctx, "bwd_adam");
    const dim3 grid((unsigned)ceil_div(n, 256));
    const bool sh_aligned = ((uintptr_t)p->sh & 15u) == 0;
#define GS_BA(D) hipLaunchKernelGGL(k_bwd_adam<D>, grid, dim3(256), 0, ctx->stream, cd, n, p->means, p->log_scales, \
                                    p->quats, p->opacity_logits, p->sh, sh_aligned, proj->slot_of, proj->g2, grad2d, \
                                    pw, a)
    switch (p->sh_degree) {
    case 0: GS_BA(0); break;
    case 1: GS_BA(1); break;
    case 2: GS_BA(2); break;
    default: GS_BA(3); break;
    }
#undef GS_BA
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_project_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, const gs_proj* proj,
                             const float* grad2d, int64_t s0, int64_t s1, float* grad3d)
{
    const CamDev cd = make_cam(cam);
    if (s1 > s0) {
        GsTimerScope ts(ctx, "project_bwd");
        const dim3 grid((unsigned)ceil_div(s1 - s0, 256));
#define GS_PB(D) hipLaunchKernelGGL(k_project_bwd<D>, grid, dim3(256), 0, ctx->stream, cd, s0, s1, p->means, \
                                    p->log_scales, p->quats, p->opacity_logits, p->sh, proj->ids, proj->g2, grad2d, \
                                    grad3d)
        switch (p->sh_degree) {
        case 0: GS_PB(0); break;
        case 1: GS_PB(1); break;
        case 2: GS_PB(2); break;
        default: GS_PB(3); break;
        }
#undef GS_PB
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_export_proj(gs_ctx* ctx, const gs_proj* proj, int field, void* dst)
{
    if (field == GS_PROJ_SLOT_OF) {
        if (proj->n > 0)
            hipLaunchKernelGGL(k_copy_i32, dim3((unsigned)ceil_div(proj->n, 256)), dim3(256), 0, ctx->stream,
                               proj->n, proj->slot_of, (int32_t*)dst);
    } else if (proj->n_cand > 0) {
        hipLaunchKernelGGL(k_export_proj, dim3((unsigned)ceil_div(proj->n_cand, 256)), dim3(256), 0, ctx->stream,
                           proj->n_cand, field, proj->ids, proj->rect, proj->g0, proj->g1, proj->g2, dst);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_exp(gs_ctx* ctx, const float* x, float* y, int64_t n, bool falloff)
{
    if (n > 0)
        hipLaunchKernelGGL(falloff ? k_exp_falloff : k_exp, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0,
                           ctx->stream, n, x, y);
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
