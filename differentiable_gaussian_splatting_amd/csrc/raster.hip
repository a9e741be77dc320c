// raster.hip -- per-leaf forward compositing and its reverse-order backward.
//
// Layout (MI355X, wave64): one workgroup of 4 wavefronts per 16x16 tile, each
// wavefront owning an independent 8x8 sub-tile (lane = pixel).  A wavefront
// stages a batch of 64 list entries in its own LDS slice (lane i gathers entry
// i's 9 floats), then every lane walks the batch with wave-uniform LDS reads
// (broadcast, no bank conflicts).  No workgroup barrier is used: wavefronts of
// one tile finish independently, and a wavefront leaves as soon as a ballot
// shows that every one of its pixels has stopped.
//
// Forward (SkipGS notes, "loss function": transmittance accumulation; the
// pages give no formulas, this is the standard compositing rule):
//   power = -0.5 (A dx^2 + C dy^2) - B dx dy, evaluated as
//           fma(fma(-A/2, dx, -B dy), dx, (-C/2 dy) dy)
//   skip if power > 0 (or < -87, where exp gives 0 and alpha < 1/255)
//   alpha = min(0.99, o exp(power)); skip if alpha < 1/255
//   T' = T (1 - alpha); stop before the entry if T' < 1e-4
//   C = fma(rgb, alpha T, C); T = T'
//   out = fma(T, bg, C)
// Backward (BoundedGS Fig. 3 A->B; SkipGS notes: atomic accumulation): per
// pixel the included entries are revisited back to front from the last one,
// with T recovered as T' / (1 - alpha) and the colour behind accumulated as S;
//   dL/dalpha = sum_ch g_ch (rgb_ch T - S_ch / (1 - alpha))
// and the 9 partials of an entry are summed over the wavefront (DPP) before a
// single lane-parallel atomic add of the 9 values.
#include "gs_device.h"
#include "gs_internal.h"

namespace {

struct LeafGeom {
    int W, H;          // image
    int ltx0, lty0;    // leaf origin (tiles)
    int TWL;           // leaf width in tiles
    int px0, py0, WL;  // leaf pixel origin and row length
    int64_t PL;        // leaf pixels
};

LeafGeom make_geom(const gs_camera* cam, const gs_bins* b, const gs_raster* r)
{
    LeafGeom g;
    g.W = cam->width; g.H = cam->height;
    g.ltx0 = b->leaf.tx0; g.lty0 = b->leaf.ty0; g.TWL = b->TWL;
    g.px0 = r->px0; g.py0 = r->py0; g.WL = r->WL;
    g.PL = r->n_pix;
    return g;
}

struct Staged {        // one wavefront's staged batch
    float4 a[64];      // x, y, -A/2, -B
    float4 b[64];      // -C/2, opacity, r, g
    float c[64];       // b
};

__global__ __launch_bounds__(256) void k_raster_fwd(LeafGeom g, const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ target, float inv_norm,
                                                    float* __restrict__ image, float* __restrict__ tfinal,
                                                    uint32_t* __restrict__ last, float* __restrict__ dldc,
                                                    double* __restrict__ l1_part)
{
    __shared__ Staged st[4];
    const int lt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tx = g.ltx0 + lt % g.TWL, ty = g.lty0 + lt / g.TWL;
    const int px = tx * 16 + (wave & 1) * 8 + (lane & 7);
    const int py = ty * 16 + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = px < g.W && py < g.H;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const uint64_t start = offsets[lt], end = offsets[lt + 1];
    Staged& S = st[wave];

    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    uint32_t lastn = 0;
    bool done = !inside;
    for (uint64_t base = start; base < end; base += 64) {
        if (gsd::ballot(!done) == 0) break;
        const uint64_t e = base + lane;
        if (e < end) {
            const uint32_t s = values[e];
            S.a[lane] = g0[s];
            S.b[lane] = g1[s];
            S.c[lane] = g2[s].x;
        }
        gsd::wave_sync();
        const int cnt = (int)min<uint64_t>(64, end - base);
        if (!done) {
            for (int j = 0; j < cnt; ++j) {
                const float4 a = S.a[j];
                const float4 b = S.b[j];
                const float dx = pxc - a.x, dy = pyc - a.y;
                float t = a.w * dy;
                t = __builtin_fmaf(a.z, dx, t);
                float u = b.x * dy;
                u = u * dy;
                const float power = __builtin_fmaf(t, dx, u);
                if (power > 0.0f || power < -87.0f) continue;
                const float G = gsd::exp_cw_core(power);
                const float av = b.y * G;
                const float alpha = av > gsd::kAlphaMax ? gsd::kAlphaMax : av;
                if (alpha < gsd::kAlphaMin) continue;
                const float Tn = T * (1.0f - alpha);
                if (Tn < gsd::kTMin) {
                    done = true;
                    break;
                }
                const float w = alpha * T;
                C0 = __builtin_fmaf(b.z, w, C0);
                C1 = __builtin_fmaf(b.w, w, C1);
                C2 = __builtin_fmaf(S.c[j], w, C2);
                T = Tn;
                lastn = (uint32_t)(base - start) + (uint32_t)j + 1u;
            }
        }
        gsd::wave_sync();
    }

    double l1 = 0.0;
    if (inside) {
        const float o0 = __builtin_fmaf(T, bg0, C0);
        const float o1 = __builtin_fmaf(T, bg1, C1);
        const float o2 = __builtin_fmaf(T, bg2, C2);
        const int64_t P = (int64_t)g.W * g.H;
        const int64_t gi = (int64_t)py * g.W + px;
        if (image) {
            image[gi] = o0;
            image[P + gi] = o1;
            image[2 * P + gi] = o2;
        }
        const int64_t lp = (int64_t)(py - g.py0) * g.WL + (px - g.px0);
        tfinal[lp] = T;
        last[lp] = lastn;
        if (target) {
            const float t0 = target[gi], t1 = target[P + gi], t2 = target[2 * P + gi];
            const float d0 = o0 - t0, d1 = o1 - t1, d2 = o2 - t2;   // sign exact in f32
            dldc[lp] = d0 > 0.0f ? inv_norm : (d0 < 0.0f ? -inv_norm : 0.0f);
            dldc[g.PL + lp] = d1 > 0.0f ? inv_norm : (d1 < 0.0f ? -inv_norm : 0.0f);
            dldc[2 * g.PL + lp] = d2 > 0.0f ? inv_norm : (d2 < 0.0f ? -inv_norm : 0.0f);
            l1 = fabs((double)o0 - (double)t0) + fabs((double)o1 - (double)t1) + fabs((double)o2 - (double)t2);
        }
    }
    if (target) {
        l1 = gsd::wave_sum_d(l1);
        if (lane == 0) l1_part[(int64_t)lt * 4 + wave] = l1;
    }
}

__global__ __launch_bounds__(256) void k_raster_bwd(LeafGeom g, const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ tfinal,
                                                    const uint32_t* __restrict__ last,
                                                    const float* __restrict__ dldc,
                                                    const float* __restrict__ dl_dimage,
                                                    float* __restrict__ grad2d)
{
    __shared__ Staged st[4];
    __shared__ uint32_t slot_s[4][64];
    const int lt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tx = g.ltx0 + lt % g.TWL, ty = g.lty0 + lt / g.TWL;
    const int px = tx * 16 + (wave & 1) * 8 + (lane & 7);
    const int py = ty * 16 + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = px < g.W && py < g.H;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const uint64_t start = offsets[lt];
    Staged& S = st[wave];

    float T = 1.0f, gr0 = 0.0f, gr1 = 0.0f, gr2 = 0.0f;
    uint32_t lst = 0;
    if (inside) {
        const int64_t lp = (int64_t)(py - g.py0) * g.WL + (px - g.px0);
        T = tfinal[lp];
        lst = last[lp];
        if (dl_dimage) {
            const int64_t P = (int64_t)g.W * g.H;
            const int64_t gi = (int64_t)py * g.W + px;
            gr0 = dl_dimage[gi];
            gr1 = dl_dimage[P + gi];
            gr2 = dl_dimage[2 * P + gi];
        } else {
            gr0 = dldc[lp];
            gr1 = dldc[g.PL + lp];
            gr2 = dldc[2 * g.PL + lp];
        }
    }
    float S0 = T * bg0, S1 = T * bg1, S2 = T * bg2;
    const uint32_t maxl = gsd::wave_max_u32(lst);

    for (int64_t hi = maxl; hi > 0; hi -= 64) {
        const int64_t lo = hi > 64 ? hi - 64 : 0;
        const int cnt = (int)(hi - lo);
        if (lane < cnt) {
            const uint32_t s = values[start + lo + lane];
            slot_s[wave][lane] = s;
            S.a[lane] = g0[s];
            S.b[lane] = g1[s];
            S.c[lane] = g2[s].x;
        }
        gsd::wave_sync();
        for (int j = cnt - 1; j >= 0; --j) {
            const uint32_t n = (uint32_t)(lo + j);
            float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f, p4 = 0.0f, p5 = 0.0f, p6 = 0.0f, p7 = 0.0f,
                  p8 = 0.0f;
            bool contrib = false;
            if (n < lst) {
                const float4 a = S.a[j];
                const float4 b = S.b[j];
                const float cb = S.c[j];
                const float dx = pxc - a.x, dy = pyc - a.y;
                float t = a.w * dy;
                t = __builtin_fmaf(a.z, dx, t);
                float u = b.x * dy;
                u = u * dy;
                const float power = __builtin_fmaf(t, dx, u);
                if (!(power > 0.0f || power < -87.0f)) {
                    const float G = gsd::exp_cw_core(power);
                    const float av = b.y * G;
                    const bool clamped = av > gsd::kAlphaMax;
                    const float alpha = clamped ? gsd::kAlphaMax : av;
                    if (!(alpha < gsd::kAlphaMin)) {
                        contrib = true;
                        const float om = 1.0f - alpha;
                        const float rom = __builtin_amdgcn_rcpf(om);
                        T = T * rom;                      // T before this entry
                        const float w = alpha * T;
                        p6 = gr0 * w;
                        p7 = gr1 * w;
                        p8 = gr2 * w;
                        const float dal = gr0 * (b.z * T - S0 * rom) + gr1 * (b.w * T - S1 * rom) +
                                          gr2 * (cb * T - S2 * rom);
                        S0 = __builtin_fmaf(b.z, w, S0);
                        S1 = __builtin_fmaf(b.w, w, S1);
                        S2 = __builtin_fmaf(cb, w, S2);
                        if (!clamped) {
                            const float dpw = dal * av;   // d alpha / d power = o G
                            p5 = dal * G;
                            // A = -2 a.z, B = -a.w, C = -2 b.x
                            p2 = -0.5f * dx * dx * dpw;
                            p3 = -dx * dy * dpw;
                            p4 = -0.5f * dy * dy * dpw;
                            p0 = (-2.0f * a.z * dx - a.w * dy) * dpw;
                            p1 = (-2.0f * b.x * dy - a.w * dx) * dpw;
                        }
                    }
                }
            }
            if (gsd::ballot(contrib) == 0) continue;
            const float r0 = gsd::wave_sum(p0), r1 = gsd::wave_sum(p1), r2 = gsd::wave_sum(p2);
            const float r3 = gsd::wave_sum(p3), r4 = gsd::wave_sum(p4), r5 = gsd::wave_sum(p5);
            const float r6 = gsd::wave_sum(p6), r7 = gsd::wave_sum(p7), r8 = gsd::wave_sum(p8);
            float mine = r0;
            mine = lane == 1 ? r1 : mine;
            mine = lane == 2 ? r2 : mine;
            mine = lane == 3 ? r3 : mine;
            mine = lane == 4 ? r4 : mine;
            mine = lane == 5 ? r5 : mine;
            mine = lane == 6 ? r6 : mine;
            mine = lane == 7 ? r7 : mine;
            mine = lane == 8 ? r8 : mine;
            if (lane < 9) unsafeAtomicAdd(&grad2d[(int64_t)slot_s[wave][j] * 9 + lane], mine);
        }
        gsd::wave_sync();
    }
}

}  // namespace

gs_status launch_raster_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            gs_raster* r, const float* target, float* image_out, double* loss_accum)
{
    const LeafGeom g = make_geom(cam, bins, r);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_fwd");
        hipLaunchKernelGGL(k_raster_fwd, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g, bins->offsets,
                           bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1], cam->bg[2], target,
                           inv_norm, image_out, r->tfinal, r->last, r->dldc, r->l1_part);
    }
    GS_HIP(ctx, hipGetLastError());
    if (target && loss_accum) return launch_sum_f64(ctx, r->l1_part, bins->n_tiles * 4, 1, loss_accum, 1);
    return GS_OK;
}

gs_status launch_raster_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            const gs_raster* r, const float* dl_dimage, float* grad2d)
{
    const LeafGeom g = make_geom(cam, bins, r);
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_bwd");
        hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g, bins->offsets,
                           bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1], cam->bg[2],
                           r->tfinal, r->last, r->dldc, dl_dimage, grad2d);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
