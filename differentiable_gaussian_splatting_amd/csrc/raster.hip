// raster.hip -- per-leaf forward compositing and its reverse-order backward.
//
// Layout (MI355X, wave64): one workgroup of 4 wavefronts per 16x16 tile, each
// wavefront owning an independent 8x8 sub-tile (lane = pixel).  A wavefront
// stages a batch of 64 list entries in its own LDS slice (lane i gathers entry
// i), then every lane walks the batch with wave-uniform LDS reads (broadcast,
// free of bank conflicts).  No workgroup barrier is used: the wavefronts of a
// tile finish independently, and one leaves as soon as a ballot shows that all
// of its pixels have stopped.
//
// Sub-tile culling: while staging, lane i also decides whether entry i can
// reach alpha >= 1/255 anywhere in the wavefront's 8x8 box of pixel centres:
// the minimum of the quadratic form q = A dx^2 + 2B dx dy + C dy^2 over the
// box (0 if the centre is inside, else the least of four clamped edge minima)
// is compared with 2 ln(255 o), with a margin that covers the f32 rounding of
// both q and the per-pixel exponent.  An entry is dropped only when every
// pixel of the box would skip it, so the per-pixel decisions are unchanged.
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
//   dL/dalpha = sum_ch g_ch (rgb_ch T - S_ch / (1 - alpha)).
// The 9 partials of an entry are summed over the wavefront by a transposed
// reduction (each step halves the lanes per value while pairing values, with
// the gfx950 lane-swap instructions and DPP) and written by one 9-lane atomic.
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

struct Staged {        // one wavefront's staged batch (entry j at byte 16 j of each array,
    float4 a[64];      // so one address register serves all three reads)
    float4 b[64];      // x, y, -A/2, -B | -C/2, opacity, r, g
    float4 c[64];      // b, slot (bits), -, -
};

// true when no pixel centre of the box [bx0, bx0+7] x [by0, by0+7] can
// include the entry (alpha < 1/255 everywhere)
__device__ __forceinline__ bool cull_box(float4 a, float4 b, float bx0, float by0)
{
    const float o = b.y;
    if (!(o * 255.0f >= 1.0f)) return true;     // alpha <= o < 1/255
    const float A = -2.0f * a.z, B = -a.w, C = -2.0f * b.x;
    const float dx0 = bx0 - a.x, dx1 = dx0 + 7.0f;
    const float dy0 = by0 - a.y, dy1 = dy0 + 7.0f;
    if (dx0 <= 0.0f && dx1 >= 0.0f && dy0 <= 0.0f && dy1 >= 0.0f) return false;
    float qmin = __builtin_inff();
    {
        const float iC = 1.0f / C, iA = 1.0f / A;
        float X = dx0, t = fminf(fmaxf(-B * X * iC, dy0), dy1);
        qmin = fminf(qmin, A * X * X + 2.0f * B * X * t + C * t * t);
        X = dx1; t = fminf(fmaxf(-B * X * iC, dy0), dy1);
        qmin = fminf(qmin, A * X * X + 2.0f * B * X * t + C * t * t);
        float Y = dy0, s = fminf(fmaxf(-B * Y * iA, dx0), dx1);
        qmin = fminf(qmin, C * Y * Y + 2.0f * B * Y * s + A * s * s);
        Y = dy1; s = fminf(fmaxf(-B * Y * iA, dx0), dx1);
        qmin = fminf(qmin, C * Y * Y + 2.0f * B * Y * s + A * s * s);
    }
    const float Xm = fmaxf(fabsf(dx0), fabsf(dx1)), Ym = fmaxf(fabsf(dy0), fabsf(dy1));
    const float S = fabsf(A) * Xm * Xm + 2.0f * fabsf(B) * Xm * Ym + fabsf(C) * Ym * Ym;
    const float thr = 2.0f * __logf(255.0f * o);
    return qmin - (0.02f + 1e-3f * qmin + 1e-5f * S) > thr;
}

template <bool STATS>
__global__ __launch_bounds__(256) void k_raster_fwd(LeafGeom g, const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ target, float inv_norm,
                                                    float* __restrict__ image, float* __restrict__ tfinal,
                                                    uint32_t* __restrict__ last, uint8_t* __restrict__ sgn,
                                                    double* __restrict__ l1_part,
                                                    unsigned long long* __restrict__ stats)
{
    __shared__ Staged st[4];
    const int lt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tx = g.ltx0 + lt % g.TWL, ty = g.lty0 + lt / g.TWL;
    const int sx0 = tx * 16 + (wave & 1) * 8, sy0 = ty * 16 + (wave >> 1) * 8;
    const int px = sx0 + (lane & 7), py = sy0 + (lane >> 3);
    const bool inside = px < g.W && py < g.H;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const float bx0 = (float)sx0 + 0.5f, by0 = (float)sy0 + 0.5f;
    const uint64_t start = offsets[lt], end = offsets[lt + 1];
    Staged& S = st[wave];

    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    uint32_t lastn = 0, n_eval = 0, n_inc = 0, ev_at_last = 0;
    bool active = inside;
    for (uint64_t base = start; base < end; base += 64) {
        if (gsd::ballot(active) == 0) break;
        const uint64_t e = base + lane;
        bool keep = false;
        if (e < end) {
            const uint32_t s = values[e];
            const float4 a = g0[s], b = g1[s];
            S.a[lane] = a;
            S.b[lane] = b;
            S.c[lane] = make_float4(g2[s].x, __builtin_bit_cast(float, s), 0.0f, 0.0f);
            keep = !cull_box(a, b, bx0, by0);
        }
        uint64_t mask = gsd::ballot(keep);
        gsd::wave_sync();
        const uint32_t n0 = (uint32_t)(base - start) + 1u;
        // Branch-free over the lanes: every lane evaluates the entry and the
        // per-lane decisions become selects, so the wavefront issues one
        // straight run of instructions per entry.  A lane's values for an
        // entry it includes are computed in exactly the order given above.
        while (mask) {
            const int j = __builtin_ctzll(mask);
            mask &= mask - 1;
            const float4 a = S.a[j];
            const float4 b = S.b[j];
            const float dx = pxc - a.x, dy = pyc - a.y;
            float t = a.w * dy;
            t = __builtin_fmaf(a.z, dx, t);
            float u = b.x * dy;
            u = u * dy;
            const float power = __builtin_fmaf(t, dx, u);
            // exp of the exponent clamped into [-87, 0]: exp(power) on every
            // lane that can include the entry (below -87 the exp is 0 and
            // alpha < 1/255; at -87 o exp(-87) < 1/255 too), finite on the others
            const bool pok = !(power > 0.0f);
            const float G = gsd::exp_cw_core(__builtin_amdgcn_fmed3f(power, -87.0f, 0.0f));
            const float av = b.y * G;
            const float alpha = av > gsd::kAlphaMax ? gsd::kAlphaMax : av;
            const bool inc = active && pok && !(alpha < gsd::kAlphaMin);
            const float ae = inc ? alpha : 0.0f;
            const float Tn = T * (1.0f - ae);
            const bool stop = inc && Tn < gsd::kTMin;
            const bool contrib = inc && !stop;
            if (STATS) {
                n_eval += active ? 1u : 0u;
                n_inc += contrib ? 1u : 0u;
                ev_at_last = contrib ? n_eval : ev_at_last;
            }
            active = active && !stop;
            const float w = contrib ? ae * T : 0.0f;   // fma(x, 0, C) = C exactly
            C0 = __builtin_fmaf(b.z, w, C0);
            C1 = __builtin_fmaf(b.w, w, C1);
            C2 = __builtin_fmaf(S.c[j].x, w, C2);
            T = contrib ? Tn : T;
            lastn = contrib ? n0 + (uint32_t)j : lastn;
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
            // dL/dout = sgn(out - target) / (3WH): 2 bits per channel, 1 = +, 2 = -
            const uint32_t c0 = d0 > 0.0f ? 1u : (d0 < 0.0f ? 2u : 0u);
            const uint32_t c1 = d1 > 0.0f ? 1u : (d1 < 0.0f ? 2u : 0u);
            const uint32_t c2 = d2 > 0.0f ? 1u : (d2 < 0.0f ? 2u : 0u);
            sgn[lp] = (uint8_t)(c0 | (c1 << 2) | (c2 << 4));
            l1 = fabs((double)o0 - (double)t0) + fabs((double)o1 - (double)t1) + fabs((double)o2 - (double)t2);
        }
    }
    if (target) {
        l1 = gsd::wave_sum_d(l1);
        if (lane == 0) l1_part[(int64_t)lt * 4 + wave] = l1;
    }
    if (STATS) {
        // [0] pairs examined, [1] pairs included, [2] sum of last, [3] pairs
        // the backward revisits (examined up to the last included entry)
        const double a0 = gsd::wave_sum_d((double)n_eval), a1 = gsd::wave_sum_d((double)n_inc);
        const double a2 = gsd::wave_sum_d((double)(inside ? lastn : 0u));
        const double a3 = gsd::wave_sum_d((double)ev_at_last);
        if (lane == 0) {
            atomicAdd(&stats[0], (unsigned long long)a0);
            atomicAdd(&stats[1], (unsigned long long)a1);
            atomicAdd(&stats[2], (unsigned long long)a2);
            atomicAdd(&stats[3], (unsigned long long)a3);
        }
    }
}

// ---- transposed wave reduction of 9 values --------------------------------
__device__ __forceinline__ uint32_t fb(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bf(uint32_t v) { return __builtin_bit_cast(float, v); }

// x, y -> x + y where the first 32 lanes hold the value of x and the last 32
// that of y (each summed over lanes l and l +- 32)
__device__ __forceinline__ float pair32(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(fb(x), fb(y), false, false);
    return bf(r[0]) + bf(r[1]);
}

// per 32-lane half: rows 0/2 of the result carry x, rows 1/3 carry y (each
// summed over the two rows of the half)
__device__ __forceinline__ float pair16(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(fb(x), fb(y), false, false);
    return bf(r[0]) + bf(r[1]);
}

// within each 16-lane row: lanes 0-7 carry x, lanes 8-15 carry y
__device__ __forceinline__ float pair8(float x, float y, int lane)
{
    const bool hi = (lane & 8) != 0;
    const float send = hi ? x : y, keep = hi ? y : x;
    return keep + gsd::dpp_f<0x140>(send);   // row_mirror
}

// within each 8-lane group: lanes 0-3 carry x, lanes 4-7 carry y
__device__ __forceinline__ float pair4(float x, float y, int lane)
{
    const bool hi = (lane & 4) != 0;
    const float send = hi ? x : y, keep = hi ? y : x;
    return keep + gsd::dpp_f<0x141>(send);   // row_half_mirror
}

// Sums p[0..8] over the wavefront.  On return the full sum of value v is in
// the first lane of quad q (lane 4q) with v = bitreverse3(q / 2) for even q
// and v = 8 for q = 1; *vidx gets that v, or -1 for lanes that hold none.
__device__ __forceinline__ float wave_reduce9(const float* p, int lane, int* vidx)
{
    const float a0 = pair32(p[0], p[1]), a1 = pair32(p[2], p[3]), a2 = pair32(p[4], p[5]);
    const float a3 = pair32(p[6], p[7]), a4 = pair32(p[8], 0.0f);
    const float b0 = pair16(a0, a1), b1 = pair16(a2, a3), b2 = pair16(a4, 0.0f);
    const float c0 = pair8(b0, b1, lane), c1 = pair8(b2, 0.0f, lane);
    float d = pair4(c0, c1, lane);
    d += gsd::dpp_f<0x4E>(d);   // quad_perm [2,3,0,1]
    d += gsd::dpp_f<0xB1>(d);   // quad_perm [1,0,3,2]
    const int q = lane >> 2;
    int v = -1;
    if ((lane & 3) == 0) {
        if ((q & 1) == 0) {
            const int k = q >> 1;
            v = ((k & 1) << 2) | (k & 2) | ((k >> 2) & 1);
        } else if (q == 1) {
            v = 8;
        }
    }
    *vidx = v;
    return d;
}

// Backward, one workgroup per tile.  The four wavefronts walk the tile's
// list together, 64 entries per batch from the last entry any pixel of the
// tile included: the batch is staged once in LDS (16 entries per wavefront),
// each wavefront culls it against its own 8 x 8 box and reduces the 9
// partials of each entry over its lanes into an LDS row, and after a barrier
// the 256 threads add the four rows of each (entry, value) and issue one
// atomic add per nonzero sum -- a quarter of the atomics of per-wavefront
// adds.  Staging and partial rows are double-buffered, so a batch costs two
// workgroup barriers: one after staging, one before the sums.
struct BwdShared {
    Staged st[2];
    float4 red[2][64 * 9];               // [entry * 9 + value] -> the 4 wavefronts' sums
    unsigned long long wmask[2][4];      // entries each wavefront wrote in the batch
    uint32_t maxl[4];
};

__global__ __launch_bounds__(256) void k_raster_bwd(LeafGeom g, const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ tfinal,
                                                    const uint32_t* __restrict__ last,
                                                    const uint8_t* __restrict__ sgn, float inv_norm,
                                                    const float* __restrict__ dl_dimage,
                                                    float* __restrict__ grad2d)
{
    __shared__ BwdShared sh;
    const int lt = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tx = g.ltx0 + lt % g.TWL, ty = g.lty0 + lt / g.TWL;
    const int sx0 = tx * 16 + (wave & 1) * 8, sy0 = ty * 16 + (wave >> 1) * 8;
    const int px = sx0 + (lane & 7), py = sy0 + (lane >> 3);
    const bool inside = px < g.W && py < g.H;
    const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
    const float bx0 = (float)sx0 + 0.5f, by0 = (float)sy0 + 0.5f;
    const uint64_t start = offsets[lt];

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
            const uint32_t c = sgn[lp];
            auto dec = [&](uint32_t code) { return code == 1u ? inv_norm : (code == 2u ? -inv_norm : 0.0f); };
            gr0 = dec(c & 3u);
            gr1 = dec((c >> 2) & 3u);
            gr2 = dec((c >> 4) & 3u);
        }
    }
    // GS = sum_ch dL/dout_ch * (colour behind the current entry, ch); it
    // starts as the background seen through T_final
    float GS = T * (gr0 * bg0 + gr1 * bg1 + gr2 * bg2);
    {
        const uint32_t m = gsd::wave_max_u32(lst);
        if (lane == 0) sh.maxl[wave] = m;
    }
    __syncthreads();
    const int64_t maxl = (int64_t)max(max(sh.maxl[0], sh.maxl[1]), max(sh.maxl[2], sh.maxl[3]));

    // stage entries [lo, hi) of the tile's list into buffer b (16 per wavefront)
    auto stage = [&](int b, int64_t hi) {
        const int64_t lo = hi > 64 ? hi - 64 : 0;
        const int e = wave * 16 + lane;
        if (lane < 16 && lo + e < hi) {
            const uint32_t s = values[start + lo + e];
            sh.st[b].a[e] = g0[s];
            sh.st[b].b[e] = g1[s];
            sh.st[b].c[e] = make_float4(g2[s].x, __builtin_bit_cast(float, s), 0.0f, 0.0f);
        }
    };
    if (maxl > 0) stage(0, maxl);
    int b = 0;
    for (int64_t hi = maxl; hi > 0; hi -= 64, b ^= 1) {
        const int64_t lo = hi > 64 ? hi - 64 : 0;
        const int cnt = (int)(hi - lo);
        __syncthreads();                       // batch staged; previous sums done
        Staged& S = sh.st[b];
        bool keep = false;
        if (lane < cnt) keep = !cull_box(S.a[lane], S.b[lane], bx0, by0);
        uint64_t mask = gsd::ballot(keep);
        uint64_t wrote = 0;
        // Branch-free over the lanes, as in the forward: the inclusion of an
        // entry is re-derived with the forward's exact f32 operations, and the
        // partials of lanes that do not include it are zero.
        while (mask) {
            const int j = 63 - __builtin_clzll(mask);
            mask &= ~(1ull << j);
            const uint32_t n = (uint32_t)(lo + j);
            const float4 a = S.a[j];
            const float4 bb = S.b[j];
            const float cb = S.c[j].x;
            const float dx = pxc - a.x, dy = pyc - a.y;
            float t = a.w * dy;
            t = __builtin_fmaf(a.z, dx, t);
            const float u1 = bb.x * dy;
            const float u = u1 * dy;
            const float power = __builtin_fmaf(t, dx, u);
            const bool pok = !(power > 0.0f);   // power < -87: alpha < 1/255 (as in the forward)
            const float G = gsd::exp_cw_core(__builtin_amdgcn_fmed3f(power, -87.0f, 0.0f));
            const float av = bb.y * G;
            const bool clamped = av > gsd::kAlphaMax;
            const float alpha = clamped ? gsd::kAlphaMax : av;
            const bool contrib = n < lst && pok && !(alpha < gsd::kAlphaMin);
            if (gsd::ballot(contrib) == 0) continue;
            // alpha of the lanes that include the entry, 0 on the others: then
            // T / (1 - 0) = T and w = 0 leave those lanes' state unchanged
            const float ae = contrib ? alpha : 0.0f;
            // T before this entry = T after it / (1 - alpha)
            const float rom = __builtin_amdgcn_rcpf(1.0f - ae);
            T = T * rom;
            const float w = ae * T;
            // dL/dalpha = sum_ch g_ch (rgb_ch T - S_ch / (1 - alpha))
            const float grgb = __builtin_fmaf(gr2, cb, __builtin_fmaf(gr1, bb.w, gr0 * bb.z));
            const float dal0 = __builtin_fmaf(T, grgb, -(rom * GS));
            GS = __builtin_fmaf(grgb, w, GS);
            float p[9];
            p[6] = gr0 * w;
            p[7] = gr1 * w;
            p[8] = gr2 * w;
            // through alpha = o G, zero where alpha is clamped or not included
            const float dal = (contrib && !clamped) ? dal0 : 0.0f;
            p[5] = dal * G;
            const float ndpw = -(dal * av);   // -dL/dpower
            // power = -(A dx^2 + C dy^2)/2 - B dx dy with A = -2 a.z, B = -a.w,
            // C = -2 b.x, dx = px - x, dy = py - y, so with q = -dL/dpower
            //   dL/dx = (A dx + B dy) dL/dpower = 2 a.z (q dx) + a.w (q dy)
            //   dL/dy = (C dy + B dx) dL/dpower = 2 b.x (q dy) + a.w (q dx)
            //   dL/dA = (q dx dx)/2, dL/dB = q dx dy, dL/dC = (q dy dy)/2.
            // The five moments q dx, q dy, q dx dx, q dx dy, q dy dy are summed
            // over the pixels and turned into the five partials once per entry.
            p[0] = ndpw * dx;
            p[1] = ndpw * dy;
            p[2] = p[0] * dx;
            p[3] = p[0] * dy;
            p[4] = p[1] * dy;
            int v;
            const float r = wave_reduce9(p, lane, &v);
            if (v >= 0) {
                float* row = reinterpret_cast<float*>(&sh.red[b][j * 9 + v]);
                row[wave] = r;
            }
            wrote |= 1ull << j;
        }
        if (lane == 0) sh.wmask[b][wave] = wrote;
        __syncthreads();                       // rows of the batch written
        // sums of the four rows, one atomic per nonzero (entry, value)
        const unsigned long long m0 = sh.wmask[b][0], m1 = sh.wmask[b][1];
        const unsigned long long m2 = sh.wmask[b][2], m3 = sh.wmask[b][3];
        auto row_sum = [&](int o, int j) {
            const float4 q = sh.red[b][o];
            float sum = 0.0f;
            sum += ((m0 >> j) & 1ull) ? q.x : 0.0f;
            sum += ((m1 >> j) & 1ull) ? q.y : 0.0f;
            sum += ((m2 >> j) & 1ull) ? q.z : 0.0f;
            sum += ((m3 >> j) & 1ull) ? q.w : 0.0f;
            return sum;
        };
        for (int o = tid; o < cnt * 9; o += 256) {
            const int j = o / 9, v = o - j * 9;
            float sum = row_sum(o, j);
            if (v < 5) {
                // moments -> partials of the mean and the conic
                const float4 a = S.a[j];
                if (v == 0) sum = 2.0f * a.z * sum + a.w * row_sum(o + 1, j);
                else if (v == 1) sum = 2.0f * S.b[j].x * sum + a.w * row_sum(o - 1, j);
                else if (v != 3) sum = 0.5f * sum;
            }
            if (sum != 0.0f) {
                const uint32_t slot = __builtin_bit_cast(uint32_t, S.c[j].y);
                unsafeAtomicAdd(&grad2d[(int64_t)slot * 9 + v], sum);
            }
        }
        if (hi - 64 > 0) stage(b ^ 1, hi - 64);
    }
}

}  // namespace

gs_status launch_raster_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            gs_raster* r, const float* target, float* image_out, double* loss_accum,
                            uint64_t* stats)
{
    const LeafGeom g = make_geom(cam, bins, r);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_fwd");
        if (stats)
            hipLaunchKernelGGL(k_raster_fwd<true>, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g,
                               bins->offsets, bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1],
                               cam->bg[2], target, inv_norm, image_out, r->tfinal, r->last, r->sgn, r->l1_part,
                               (unsigned long long*)stats);
        else
            hipLaunchKernelGGL(k_raster_fwd<false>, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g,
                               bins->offsets, bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1],
                               cam->bg[2], target, inv_norm, image_out, r->tfinal, r->last, r->sgn, r->l1_part,
                               nullptr);
    }
    GS_HIP(ctx, hipGetLastError());
    if (target && loss_accum) return launch_sum_f64(ctx, r->l1_part, bins->n_tiles * 4, 1, loss_accum, 1);
    return GS_OK;
}

gs_status launch_raster_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            const gs_raster* r, const float* dl_dimage, float* grad2d)
{
    const LeafGeom g = make_geom(cam, bins, r);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_bwd");
        hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g, bins->offsets,
                           bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1], cam->bg[2],
                           r->tfinal, r->last, r->sgn, inv_norm, dl_dimage, grad2d);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}
