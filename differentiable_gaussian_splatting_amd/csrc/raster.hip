// raster.hip -- per-leaf forward compositing and its reverse-order backward.
//
// Layout (MI355X, wave64).  Forward: one workgroup of 4 wavefronts per 16x16
// tile, each wavefront owning an independent 8x8 sub-tile (lane = pixel).
// Backward: one wavefront per 16x16 tile (lane = one pixel in each of the four
// 8x8 quadrants), four tiles per workgroup.  A wavefront stages a batch of 64
// list entries in its own LDS slice (lane i gathers entry i), then every lane
// walks the batch with wave-uniform LDS reads (broadcast, free of bank
// conflicts).  No workgroup barrier is used: wavefronts finish independently,
// and a forward wavefront leaves as soon as a ballot shows that all of its
// pixels have stopped.
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
//   skip if power > 0
//   alpha = min(0.99, o E(power)); skip if alpha < 1/255, where E is exp on
//           [-6, 0] and E(-6) below it (alpha < 1/255 there either way)
//   T' = T (1 - alpha); stop before the entry if T' < 1e-4
//   C = fma(rgb, alpha T, C); T = T'
//   out = fma(T, bg, C)
// Backward (BoundedGS Fig. 3 A->B; SkipGS notes: atomic accumulation): per
// pixel the included entries are revisited back to front, starting at the end
// of the pixel's forward walk (the position of the entry before which it
// stopped, else the list length: no entry from there on is included), with T
// recovered as T' / (1 - alpha) and the colour behind accumulated as S;
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

// list positions whose forward quadrant masks the fused kernel keeps in LDS
// for its backward (one byte each); entries further down the list are culled
// again by the backward
constexpr uint32_t kQCache = 2048;

struct Staged {        // one wavefront's staged batch (entry j at byte 16 j of each array,
    float4 a[64];      // so one address register serves all three reads)
    float4 b[64];      // x, y, -A/2, -B | -C/2, opacity, r, g
    float4 c[64];      // b, slot (bits), list position (bits, backward), -
    uint32_t idx[64];  // group walk: list positions of the batch's covering entries
};


// Per-entry part of the sub-tile cull: the conic, the reciprocals of its
// diagonal and the threshold 2 ln(255 o), shared by every box the entry is
// tested against.
struct CullPrep {
    float x, y, A, B, C, iA, iC, thr;
    bool faint;   // o < 1/255: alpha <= o stays below 1/255 everywhere
};

__device__ __forceinline__ CullPrep cull_prep(float4 a, float4 b)
{
    CullPrep p;
    const float o = b.y;
    p.faint = !(o * 255.0f >= 1.0f);
    p.x = a.x;
    p.y = a.y;
    p.A = -2.0f * a.z;
    p.B = -a.w;
    p.C = -2.0f * b.x;
    p.iC = 1.0f / p.C;
    p.iA = 1.0f / p.A;
    p.thr = 2.0f * __logf(255.0f * o);
    return p;
}

// true when no pixel centre of the box [bx0, bx0+7] x [by0, by0+7] can
// include the entry (alpha < 1/255 everywhere)
__device__ __forceinline__ bool cull_test(const CullPrep& p, float bx0, float by0)
{
    if (p.faint) return true;
    const float A = p.A, B = p.B, C = p.C;
    const float dx0 = bx0 - p.x, dx1 = dx0 + 7.0f;
    const float dy0 = by0 - p.y, dy1 = dy0 + 7.0f;
    if (dx0 <= 0.0f && dx1 >= 0.0f && dy0 <= 0.0f && dy1 >= 0.0f) return false;
    float qmin = __builtin_inff();
    {
        float X = dx0, t = fminf(fmaxf(-B * X * p.iC, dy0), dy1);
        qmin = fminf(qmin, A * X * X + 2.0f * B * X * t + C * t * t);
        X = dx1; t = fminf(fmaxf(-B * X * p.iC, dy0), dy1);
        qmin = fminf(qmin, A * X * X + 2.0f * B * X * t + C * t * t);
        float Y = dy0, s = fminf(fmaxf(-B * Y * p.iA, dx0), dx1);
        qmin = fminf(qmin, C * Y * Y + 2.0f * B * Y * s + A * s * s);
        Y = dy1; s = fminf(fmaxf(-B * Y * p.iA, dx0), dx1);
        qmin = fminf(qmin, C * Y * Y + 2.0f * B * Y * s + A * s * s);
    }
    const float Xm = fmaxf(fabsf(dx0), fabsf(dx1)), Ym = fmaxf(fabsf(dy0), fabsf(dy1));
    const float S = fabsf(A) * Xm * Xm + 2.0f * fabsf(B) * Xm * Ym + fabsf(C) * Ym * Ym;
    return qmin - (0.02f + 1e-3f * qmin + 1e-5f * S) > p.thr;
}

__device__ __forceinline__ bool cull_box(float4 a, float4 b, float bx0, float by0)
{
    return cull_test(cull_prep(a, b), bx0, by0);
}

// Whether a super-tile group entry (coarse key: its rectangle inside the
// super-tile above bit kCellBits) covers the tile at local position cr =
// column | row << 3 of the super-tile.  A tile's list is the subsequence of
// its super-tile's group that covers it, in group order.
__device__ __forceinline__ bool covers(uint32_t key, uint32_t cr)
{
    const uint32_t lr = key >> kCellBits, c = cr & 7u, r = cr >> 3;
    return (lr & 7u) <= c && c <= ((lr >> 3) & 7u) && ((lr >> 6) & 7u) <= r && r <= ((lr >> 9) & 7u);
}

// The next batch of a tile's group walk: up to 64 entries of the group that
// cover the tile, in group order (FWD: ascending from *scan, into idx[0..n);
// else descending from *scan - 1, into idx[64 - n..64)), examining 64 group
// positions per step; *scan moves past what was examined, stopping at the
// first covering entry that did not fit.  Returns n; the caller waits
// (wave_sync) before reading idx.
template <bool FWD>
__device__ __forceinline__ int collect_covering(Staged& S, int lane, const uint32_t* __restrict__ keys,
                                                uint64_t start, uint64_t end_pos, uint32_t cr, uint64_t* scan,
                                                uint8_t* qmark = nullptr)
{
    int n = 0;
    uint64_t sc = *scan;
    while (n < 64 && (FWD ? sc < end_pos : sc > 0)) {
        const int64_t p = FWD ? (int64_t)(sc + (uint64_t)lane) : (int64_t)sc - 1 - lane;
        const bool in = FWD ? p < (int64_t)end_pos : p >= 0;
        const bool cov = in && covers(keys[start + (uint64_t)p], cr);
        // qmark: positions that do not cover the tile get an empty quadrant mask
        if (qmark && in && !cov && (uint64_t)p < kQCache) qmark[p] = 0;
        const uint64_t m = gsd::ballot(cov);
        const int cnt = __builtin_popcountll(m);
        const int take = min(cnt, 64 - n);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (cov && rank < take) S.idx[FWD ? n + rank : 63 - n - rank] = (uint32_t)p;
        if (take < cnt) {
            // the first covering lane left over starts the next batch
            uint64_t mm = m;
            for (int t = 0; t < take; ++t) mm &= mm - 1ull;
            const uint64_t L = (uint64_t)__builtin_ctzll(mm);
            sc = FWD ? sc + L : sc - L;
        } else {
            sc = FWD ? sc + 64 : (sc > 64 ? sc - 64 : 0);
        }
        n += take;
    }
    *scan = sc;
    return n;
}

// The next backward batch of a fused tile: up to 64 list positions below
// *scan (descending, into idx[64 - n..64)) whose entry the backward must
// evaluate: below kQCache, those whose forward quadrant mask has a quadrant
// whose walks reach the position (entries culled there, or not covering the
// tile, are skipped); further down, every entry of a list, or every group
// entry that covers the tile.
template <bool GROUPS>
__device__ __forceinline__ int collect_live(Staged& S, int lane, const uint32_t* __restrict__ keys, uint64_t start,
                                            uint32_t cr, const uint8_t* qc, const uint32_t (&mq)[4],
                                            uint64_t* scan)
{
    int n = 0;
    uint64_t sc = *scan;
    while (n < 64 && sc > 0) {
        const int64_t p = (int64_t)sc - 1 - lane;
        bool keep = false;
        if (p >= 0) {
            const uint32_t up = (uint32_t)p;
            if (up < kQCache) {
                const uint32_t live = (up < mq[0] ? 1u : 0u) | (up < mq[1] ? 2u : 0u) | (up < mq[2] ? 4u : 0u) |
                                      (up < mq[3] ? 8u : 0u);
                keep = ((uint32_t)qc[up] & live) != 0;
            } else {
                keep = !GROUPS || covers(keys[start + (uint64_t)p], cr);
            }
        }
        const uint64_t m = gsd::ballot(keep);
        const int cnt = __builtin_popcountll(m);
        const int take = min(cnt, 64 - n);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (keep && rank < take) S.idx[63 - n - rank] = (uint32_t)p;
        if (take < cnt) {
            uint64_t mm = m;
            for (int t = 0; t < take; ++t) mm &= mm - 1ull;
            sc -= (uint64_t)__builtin_ctzll(mm);
        } else {
            sc = sc > 64 ? sc - 64 : 0;
        }
        n += take;
    }
    *scan = sc;
    return n;
}

// One kept entry of the staged batch (geometry a, b, blue cb, list position
// pos) at one pixel of the forward walk.  Every lane evaluates the entry; the per-lane decisions (skip, stop,
// include) become lane masks, and the updates of a lane that includes the
// entry run under that mask.  A lane's values for an entry it includes are
// computed in exactly the order given above.
// Returns whether the pixel stops before this entry.
template <bool STATS>
__device__ __forceinline__ bool fwd_step(const float4 a, const float4 b, float cb, uint32_t pos, float pxc, float pyc,
                                         float& T, float& C0, float& C1, float& C2, bool active, uint32_t& lastn,
                                         uint32_t& n_eval, uint32_t& n_inc)
{
    const float dx = pxc - a.x, dy = pyc - a.y;
    float t = a.w * dy;
    t = __builtin_fmaf(a.z, dx, t);
    float u = b.x * dy;
    u = u * dy;
    const float power = __builtin_fmaf(t, dx, u);
    // -6 <= power <= 0: outside, alpha < 1/255 or power > 0, and the exp's
    // value (unclamped, so arbitrary) is unused
    const bool pok = gsd::falloff_in_range(power);
    const float G = gsd::exp_falloff_core(power);
    const float alpha = fminf(b.y * G, gsd::kAlphaMax);
    const bool inc = active && pok && !(alpha < gsd::kAlphaMin);
    const float Tn = T * (1.0f - alpha);
    const bool stop = inc && Tn < gsd::kTMin;
    const bool contrib = inc && !stop;
    if (STATS) {
        n_eval += active ? 1u : 0u;
        n_inc += contrib ? 1u : 0u;
    }
    // the empty volatile asm keeps the compiler from turning these branches
    // into selects on every lane
    if (contrib) {
        asm volatile("");
        const float w = alpha * T;
        C0 = __builtin_fmaf(b.z, w, C0);
        C1 = __builtin_fmaf(b.w, w, C1);
        C2 = __builtin_fmaf(cb, w, C2);
        T = Tn;
    }
    // a lane stops once per list: the end of its walk is the stopping entry's
    // list position
    if (stop) {
        asm volatile("");
        lastn = pos;
    }
    return stop;
}

template <bool STATS>
__global__ __launch_bounds__(256) void k_raster_fwd(LeafGeom g, const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ target, PixFrame tf, float inv_norm,
                                                    float* __restrict__ image, PixFrame imf,
                                                    float* __restrict__ tfinal,
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
    // end of the pixel's walk: the list position of the entry before which
    // compositing stopped, else the list length (no entry at or after it is
    // included, so the backward revisits the entries before it)
    uint32_t lastn = (uint32_t)(end - start), n_eval = 0, n_inc = 0;
    bool active = inside;
    for (uint64_t base = start; base < end; base += 64) {
        if (gsd::ballot(active) == 0) break;
        // lane i gathers entry i and tests it against the sub-tile; the kept
        // entries are packed to the front of the wavefront's LDS slice in list
        // order, each with its list position
        const uint64_t e = base + lane;
        bool keep = false;
        float4 a, b;
        float c = 0.0f;
        if (e < end) {
            const uint32_t s = values[e];
            a = g0[s];
            b = g1[s];
            c = g2[s].x;
            keep = !cull_box(a, b, bx0, by0);
        }
        const uint64_t km = gsd::ballot(keep);
        if (keep) {
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
            S.a[pos] = a;
            S.b[pos] = b;
            S.c[pos] = make_float4(c, __builtin_bit_cast(float, (uint32_t)(base - start) + (uint32_t)lane), 0.0f, 0.0f);
        }
        const int nk = __builtin_popcountll(km);
        gsd::wave_sync();
        for (int j = 0; j < nk; ++j) {
            const float4 ec = S.c[j];
            active = active && !fwd_step<STATS>(S.a[j], S.b[j], ec.x, __builtin_bit_cast(uint32_t, ec.y), pxc, pyc, T,
                                                C0, C1, C2, active, lastn, n_eval, n_inc);
        }
        gsd::wave_sync();
    }

    double l1 = 0.0;
    if (inside) {
        const float o0 = __builtin_fmaf(T, bg0, C0);
        const float o1 = __builtin_fmaf(T, bg1, C1);
        const float o2 = __builtin_fmaf(T, bg2, C2);
        if (image) {
            const int64_t ii = (int64_t)(py - imf.oy) * imf.stride + (px - imf.ox);
            image[ii] = o0;
            image[imf.plane + ii] = o1;
            image[2 * imf.plane + ii] = o2;
        }
        const int64_t lp = (int64_t)(py - g.py0) * g.WL + (px - g.px0);
        tfinal[lp] = T;
        last[lp] = lastn;
        if (target) {
            const int64_t ti = (int64_t)(py - tf.oy) * tf.stride + (px - tf.ox);
            const float t0 = target[ti], t1 = target[tf.plane + ti], t2 = target[2 * tf.plane + ti];
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
        // the backward revisits (those the forward examined: the backward
        // walks each pixel's list from the end of its forward walk)
        const double a0 = gsd::wave_sum_d((double)n_eval), a1 = gsd::wave_sum_d((double)n_inc);
        const double a2 = gsd::wave_sum_d((double)(inside ? lastn : 0u));
        const double a3 = gsd::wave_sum_d((double)n_eval);
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

// The backward walk of one tile by one wavefront (see k_raster_bwd): T, GS,
// the dL/dout factors gr0..gr2 and the walk ends lst of the lane's pixel in
// each quadrant, mq the largest end in each quadrant.
template <bool GROUPS>
__device__ __forceinline__ void bwd_walk(Staged& S, int lane, uint64_t start, const float (&pxc)[2],
                                         const float (&pyc)[2], const float (&bx)[2], const float (&by)[2],
                                         float (&T)[4], float (&GS)[4], const float (&gr0)[4],
                                         const float (&gr1)[4], const float (&gr2)[4], const uint32_t (&lst)[4],
                                         const uint32_t (&mq)[4], const uint32_t* __restrict__ values,
                                         const float4* __restrict__ g0, const float4* __restrict__ g1,
                                         const float4* __restrict__ g2, float* __restrict__ grad2d,
                                         const uint32_t* __restrict__ keys = nullptr, uint32_t cr = 0,
                                         const uint8_t* qcache = nullptr)
{
    const uint32_t maxl = max(max(mq[0], mq[1]), max(mq[2], mq[3]));

    // batches of 64 list entries, back to front; a group walk batches the
    // covering entries (collect_covering), the highest position in slot 63
    uint64_t scan = maxl;
    for (int64_t hi = maxl; (GROUPS || qcache) ? scan > 0 : hi > 0; hi -= 64) {
        bool has;
        uint32_t n_l;   // the lane's list position
        if (qcache) {
            const int nb = collect_live<GROUPS>(S, lane, keys, start, cr, qcache, mq, &scan);
            gsd::wave_sync();
            has = lane >= 64 - nb;
            n_l = has ? S.idx[lane] : 0u;
        } else if constexpr (GROUPS) {
            const int nb = collect_covering<false>(S, lane, keys, start, 0, cr, &scan);
            gsd::wave_sync();
            has = lane >= 64 - nb;
            n_l = has ? S.idx[lane] : 0u;
        } else {
            const int64_t lo = hi > 64 ? hi - 64 : 0;
            has = lane < (int)(hi - lo);
            n_l = (uint32_t)(lo + lane);
        }
        uint32_t qb = 0;
        if (has) {
            const uint32_t s = values[start + n_l];
            const float4 a = g0[s], b = g1[s];
            S.a[lane] = a;
            S.b[lane] = b;
            S.c[lane] = make_float4(g2[s].x, __builtin_bit_cast(float, s), __builtin_bit_cast(float, n_l), 0.0f);
            if (qcache && n_l < kQCache) {
                // the forward's cull of this entry, for the quadrants whose
                // walks reach it (they were compositing when it was culled)
                const uint32_t live = (n_l < mq[0] ? 1u : 0u) | (n_l < mq[1] ? 2u : 0u) | (n_l < mq[2] ? 4u : 0u) |
                                      (n_l < mq[3] ? 8u : 0u);
                qb = (uint32_t)qcache[n_l] & live;
            } else {
                const CullPrep cp = cull_prep(a, b);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (n_l < mq[k] && !cull_test(cp, bx[k & 1], by[k >> 1])) qb |= 1u << k;
            }
        }
        gsd::wave_sync();
        uint64_t mask = gsd::ballot(qb != 0);
        while (mask) {
            const int j = 63 - __builtin_clzll(mask);
            mask &= ~(1ull << j);
            const uint32_t qm = __builtin_amdgcn_readlane(qb, j);
            const float4 a = S.a[j];
            const float4 bb = S.b[j];
            const float4 cs = S.c[j];
            const uint32_t n = __builtin_bit_cast(uint32_t, cs.z);
            float p[9];
#pragma unroll
            for (int v = 0; v < 9; ++v) p[v] = 0.0f;
            bool any = false;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (!((qm >> k) & 1u)) continue;
                // Branch-free over the lanes, as in the forward: the inclusion
                // is re-derived with the forward's exact f32 operations, and
                // lanes that do not include the entry add zero partials.
                const float dx = pxc[k & 1] - a.x, dy = pyc[k >> 1] - a.y;
                float t = a.w * dy;
                t = __builtin_fmaf(a.z, dx, t);
                const float u1 = bb.x * dy;
                const float u = u1 * dy;
                const float power = __builtin_fmaf(t, dx, u);
                const bool pok = !(power > 0.0f);
                const float G = gsd::exp_falloff(power);
                const float av = bb.y * G;
                const bool clamped = av > gsd::kAlphaMax;
                const float alpha = clamped ? gsd::kAlphaMax : av;
                const bool contrib = n < lst[k] && pok && !(alpha < gsd::kAlphaMin);
                if (gsd::ballot(contrib) == 0) continue;
                any = true;
                // alpha of the lanes that include the entry, 0 on the others:
                // T / (1 - 0) = T and w = 0 leave those lanes' state unchanged
                const float ae = contrib ? alpha : 0.0f;
                // T before this entry = T after it / (1 - alpha)
                const float rom = __builtin_amdgcn_rcpf(1.0f - ae);
                T[k] = T[k] * rom;
                const float w = ae * T[k];
                // dL/dalpha = sum_ch g_ch (rgb_ch T - S_ch / (1 - alpha))
                const float grgb = __builtin_fmaf(gr2[k], cs.x, __builtin_fmaf(gr1[k], bb.w, gr0[k] * bb.z));
                const float dal0 = __builtin_fmaf(T[k], grgb, -(rom * GS[k]));
                GS[k] = __builtin_fmaf(grgb, w, GS[k]);
                p[6] = __builtin_fmaf(gr0[k], w, p[6]);
                p[7] = __builtin_fmaf(gr1[k], w, p[7]);
                p[8] = __builtin_fmaf(gr2[k], w, p[8]);
                // through alpha = o G, zero where alpha is clamped or not included
                const float dal = (contrib && !clamped) ? dal0 : 0.0f;
                p[5] = __builtin_fmaf(dal, G, p[5]);
                // power = -(A dx^2 + C dy^2)/2 - B dx dy with A = -2 a.z,
                // B = -a.w, C = -2 bb.x, dx = px - x, dy = py - y; with
                // q = -dL/dpower the five moments q dx, q dy, q dx dx,
                // q dx dy, q dy dy are summed here and give, once per entry,
                //   dL/dx = (A dx + B dy) dL/dpower = 2 a.z (q dx) + a.w (q dy)
                //   dL/dy = (C dy + B dx) dL/dpower = 2 bb.x (q dy) + a.w (q dx)
                //   dL/dA = (q dx dx)/2, dL/dB = q dx dy, dL/dC = (q dy dy)/2.
                const float q = -(dal * av);
                const float qdx = q * dx, qdy = q * dy;
                p[0] += qdx;
                p[1] += qdy;
                p[2] = __builtin_fmaf(qdx, dx, p[2]);
                p[3] = __builtin_fmaf(qdx, dy, p[3]);
                p[4] = __builtin_fmaf(qdy, dy, p[4]);
            }
            if (!any) continue;
            const float m0 = p[0], m1 = p[1];
            p[0] = 2.0f * a.z * m0 + a.w * m1;
            p[1] = 2.0f * bb.x * m1 + a.w * m0;
            p[2] = 0.5f * p[2];
            p[4] = 0.5f * p[4];
            int v;
            const float r = wave_reduce9(p, lane, &v);
            if (v >= 0 && r != 0.0f) {
                const uint32_t slot = __builtin_bit_cast(uint32_t, cs.y);
                unsafeAtomicAdd(&grad2d[(int64_t)slot * 9 + v], r);
            }
        }
        gsd::wave_sync();
    }
}

// Backward, one wavefront per 16 x 16 tile, four tiles per workgroup and no
// workgroup barrier.  Lane l owns pixel l (x = l % 8, y = l / 8) of each 8 x 8
// quadrant k of the tile (k & 1: right half, k >> 1: bottom half).  The
// wavefront walks the tile's list back to front from the furthest end of its
// pixels' forward walks, 64 entries per batch staged in its own LDS slice;
// lane i gathers entry i and sets bit k of the entry's quadrant mask when the
// entry precedes the end of some forward walk in quadrant k and survives the cull
// against quadrant k's box.  Per entry, the quadrants of the mask are
// evaluated in turn (one wave-uniform branch each, skipped when none of the
// quadrant's pixels includes the entry); the partials of a lane's four pixels
// are summed in registers, the moments become the partials of the mean and
// the conic, and one transposed reduction over the wavefront and one 9-lane
// atomic add follow.  Entries that reach a tile mostly cover all of its
// quadrants, so a tile-wide reduction replaces up to four per-quadrant ones.
__global__ __launch_bounds__(256) void k_raster_bwd(LeafGeom g, int64_t n_tiles,
                                                    const uint64_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ values,
                                                    const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                    const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                    const float* __restrict__ tfinal,
                                                    const uint32_t* __restrict__ last,
                                                    const uint8_t* __restrict__ sgn, float inv_norm,
                                                    const float* __restrict__ dl_dimage, PixFrame dlf,
                                                    float* __restrict__ grad2d)
{
    __shared__ Staged st[4];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t lt = (int64_t)blockIdx.x * 4 + wave;
    if (lt >= n_tiles) return;
    Staged& S = st[wave];
    const int tx = g.ltx0 + (int)(lt % g.TWL), ty = g.lty0 + (int)(lt / g.TWL);
    const int qx = lane & 7, qy = lane >> 3;
    float pxc[2], pyc[2], bx[2], by[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        pxc[h] = (float)(tx * 16 + h * 8 + qx) + 0.5f;
        pyc[h] = (float)(ty * 16 + h * 8 + qy) + 0.5f;
        bx[h] = (float)(tx * 16 + h * 8) + 0.5f;
        by[h] = (float)(ty * 16 + h * 8) + 0.5f;
    }
    const uint64_t start = offsets[lt];

    // per quadrant k: transmittance after the last included entry, dL/dout,
    // GS = sum_ch dL/dout_ch * (colour behind the current entry, ch), which
    // starts as the background seen through T_final, and the end of the walk
    float T[4], GS[4], gr0[4], gr1[4], gr2[4];
    uint32_t lst[4], mq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int px = tx * 16 + (k & 1) * 8 + qx, py = ty * 16 + (k >> 1) * 8 + qy;
        T[k] = 1.0f;
        gr0[k] = gr1[k] = gr2[k] = 0.0f;
        lst[k] = 0;
        if (px < g.W && py < g.H) {
            const int64_t lp = (int64_t)(py - g.py0) * g.WL + (px - g.px0);
            T[k] = tfinal[lp];
            lst[k] = last[lp];
            if (dl_dimage) {
                const int64_t di = (int64_t)(py - dlf.oy) * dlf.stride + (px - dlf.ox);
                gr0[k] = dl_dimage[di];
                gr1[k] = dl_dimage[dlf.plane + di];
                gr2[k] = dl_dimage[2 * dlf.plane + di];
            } else {
                const uint32_t c = sgn[lp];
                auto dec = [&](uint32_t code) { return code == 1u ? inv_norm : (code == 2u ? -inv_norm : 0.0f); };
                gr0[k] = dec(c & 3u);
                gr1[k] = dec((c >> 2) & 3u);
                gr2[k] = dec((c >> 4) & 3u);
            }
        }
        GS[k] = T[k] * (gr0[k] * bg0 + gr1[k] * bg1 + gr2[k] * bg2);
        mq[k] = __builtin_amdgcn_readfirstlane(gsd::wave_max_u32(lst[k]));
    }
    bwd_walk<false>(S, lane, start, pxc, pyc, bx, by, T, GS, gr0, gr1, gr2, lst, mq, values, g0, g1, g2, grad2d);
}


// Forward, L1 loss and backward of one tile in one wavefront, for views
// whose loss gradient at a pixel depends on that pixel alone (L1): the
// per-pixel state the backward needs (T_final, the end of the walk, the
// residual signs) stays in registers instead of going through memory, and
// each tile's list is gathered and culled once for its four quadrants.
// Lane l owns pixel l of each 8 x 8 quadrant, as in the backward.  Forward:
// 64 entries per batch; lane i gathers entry i and marks the quadrants (with
// a pixel still compositing) whose box it can reach; the kept entries are
// packed in LDS with their list position and quadrant mask, and each is
// composited into the pixels of its quadrants (fwd_step, the same operations
// as k_raster_fwd).  The image, the L1 partial of the tile and dL/dout =
// sgn(out - target) / (3WH) follow, then the backward walk (bwd_walk).
// One wavefront per workgroup: a tile's wavefront frees its slot the moment
// it ends, instead of waiting for the other tiles of a shared workgroup.
// GROUPS = false: the tile's list is [offsets[lt], offsets[lt + 1]) of
// `values`.  GROUPS = true: the tile walks its super-tile's group
// [offsets[sc], offsets[sc + 1]) of `values` (slots) and `keys` (coarse keys),
// taking the entries that cover it (`covers`) -- the same entries in the same
// order, so every value is the same, and no per-tile list is written.  List
// positions (walk ends) then count group entries.
constexpr int kFusedWaves = 1;
template <bool BWD, bool GROUPS>   // BWD false: forward and L1 only (a view whose backward is skipped)
__global__ __launch_bounds__(64 * kFusedWaves) void k_raster_fused(LeafGeom g, int64_t n_tiles,
                                                      const uint64_t* __restrict__ offsets,
                                                      const uint32_t* __restrict__ values,
                                                      const float4* __restrict__ g0, const float4* __restrict__ g1,
                                                      const float4* __restrict__ g2, float bg0, float bg1, float bg2,
                                                      const float* __restrict__ target, PixFrame tf, float inv_norm,
                                                      float* __restrict__ image, double* __restrict__ l1_part,
                                                      float* __restrict__ grad2d, const uint32_t* __restrict__ order,
                                                      const uint32_t* __restrict__ keys, int SW)
{
    __shared__ Staged st[kFusedWaves];
    __shared__ uint8_t qc[kFusedWaves][kQCache];   // the forward's quadrant mask of each list position
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kFusedWaves + wave;
    if (w >= n_tiles) return;
    const int64_t lt = order[w];
    Staged& S = st[wave];
    const int tx = g.ltx0 + (int)(lt % g.TWL), ty = g.lty0 + (int)(lt / g.TWL);
    const int qx = lane & 7, qy = lane >> 3;
    float pxc[2], pyc[2], bx[2], by[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        pxc[h] = (float)(tx * 16 + h * 8 + qx) + 0.5f;
        pyc[h] = (float)(ty * 16 + h * 8 + qy) + 0.5f;
        bx[h] = (float)(tx * 16 + h * 8) + 0.5f;
        by[h] = (float)(ty * 16 + h * 8) + 0.5f;
    }
    // the tile's own list, or its super-tile's group and its place in it
    const int64_t li = GROUPS ? (int64_t)((ty >> kSuperShift) - (g.lty0 >> kSuperShift)) * SW +
                                    ((tx >> kSuperShift) - (g.ltx0 >> kSuperShift))
                              : lt;
    const uint32_t cr = (uint32_t)(tx & 7) | ((uint32_t)(ty & 7) << 3);
    const uint64_t start = offsets[li], end = offsets[li + 1];

    // ---- forward over the four quadrants
    // a pixel is still compositing while its walk end is the list length:
    // a stop sets it to the stopping entry's position, which is smaller;
    // pixels outside the image start at 0 (nothing to walk)
    float T[4], C0[4], C1[4], C2[4];
    uint32_t lst[4];
    bool inside[4];
    const uint32_t len = (uint32_t)(end - start);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int px = tx * 16 + (k & 1) * 8 + qx, py = ty * 16 + (k >> 1) * 8 + qy;
        inside[k] = px < g.W && py < g.H;
        T[k] = 1.0f;
        C0[k] = C1[k] = C2[k] = 0.0f;
        lst[k] = inside[k] ? len : 0u;
    }
    uint32_t n_eval = 0, n_inc = 0;   // unused (no statistics here)
    // batches of 64 list entries; a group walk batches the covering entries
    uint64_t scan = start;
    for (uint64_t base = start; GROUPS ? scan < end : base < end; base += 64) {
        uint32_t aq = 0;   // quadrants with a pixel still compositing
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (gsd::ballot(lst[k] == len) != 0) aq |= 1u << k;
        if (aq == 0) break;
        bool has;
        uint32_t ep;   // the lane's list position
        if constexpr (GROUPS) {
            uint64_t rel = scan - start;
            const int nb = collect_covering<true>(S, lane, keys, start, end - start, cr, &rel,
                                                  BWD ? qc[wave] : nullptr);
            scan = start + rel;
            gsd::wave_sync();
            has = lane < nb;
            ep = has ? S.idx[lane] : 0u;
        } else {
            has = base + lane < end;
            ep = (uint32_t)(base - start) + (uint32_t)lane;
        }
        uint32_t qb = 0;
        float4 a, b;
        float c = 0.0f;
        if (has) {
            const uint32_t s = values[start + ep];
            a = g0[s];
            b = g1[s];
            c = g2[s].x;
            const CullPrep cp = cull_prep(a, b);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (((aq >> k) & 1u) && !cull_test(cp, bx[k & 1], by[k >> 1])) qb |= 1u << k;
            if (BWD && ep < kQCache) qc[wave][ep] = (uint8_t)qb;
        }
        const uint64_t km = gsd::ballot(qb != 0);
        if (qb != 0) {
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
            S.a[pos] = a;
            S.b[pos] = b;
            S.c[pos] = make_float4(c, __builtin_bit_cast(float, ep), __builtin_bit_cast(float, qb), 0.0f);
        }
        const int nk = __builtin_popcountll(km);
        gsd::wave_sync();
        for (int j = 0; j < nk; ++j) {
            const float4 ea = S.a[j];
            const float4 eb = S.b[j];
            const float4 ec = S.c[j];
            const uint32_t qm = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, ec.z));
            const uint32_t pos = __builtin_bit_cast(uint32_t, ec.y);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((qm >> k) & 1u)
                    (void)fwd_step<false>(ea, eb, ec.x, pos, pxc[k & 1], pyc[k >> 1], T[k], C0[k], C1[k], C2[k],
                                          lst[k] == len, lst[k], n_eval, n_inc);
        }
        gsd::wave_sync();
    }

    // ---- image, L1 and dL/dout
    float GS[4], gr0[4], gr1[4], gr2[4];
    uint32_t mq[4];
    double l1 = 0.0;
    const int64_t P = (int64_t)g.W * g.H;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        gr0[k] = gr1[k] = gr2[k] = 0.0f;
        if (inside[k]) {
            const int px = tx * 16 + (k & 1) * 8 + qx, py = ty * 16 + (k >> 1) * 8 + qy;
            const float o0 = __builtin_fmaf(T[k], bg0, C0[k]);
            const float o1 = __builtin_fmaf(T[k], bg1, C1[k]);
            const float o2 = __builtin_fmaf(T[k], bg2, C2[k]);
            const int64_t gi = (int64_t)py * g.W + px;
            if (image) {
                image[gi] = o0;
                image[P + gi] = o1;
                image[2 * P + gi] = o2;
            }
            const int64_t ti = (int64_t)(py - tf.oy) * tf.stride + (px - tf.ox);
            const float t0 = target[ti], t1 = target[tf.plane + ti], t2 = target[2 * tf.plane + ti];
            const float d0 = o0 - t0, d1 = o1 - t1, d2 = o2 - t2;   // sign exact in f32
            gr0[k] = d0 > 0.0f ? inv_norm : (d0 < 0.0f ? -inv_norm : 0.0f);
            gr1[k] = d1 > 0.0f ? inv_norm : (d1 < 0.0f ? -inv_norm : 0.0f);
            gr2[k] = d2 > 0.0f ? inv_norm : (d2 < 0.0f ? -inv_norm : 0.0f);
            l1 += fabs((double)o0 - (double)t0) + fabs((double)o1 - (double)t1) + fabs((double)o2 - (double)t2);
        }
        GS[k] = T[k] * (gr0[k] * bg0 + gr1[k] * bg1 + gr2[k] * bg2);
        mq[k] = __builtin_amdgcn_readfirstlane(gsd::wave_max_u32(lst[k]));
    }
    l1 = gsd::wave_sum_d(l1);
    if (lane < 4) l1_part[lt * 4 + lane] = lane == 0 ? l1 : 0.0;
    if (!BWD) return;

    // ---- backward
    bwd_walk<GROUPS>(S, lane, start, pxc, pyc, bx, by, T, GS, gr0, gr1, gr2, lst, mq, values, g0, g1, g2, grad2d,
                     keys, cr, qc[wave]);
}


// ---- launch order of the fused kernel's tiles -------------------------------
// A wavefront's work grows with its tile's list, and the lists of one leaf
// differ by orders of magnitude, so the tiles are launched longest first
// (bucketed by half octaves of the list length; order inside a bucket
// unspecified): the last wavefronts of the launch are then short ones.
__device__ __forceinline__ int len_bucket(uint64_t len)
{
    if (len < 2) return (int)len;
    const int msb = 63 - __builtin_clzll(len);
    return 2 * msb + (int)((len >> (msb - 1)) & 1u);   // 2 .. 127 for len < 2^64
}

// Lanes with b >= 0 add themselves to ctr[b] (one LDS atomic per distinct b
// in the wavefront); each gets its rank among all adds to its counter.
__device__ __forceinline__ uint32_t wave_bucket_add(int b, uint32_t* ctr, int lane)
{
    uint32_t slot = 0;
    uint64_t pending = gsd::ballot(b >= 0);
    while (pending) {
        const int leader = __builtin_ctzll(pending);
        const int bl = __builtin_amdgcn_readlane(b, leader);
        const uint64_t grp = gsd::ballot(b == bl);
        uint32_t old = 0;
        if (lane == leader) old = atomicAdd(&ctr[bl], (uint32_t)__builtin_popcountll(grp));
        old = __builtin_amdgcn_readlane(old, leader);
        if (b == bl)
            slot = old + __builtin_amdgcn_mbcnt_hi((uint32_t)(grp >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)grp, 0u));
        pending &= ~grp;
    }
    return slot;
}

// The tiles of list set L (its offsets start at offsets0 + base[L], its
// order goes to order0 + base[L], base[L + 1] - base[L] - 1 tiles; base =
// null: one set of n1 tiles at 0) by bucket, longest first, on a grid of
// (chunk of kOrderChunk tiles, set): every block counts its tiles per bucket
// in LDS and adds the counts to the set's (k_order_count); one thread per set
// turns them into the buckets' starts, longest bucket first (k_order_base);
// every block counts again, reserves a range of each bucket of its set with
// one atomic per bucket, and places its tiles there (k_order_place).  The
// order of the tiles inside a bucket depends on the order of those atomics.
constexpr int kOrderChunk = 4096;

__device__ __forceinline__ void order_set(const uint64_t* base, int64_t n1, int set, uint64_t& b0, int64_t& n)
{
    b0 = base ? base[set] : 0;
    n = base ? (int64_t)(base[set + 1] - b0) - 1 : n1;
}

__global__ __launch_bounds__(256) void k_order_count(int64_t n1, const uint64_t* __restrict__ base,
                                                     const uint64_t* __restrict__ offsets0, uint32_t* __restrict__ cnt)
{
    __shared__ uint32_t ctr[128];
    uint64_t b0;
    int64_t n;
    order_set(base, n1, blockIdx.y, b0, n);
    const int64_t i0 = (int64_t)blockIdx.x * kOrderChunk, i1 = min(n, i0 + kOrderChunk);
    if (i0 >= i1) return;
    const uint64_t* __restrict__ offsets = offsets0 + b0;
    const int t = threadIdx.x, lane = t & 63;
    if (t < 128) ctr[t] = 0;
    __syncthreads();
    for (int64_t c = i0; c < i1; c += 256) {
        const int64_t i = c + t;
        const int b = i < i1 ? len_bucket(offsets[i + 1] - offsets[i]) : -1;
        (void)wave_bucket_add(b, ctr, lane);
    }
    __syncthreads();
    if (t < 128 && ctr[t]) atomicAdd(&cnt[(int64_t)blockIdx.y * 128 + t], ctr[t]);
}

__global__ __launch_bounds__(256) void k_order_base(int n_sets, uint32_t* __restrict__ cnt)
{
    for (int L = blockIdx.x * 256 + threadIdx.x; L < n_sets; L += gridDim.x * 256) {
        uint32_t run = 0;
        for (int b = 127; b >= 0; --b) {
            const uint32_t c = cnt[(int64_t)L * 128 + b];
            cnt[(int64_t)L * 128 + b] = run;
            run += c;
        }
    }
}

__global__ __launch_bounds__(256) void k_order_place(int64_t n1, const uint64_t* __restrict__ base,
                                                     const uint64_t* __restrict__ offsets0, uint32_t* __restrict__ cursor,
                                                     uint32_t* __restrict__ order0)
{
    __shared__ uint32_t ctr[128], start[128];
    uint64_t b0;
    int64_t n;
    order_set(base, n1, blockIdx.y, b0, n);
    const int64_t i0 = (int64_t)blockIdx.x * kOrderChunk, i1 = min(n, i0 + kOrderChunk);
    if (i0 >= i1) return;
    const uint64_t* __restrict__ offsets = offsets0 + b0;
    uint32_t* __restrict__ order = order0 + b0;
    const int t = threadIdx.x, lane = t & 63;
    if (t < 128) ctr[t] = 0;
    __syncthreads();
    for (int64_t c = i0; c < i1; c += 256) {
        const int64_t i = c + t;
        const int b = i < i1 ? len_bucket(offsets[i + 1] - offsets[i]) : -1;
        (void)wave_bucket_add(b, ctr, lane);
    }
    __syncthreads();
    if (t < 128) {
        start[t] = ctr[t] ? atomicAdd(&cursor[(int64_t)blockIdx.y * 128 + t], ctr[t]) : 0u;
        ctr[t] = 0;
    }
    __syncthreads();
    for (int64_t c = i0; c < i1; c += 256) {
        const int64_t i = c + t;
        const int b = i < i1 ? len_bucket(offsets[i + 1] - offsets[i]) : -1;
        const uint32_t pos = wave_bucket_add(b, ctr, lane);
        if (b >= 0) order[start[b] + pos] = (uint32_t)i;
    }
}

}  // namespace

gs_status launch_raster_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            gs_raster* r, const float* target, PixFrame tf, float* image_out, PixFrame imf,
                            double* loss_accum, uint64_t* stats)
{
    const LeafGeom g = make_geom(cam, bins, r);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_fwd");
        if (stats)
            hipLaunchKernelGGL(k_raster_fwd<true>, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g,
                               bins->offsets, bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1],
                               cam->bg[2], target, tf, inv_norm, image_out, imf, r->tfinal, r->last, r->sgn, r->l1_part,
                               (unsigned long long*)stats);
        else
            hipLaunchKernelGGL(k_raster_fwd<false>, dim3((unsigned)bins->n_tiles), dim3(256), 0, ctx->stream, g,
                               bins->offsets, bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1],
                               cam->bg[2], target, tf, inv_norm, image_out, imf, r->tfinal, r->last, r->sgn, r->l1_part,
                               nullptr);
    }
    GS_HIP(ctx, hipGetLastError());
    if (target && loss_accum) return launch_sum_f64(ctx, r->l1_part, bins->n_tiles * 4, 1, loss_accum, 1);
    return GS_OK;
}

gs_status launch_raster_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            const gs_raster* r, const float* dl_dimage, PixFrame dlf, float* grad2d)
{
    const LeafGeom g = make_geom(cam, bins, r);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    if (bins->n_tiles > 0) {
        GsTimerScope ts(ctx, "raster_bwd");
        const int64_t nt = bins->n_tiles;
        hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)((nt + 3) / 4)), dim3(256), 0, ctx->stream, g, nt,
                           bins->offsets, bins->values, proj->g0, proj->g1, proj->g2, cam->bg[0], cam->bg[1], cam->bg[2],
                           r->tfinal, r->last, r->sgn, inv_norm, dl_dimage, dlf, grad2d);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

// The fused raster of one leaf over its tiles in `order` (null: longest list
// first, computed here from the tile offsets; lists only).  groups: the tiles
// walk their super-tiles' groups (offsets = group offsets, values = slots,
// keys = coarse keys); else their own lists.
static gs_status fused_launch(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, gs_tile_rect leaf,
                              const uint64_t* offsets, const uint32_t* values, const uint32_t* keys, bool groups,
                              const uint32_t* order, const float* target, PixFrame tf, float* image_out,
                              double* l1_part, float* grad2d, bool backward)
{
    LeafGeom g;
    g.W = cam->width;
    g.H = cam->height;
    g.ltx0 = leaf.tx0;
    g.lty0 = leaf.ty0;
    g.TWL = leaf.tx1 - leaf.tx0;
    g.px0 = leaf.tx0 * 16;
    g.py0 = leaf.ty0 * 16;
    g.WL = std::min(leaf.tx1 * 16, cam->width) - g.px0;
    g.PL = (int64_t)g.WL * (std::min(leaf.ty1 * 16, cam->height) - g.py0);
    const int SW = super_cols(leaf);
    const float inv_norm = (float)(1.0 / (3.0 * (double)cam->width * (double)cam->height));
    const int64_t nt = (int64_t)g.TWL * (leaf.ty1 - leaf.ty0);
    if (nt > 0) {
        std::vector<GsAlloc> tmp;
        if (!order) {
            if (groups) return gs_fail(ctx, GS_ERR_INVALID_ARG, "group-walking raster without a tile order");
            uint32_t* o = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nt, GS_MEM_RASTER, &tmp);
            if (!o) return GS_ERR_OOM;
            gs_leaf one{};
            one.tx1 = g.TWL;
            one.ty1 = leaf.ty1 - leaf.ty0;
            const gs_status so = launch_tile_order(ctx, 1, &one, nullptr, nt, offsets, o);
            if (so != GS_OK) {
                gs_free_all(ctx, &tmp);
                return so;
            }
            order = o;
        }
        {
            GsTimerScope ts(ctx, backward ? "raster_fused" : "raster_fused_fwd");
            const dim3 grid((unsigned)ceil_div(nt, kFusedWaves)), block(64 * kFusedWaves);
#define GS_FUSED(B, G)                                                                                            \
    hipLaunchKernelGGL((k_raster_fused<B, G>), grid, block, 0, ctx->stream, g, nt, offsets, values, proj->g0,     \
                       proj->g1, proj->g2, cam->bg[0], cam->bg[1], cam->bg[2], target, tf, inv_norm, image_out,   \
                       l1_part, grad2d, order, keys, SW)
            if (backward) {
                if (groups) GS_FUSED(true, true);
                else GS_FUSED(true, false);
            } else {
                if (groups) GS_FUSED(false, true);
                else GS_FUSED(false, false);
            }
#undef GS_FUSED
        }
        gs_free_all(ctx, &tmp);
    }
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_raster_fused(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                              const float* target, PixFrame tf, float* image_out, double* l1_part, float* grad2d,
                              bool backward)
{
    return fused_launch(ctx, cam, proj, bins->leaf, bins->offsets, bins->values, nullptr, false, bins->order, target,
                        tf, image_out, l1_part, grad2d, backward);
}

gs_status launch_raster_groups(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, gs_tile_rect leaf,
                               const uint64_t* soff, const uint32_t* group, const uint32_t* gkey,
                               const uint32_t* order, const float* target, PixFrame tf, float* image_out,
                               double* l1_part, float* grad2d, bool backward)
{
    return fused_launch(ctx, cam, proj, leaf, soff, group, gkey, true, order, target, tf, image_out, l1_part, grad2d,
                        backward);
}

gs_status launch_tile_order(gs_ctx* ctx, int32_t n_sets, const gs_leaf* hleaves, const uint64_t* base, int64_t n1,
                            const uint64_t* offsets, uint32_t* order)
{
    if (n_sets <= 0) return GS_OK;
    int64_t nch = 1;
    for (int32_t L = 0; L < n_sets; ++L)
        nch = std::max<int64_t>(nch, ceil_div((int64_t)(hleaves[L].tx1 - hleaves[L].tx0) *
                                              (hleaves[L].ty1 - hleaves[L].ty0), kOrderChunk));
    std::vector<GsAlloc> tmp;
    uint32_t* cnt = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * 128 * (size_t)n_sets, GS_MEM_SCRATCH, &tmp);
    if (!cnt) return GS_ERR_OOM;
    gs_status st = launch_fill_u32(ctx, cnt, 0u, 128 * (int64_t)n_sets);
    if (st == GS_OK) {
        GsTimerScope ts(ctx, "tile_order");
        const dim3 grid((unsigned)nch, (unsigned)n_sets);
        hipLaunchKernelGGL(k_order_count, grid, dim3(256), 0, ctx->stream, n1, base, offsets, cnt);
        hipLaunchKernelGGL(k_order_base, dim3((unsigned)ceil_div(n_sets, 256)), dim3(256), 0, ctx->stream, n_sets, cnt);
        hipLaunchKernelGGL(k_order_place, grid, dim3(256), 0, ctx->stream, n1, base, offsets, cnt, order);
    }
    gs_free_all(ctx, &tmp);
    if (st != GS_OK) return st;
    GS_HIP(ctx, hipGetLastError());
    return GS_OK;
}

gs_status launch_tile_order_sets(gs_ctx* ctx, int32_t n_sets, const gs_leaf* hleaves, const uint64_t* base,
                                 const uint64_t* offsets, uint32_t* order)
{
    return launch_tile_order(ctx, n_sets, hleaves, base, 0, offsets, order);
}
