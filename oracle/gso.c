/*
 * gso.c -- CPU oracle for one training view of differentiable tile-based 3D
 * Gaussian splatting with load-budgeted leaves.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU baseline load it.
 * Plain, slow, single-threaded C; see gso.h for what each entry computes and
 * which passage of the pages it follows.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (contraction off, so every a*b+c below is two roundings unless fma() is
 * written; no -march flags, so the library runs on any x86-64 host).
 */
#include "gso.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n;        /* index in the tile list */
    uint32_t slot;    /* candidate slot */
    int32_t clamped;  /* alpha was clamped to 0.99 */
} gso_rec;

/* ---------------------------------------------------------------------- */
/* exp_cw: exp(x) in f32 by Cody & Waite's argument reduction (Cody and
 * Waite, "Software Manual for the Elementary Functions", 1980):
 *   k = rint(x log2 e),  r = x - k ln2  with ln2 = ln2_hi + ln2_lo, where
 *   ln2_hi is ln2 rounded to f32 with the low 12 significand bits cleared
 *   (so k * ln2_hi is exact for |k| < 2^12), ln2_lo = f32(ln2 - ln2_hi);
 *   e^r by the degree-7 Taylor polynomial sum r^n/n! in Horner form (fma),
 *   coefficients 1/n! rounded to f32;  result ldexp(p, k).
 * x < -87 gives 0, x > 88.7 gives +inf, NaN propagates.  The same
 * definition is what the rasterizer's alpha uses, so that both sides take
 * every alpha threshold decision on identical bits.                       */
static float ln2_hi_f32(void)
{
    float f = (float)0.693147180559945309417232121458;   /* ln 2 */
    uint32_t u;
    memcpy(&u, &f, 4);
    u &= 0xFFFFF000u;
    memcpy(&f, &u, 4);
    return f;
}

float gso_exp_cw(float x)
{
    static int init = 0;
    static float ln2_hi, ln2_lo, log2e, c[8];
    if (!init) {
        ln2_hi = ln2_hi_f32();
        ln2_lo = (float)(0.693147180559945309417232121458 - (double)ln2_hi);
        log2e = 1.44269504088896340736f;                    /* 1/ln 2 */
        double fact = 1.0;
        for (int k = 0; k < 8; ++k) {
            if (k > 0) fact *= k;
            c[k] = (float)(1.0 / fact);                     /* 1/k!, exact double then f32 */
        }
        init = 1;
    }
    if (x < -87.0f) return 0.0f;
    if (x > 88.7f) return INFINITY;
    if (x != x) return x;
    const float k = rintf(x * log2e);
    float r = fmaf(-k, ln2_hi, x);
    r = fmaf(-k, ln2_lo, r);
    float p = c[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, c[i]);
    return ldexpf(p, (int)k);
}

void gso_exp_cw_array(const float* x, float* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = gso_exp_cw(x[i]);
}

/* exp_falloff: the f32 exp of the Gaussian falloff in alpha = min(0.99,
 * o exp(power)).  Since o <= 1, alpha >= 1/255 needs power > -ln 255 = -5.54,
 * so the argument is first clamped into [-6, 0]: below -6 every pixel skips
 * the entry whatever the value (o exp(-6) < 1/255), above 0 the entry is
 * skipped before exp is taken.  On [-6, 0]:
 *   k = x log2 e rounded once to the nearest integer (ties to even), taken
 *       from t = fma(x, log2 e, 1.5 * 2^23): at that magnitude the f32 ulp is
 *       1, so t - 1.5 * 2^23 is exactly that integer;
 *   r = fma(-k, ln2, x) with ln 2 rounded to f32 (|k| <= 9 keeps the error of
 *       the one-constant reduction below 2e-8);
 *   e^r = 1 + r + r^2 (c2 + c3 r + c4 r^2 + c5 r^3 + c6 r^4) in Horner form
 *       (fma): the degree-6 polynomial with constant and linear terms 1 and
 *       the least maximum relative error on |r| <= ln2/2 (a linear-programming
 *       minimax fit; 4.9e-9 with the coefficients rounded to f32, given below
 *       by their bit patterns);
 *   result ldexp(p, k).
 * Within 1 ulp of exp on [-6, 0] (every f32 there: 0.39 % of them 1 ulp
 * away from the correctly rounded value, the rest exact).  NaN gives an
 * unspecified value.                                                       */
static float f32_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float gso_exp_falloff(float x)
{
    const float c2 = f32_bits(0x3efffffeu), c3 = f32_bits(0x3e2aaa2du), c4 = f32_bits(0x3d2aabbeu);
    const float c5 = f32_bits(0x3c092e32u), c6 = f32_bits(0x3ab5dcf3u);
    if (x < -6.0f) x = -6.0f;
    if (x > 0.0f) x = 0.0f;
    const float magic = 12582912.0f;                        /* 1.5 * 2^23 */
    const float t = fmaf(x, 1.44269504088896340736f, magic);
    const float k = t - magic;
    const float r = fmaf(-k, (float)0.693147180559945309417232121458, x);
    float p = c6;
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)k);
}

void gso_exp_falloff_array(const float* x, float* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = gso_exp_falloff(x[i]);
}

/* ---------------------------------------------------------------------- */
/* The REAL-generic forward arithmetic, compiled in f32 and in f64.        */
#define SFX(name) name##_f32
#define REAL float
#define LIT(x) x##f
#define EXPF(x) gso_exp_cw(x)
#define EXP_FALLOFF(x) gso_exp_falloff(x)
#define SQRTF(x) sqrtf(x)
#define CEILF(x) ceilf(x)
#define FLOORF(x) floorf(x)
#define FMA(a, b, c) fmaf(a, b, c)
#define ISFIN(x) isfinite(x)
#include "gso_real.inc"
#undef SFX
#undef REAL
#undef LIT
#undef EXPF
#undef EXP_FALLOFF
#undef SQRTF
#undef CEILF
#undef FLOORF
#undef FMA

#define SFX(name) name##_f64
#define REAL double
#define LIT(x) x
#define EXPF(x) exp(x)
#define EXP_FALLOFF(x) exp(x)
#define SQRTF(x) sqrt(x)
#define CEILF(x) ceil(x)
#define FLOORF(x) floor(x)
#define FMA(a, b, c) fma(a, b, c)
#include "gso_real.inc"
#undef SFX
#undef REAL
#undef LIT
#undef EXPF
#undef EXP_FALLOFF
#undef SQRTF
#undef CEILF
#undef FLOORF
#undef FMA

/* ---------------------------------------------------------------------- */
/* Binning (integer).  BoundedGS page, "01": raster buffers grow with the
 * overlaps of Gaussians and image tiles.  One entry per (candidate, tile of
 * its rectangle inside the leaf), ordered by (global tile, depth, slot).   */
typedef struct { uint32_t tile; uint32_t slot; double depth; } bin_ent;

static int bin_cmp(const void* pa, const void* pb)
{
    const bin_ent* a = (const bin_ent*)pa;
    const bin_ent* b = (const bin_ent*)pb;
    if (a->tile != b->tile) return a->tile < b->tile ? -1 : 1;
    if (a->depth != b->depth) return a->depth < b->depth ? -1 : 1;
    if (a->slot != b->slot) return a->slot < b->slot ? -1 : 1;
    return 0;
}

int64_t gso_bin(int32_t tiles_x, gso_rect leaf, int64_t n_cand, const int32_t* rect,
                const double* depth, const uint32_t* depth_bits,
                uint32_t* counts, uint64_t* offsets, uint32_t* values, uint64_t* keys,
                int64_t cap)
{
    const int32_t TWL = leaf.tx1 - leaf.tx0, THL = leaf.ty1 - leaf.ty0;
    const int64_t TL = (int64_t)TWL * THL;
    for (int64_t t = 0; t < TL; ++t) counts[t] = 0;
    for (int64_t j = 0; j < n_cand; ++j) {
        const int32_t* r = rect + 4 * j;
        for (int32_t ty = r[1]; ty < r[3]; ++ty)
            for (int32_t tx = r[0]; tx < r[2]; ++tx)
                if (tx >= leaf.tx0 && tx < leaf.tx1 && ty >= leaf.ty0 && ty < leaf.ty1)
                    counts[(int64_t)(ty - leaf.ty0) * TWL + (tx - leaf.tx0)] += 1;
    }
    uint64_t total = 0;
    for (int64_t t = 0; t < TL; ++t) { offsets[t] = total; total += counts[t]; }
    offsets[TL] = total;
    if (values == NULL || cap < (int64_t)total) return (int64_t)total;

    bin_ent* e = (bin_ent*)malloc(sizeof(bin_ent) * (total ? total : 1));
    int64_t m = 0;
    for (int64_t j = 0; j < n_cand; ++j) {
        const int32_t* r = rect + 4 * j;
        for (int32_t ty = r[1]; ty < r[3]; ++ty)
            for (int32_t tx = r[0]; tx < r[2]; ++tx)
                if (tx >= leaf.tx0 && tx < leaf.tx1 && ty >= leaf.ty0 && ty < leaf.ty1) {
                    e[m].tile = (uint32_t)((int64_t)ty * tiles_x + tx);
                    e[m].slot = (uint32_t)j;
                    e[m].depth = depth[j];
                    ++m;
                }
    }
    qsort(e, (size_t)m, sizeof(bin_ent), bin_cmp);
    for (int64_t k = 0; k < m; ++k) {
        values[k] = e[k].slot;
        if (keys) keys[k] = ((uint64_t)e[k].tile << 32) | (depth_bits ? depth_bits[e[k].slot] : 0u);
    }
    free(e);
    return (int64_t)total;
}

/* ---------------------------------------------------------------------- */
/* Losses (f64).  L1 with the full-image normaliser on every leaf, so the
 * leaf losses add up to the view's loss (BoundedGS page, "01": one
 * gradient for the complete view).                                        */
double gso_loss_l1(int32_t W, int32_t H, gso_rect leaf, const double* image,
                   const float* target, double* dloss)
{
    const double inv = 1.0 / (3.0 * (double)W * (double)H);
    const int64_t P = (int64_t)W * H;
    const int32_t x0 = leaf.tx0 * 16, y0 = leaf.ty0 * 16;
    const int32_t x1 = leaf.tx1 * 16 < W ? leaf.tx1 * 16 : W;
    const int32_t y1 = leaf.ty1 * 16 < H ? leaf.ty1 * 16 : H;
    double sum = 0.0;
    for (int ch = 0; ch < 3; ++ch)
        for (int32_t py = y0; py < y1; ++py)
            for (int32_t px = x0; px < x1; ++px) {
                const int64_t k = ch * P + (int64_t)py * W + px;
                const double d = image[k] - (double)target[k];
                sum += fabs(d);
                dloss[k] = (double)((d > 0.0) - (d < 0.0)) * inv;
            }
    return sum * inv;
}

/* SSIM with an 11x11 Gaussian window (sigma 1.5, weights sum to 1),
 * K1 = 0.01, K2 = 0.03 on a [0,1] range, zero padding outside the image,
 * mean over channels and pixels.  SkipGS notes, "loss function": the loss is
 * (1 - lambda) L1 + lambda (1 - SSIM), lambda = 0.2.  Written as direct
 * window sums; the gradient is the chain rule through the five windowed
 * statistics and the adjoint of the zero-padded window sum.              */
double gso_loss_ssim(int32_t W, int32_t H, const double* image, const float* target,
                     double lambda, double* dloss, double* ssim_out)
{
    const int64_t P = (int64_t)W * H;
    const double C1 = 0.01 * 0.01, C2 = 0.03 * 0.03;
    double g1[11], gs = 0.0;
    for (int i = 0; i < 11; ++i) { g1[i] = exp(-((i - 5) * (i - 5)) / (2.0 * 1.5 * 1.5)); gs += g1[i]; }
    for (int i = 0; i < 11; ++i) g1[i] /= gs;

    double* dA = (double*)malloc(sizeof(double) * P);
    double* dB = (double*)malloc(sizeof(double) * P);
    double* dC = (double*)malloc(sizeof(double) * P);
    const double inv = 1.0 / (3.0 * (double)P);
    double ssim_sum = 0.0, l1 = 0.0;
    for (int ch = 0; ch < 3; ++ch) {
        const double* X = image + ch * P;
        const float* Yt = target + ch * P;
        for (int32_t py = 0; py < H; ++py)
            for (int32_t px = 0; px < W; ++px) {
                double mx = 0, my = 0, exx = 0, eyy = 0, exy = 0;
                for (int a = 0; a < 11; ++a) {
                    const int32_t qy = py + a - 5;
                    if (qy < 0 || qy >= H) continue;
                    for (int b = 0; b < 11; ++b) {
                        const int32_t qx = px + b - 5;
                        if (qx < 0 || qx >= W) continue;
                        const double wgt = g1[a] * g1[b];
                        const double xv = X[(int64_t)qy * W + qx], yv = (double)Yt[(int64_t)qy * W + qx];
                        mx += wgt * xv; my += wgt * yv;
                        exx += wgt * xv * xv; eyy += wgt * yv * yv; exy += wgt * xv * yv;
                    }
                }
                const double sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
                const double N1 = 2 * mx * my + C1, N2 = 2 * sxy + C2;
                const double D1 = mx * mx + my * my + C1, D2 = sxx + syy + C2;
                const double S = (N1 * N2) / (D1 * D2);
                ssim_sum += S;
                /* partials of S in the window statistics */
                const double dS_dmx = (2 * my * N2) / (D1 * D2) - S * (2 * mx) / D1;
                const double dS_dsxx = -S / D2;
                const double dS_dsxy = 2 * N1 / (D1 * D2);
                const int64_t k = (int64_t)py * W + px;
                dA[k] = dS_dmx + dS_dsxx * (-2 * mx) + dS_dsxy * (-my);  /* per unit mean_x   */
                dB[k] = dS_dsxx;                                          /* per unit E[x^2]   */
                dC[k] = dS_dsxy;                                          /* per unit E[xy]    */
            }
        for (int32_t qy = 0; qy < H; ++qy)
            for (int32_t qx = 0; qx < W; ++qx) {
                double sa = 0, sb = 0, sc = 0;
                for (int a = 0; a < 11; ++a) {
                    const int32_t py = qy - (a - 5);
                    if (py < 0 || py >= H) continue;
                    for (int b = 0; b < 11; ++b) {
                        const int32_t px = qx - (b - 5);
                        if (px < 0 || px >= W) continue;
                        const double wgt = g1[a] * g1[b];
                        const int64_t k = (int64_t)py * W + px;
                        sa += wgt * dA[k]; sb += wgt * dB[k]; sc += wgt * dC[k];
                    }
                }
                const int64_t k = (int64_t)qy * W + qx;
                const double xv = X[k], yv = (double)Yt[k];
                const double dssim = sa + 2 * xv * sb + yv * sc;       /* d(sum S)/dx */
                const double d = xv - yv;
                l1 += fabs(d);
                dloss[ch * P + k] = (1.0 - lambda) * (double)((d > 0) - (d < 0)) * inv
                                    - lambda * dssim * inv;
            }
    }
    free(dA); free(dB); free(dC);
    const double ssim = ssim_sum * inv;
    if (ssim_out) *ssim_out = ssim;
    return (1.0 - lambda) * l1 * inv + lambda * (1.0 - ssim);
}

/* ---------------------------------------------------------------------- */
/* Raster backward (f64 values along given decisions).  BoundedGS page, Fig. 3
 * A->B: the rasterization backward runs first and collects the gradients of
 * the projected attributes; SkipGS notes, "loss function": the gradient runs
 * through the transmittance chain.  For a pixel with included entries
 * i = 0..m-1 (front to back), T_i = prod_{k<i} (1 - alpha_k), and
 *   C = sum_i c_i alpha_i T_i + T_m bg,
 *   dC/dalpha_i = c_i T_i - S_i / (1 - alpha_i),
 *   S_i = sum_{k>i} c_k alpha_k T_k + T_m bg.
 * alpha_i = opacity_i * exp(power_i) unless clamped (then constant 0.99).  */
typedef struct { double T, alpha, G, dx, dy; } bwd_tmp;

static uint64_t fnv_mix(uint64_t h, uint64_t v)
{
    for (int b = 0; b < 8; ++b) { h ^= (v >> (8 * b)) & 0xFFu; h *= 1099511628211ull; }
    return h;
}

static void bwd_pixel(double pxc, double pyc, const gso_rec* rec, int64_t nrec,
                      const double* xy, const double* conic, const double* opac,
                      const double* rgb, const double bg[3], const double g[3],
                      double* grad2d, bwd_tmp* tmp)
{
    double T = 1.0;
    for (int64_t i = 0; i < nrec; ++i) {
        const int64_t j = rec[i].slot;
        const double A = conic[3 * j], B = conic[3 * j + 1], C = conic[3 * j + 2];
        const double dx = pxc - xy[2 * j], dy = pyc - xy[2 * j + 1];
        const double power = -0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy;
        const double G = exp(power);
        const double alpha = rec[i].clamped ? 0.99 : opac[j] * G;
        tmp[i].T = T; tmp[i].alpha = alpha; tmp[i].G = G; tmp[i].dx = dx; tmp[i].dy = dy;
        T *= (1.0 - alpha);
    }
    double S[3] = {T * bg[0], T * bg[1], T * bg[2]};
    for (int64_t i = nrec - 1; i >= 0; --i) {
        const int64_t j = rec[i].slot;
        const double Ti = tmp[i].T, al = tmp[i].alpha, wgt = al * Ti;
        double* gj = grad2d + 9 * j;
        double dal = 0.0;
        for (int ch = 0; ch < 3; ++ch) {
            const double c = rgb[3 * j + ch];
            gj[6 + ch] += g[ch] * wgt;
            dal += g[ch] * (c * Ti - S[ch] / (1.0 - al));
            S[ch] += c * wgt;
        }
        if (!rec[i].clamped) {
            const double A = conic[3 * j], B = conic[3 * j + 1], C = conic[3 * j + 2];
            const double dx = tmp[i].dx, dy = tmp[i].dy, G = tmp[i].G;
            const double dpow = dal * opac[j] * G;
            gj[5] += dal * G;
            gj[2] += -0.5 * dx * dx * dpow;
            gj[3] += -dx * dy * dpow;
            gj[4] += -0.5 * dy * dy * dpow;
            gj[0] += (A * dx + B * dy) * dpow;
            gj[1] += (C * dy + B * dx) * dpow;
        }
    }
}

static void render_bwd_common(int dec32, const gso_camera* cam, gso_rect leaf,
                              const uint64_t* offsets, const uint32_t* values,
                              const float* xy32, const float* conic32, const float* opacity32,
                              const double* xy, const double* conic, const double* opacity,
                              const double* rgb, const double* dloss, double* grad2d,
                              int64_t* q_bwd, uint64_t* signature)
{
    const int32_t W = cam->width, H = cam->height;
    const int32_t TWL = leaf.tx1 - leaf.tx0;
    const int64_t P = (int64_t)W * H;
    const double bg[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
    const float bg32[3] = {cam->bg[0], cam->bg[1], cam->bg[2]};
    int64_t maxlen = 1;
    for (int64_t t = 0; t < (int64_t)TWL * (leaf.ty1 - leaf.ty0); ++t) {
        const int64_t len = (int64_t)(offsets[t + 1] - offsets[t]);
        if (len > maxlen) maxlen = len;
    }
    gso_rec* rec = (gso_rec*)malloc(sizeof(gso_rec) * maxlen);
    bwd_tmp* tmp = (bwd_tmp*)malloc(sizeof(bwd_tmp) * maxlen);
    uint64_t h = signature ? *signature : 1469598103934665603ull;
    int64_t qb = 0, ev = 0;
    for (int32_t ty = leaf.ty0; ty < leaf.ty1; ++ty)
        for (int32_t tx = leaf.tx0; tx < leaf.tx1; ++tx) {
            const int64_t lt = (int64_t)(ty - leaf.ty0) * TWL + (tx - leaf.tx0);
            const uint32_t* list = values + offsets[lt];
            const int64_t len = (int64_t)(offsets[lt + 1] - offsets[lt]);
            for (int32_t py = ty * 16; py < ty * 16 + 16 && py < H; ++py)
                for (int32_t px = tx * 16; px < tx * 16 + 16 && px < W; ++px) {
                    int64_t nrec;
                    int32_t ls;
                    if (dec32) {
                        float out[3], tf;
                        nrec = fwd_pixel_f32((float)px + 0.5f, (float)py + 0.5f, list, len, xy32,
                                             conic32, opacity32, NULL, bg32, out, &tf, &ls, &ev, rec);
                    } else {
                        double out[3], tf;
                        nrec = fwd_pixel_f64((double)px + 0.5, (double)py + 0.5, list, len, xy,
                                             conic, opacity, NULL, bg, out, &tf, &ls, &ev, rec);
                    }
                    qb += ls;
                    const int64_t pi = (int64_t)py * W + px;
                    const double g[3] = {dloss[pi], dloss[P + pi], dloss[2 * P + pi]};
                    bwd_pixel((double)px + 0.5, (double)py + 0.5, rec, nrec, xy, conic, opacity, rgb,
                              bg, g, grad2d, tmp);
                    if (signature) {
                        h = fnv_mix(h, (uint64_t)pi);
                        for (int64_t i = 0; i < nrec; ++i)
                            h = fnv_mix(h, ((uint64_t)rec[i].slot << 1) | (uint64_t)rec[i].clamped);
                    }
                }
        }
    free(rec);
    free(tmp);
    if (q_bwd) *q_bwd = qb;
    if (signature) *signature = h;
}

void gso_render_bwd_f32dec(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                           const uint32_t* values,
                           const float* xy32, const float* conic32, const float* opacity32,
                           const double* xy, const double* conic, const double* opacity,
                           const double* rgb, const double* dloss, double* grad2d,
                           int64_t* q_bwd, uint64_t* signature)
{
    render_bwd_common(1, cam, leaf, offsets, values, xy32, conic32, opacity32, xy, conic, opacity,
                      rgb, dloss, grad2d, q_bwd, signature);
}

void gso_render_bwd_f64dec(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                           const uint32_t* values,
                           const double* xy, const double* conic, const double* opacity,
                           const double* rgb, const double* dloss, double* grad2d,
                           int64_t* q_bwd, uint64_t* signature)
{
    render_bwd_common(0, cam, leaf, offsets, values, NULL, NULL, NULL, xy, conic, opacity, rgb,
                      dloss, grad2d, q_bwd, signature);
}

/* ---------------------------------------------------------------------- */
/* Projection backward (f64).  BoundedGS page, Fig. 3 A->B and C->D->E: runs
 * once per view after all leaves, from the collected 2D gradients, into
 * state kept only for candidates.  SkipGS notes, "loss function": gradients
 * reach the means, quaternions, scales, opacities and SH coefficients.
 * Scalar chain rule through each assignment of the projection, with the
 * clamp decisions of the forward projection.                              */
static void sh_grad_dir(int deg, double x, double y, double z, double* D /*[16][3]*/)
{
    const double c1 = 0.488602511902919921, c2a = 1.09254843059207907, c2b = 0.315391565252520050,
                 c2c = 0.546274215296039535, c3a = 0.590043589926643510, c3b = 2.89061144264055405,
                 c3c = 0.457045799464465739, c3d = 0.373176332590115391, c3e = 1.44530572132027703;
    for (int k = 0; k < 48; ++k) D[k] = 0.0;
    if (deg < 1) return;
    D[3 * 1 + 1] = c1;
    D[3 * 2 + 2] = c1;
    D[3 * 3 + 0] = c1;
    if (deg < 2) return;
    const double xx = x * x, yy = y * y, zz = z * z;
    D[3 * 4 + 0] = c2a * y;       D[3 * 4 + 1] = c2a * x;
    D[3 * 5 + 1] = c2a * z;       D[3 * 5 + 2] = c2a * y;
    D[3 * 6 + 0] = -2 * c2b * x;  D[3 * 6 + 1] = -2 * c2b * y;  D[3 * 6 + 2] = 4 * c2b * z;
    D[3 * 7 + 0] = c2a * z;       D[3 * 7 + 2] = c2a * x;
    D[3 * 8 + 0] = 2 * c2c * x;   D[3 * 8 + 1] = -2 * c2c * y;
    if (deg < 3) return;
    D[3 * 9 + 0] = c3a * 6 * x * y;             D[3 * 9 + 1] = c3a * (3 * xx - 3 * yy);
    D[3 * 10 + 0] = c3b * y * z;                D[3 * 10 + 1] = c3b * x * z;   D[3 * 10 + 2] = c3b * x * y;
    D[3 * 11 + 0] = c3c * (-2 * x * y);         D[3 * 11 + 1] = c3c * (4 * zz - xx - 3 * yy);
    D[3 * 11 + 2] = c3c * 8 * y * z;
    D[3 * 12 + 0] = c3d * (-6 * x * z);         D[3 * 12 + 1] = c3d * (-6 * y * z);
    D[3 * 12 + 2] = c3d * (6 * zz - 3 * xx - 3 * yy);
    D[3 * 13 + 0] = c3c * (4 * zz - 3 * xx - yy); D[3 * 13 + 1] = c3c * (-2 * x * y);
    D[3 * 13 + 2] = c3c * 8 * x * z;
    D[3 * 14 + 0] = c3e * 2 * x * z;            D[3 * 14 + 1] = c3e * (-2 * y * z);
    D[3 * 14 + 2] = c3e * (xx - yy);
    D[3 * 15 + 0] = c3a * (3 * xx - 3 * yy);    D[3 * 15 + 1] = c3a * (-6 * x * y);
}

void gso_project_bwd(const gso_camera* cam, int64_t n, int deg,
                     const double* means, const double* log_scales, const double* quats,
                     const double* logits, const double* sh,
                     const uint8_t* cand, const uint32_t* flags, const int64_t* slot_of,
                     const double* grad2d, double* grad3d)
{
    const int K = (deg + 1) * (deg + 1);
    const int F = 11 + 3 * K;
    double Rc[9], tc[3], cc[3];
    for (int k = 0; k < 9; ++k) Rc[k] = cam->R[k];
    for (int k = 0; k < 3; ++k) tc[k] = cam->t[k];
    for (int k = 0; k < 3; ++k) cc[k] = -(Rc[k] * tc[0] + Rc[3 + k] * tc[1] + Rc[6 + k] * tc[2]);
    const double fx = cam->fx, fy = cam->fy;
    const double limx = 1.3 * (0.5 * cam->width / fx), limy = 1.3 * (0.5 * cam->height / fy);

    for (int64_t i = 0; i < n; ++i) {
        double* out = grad3d + (int64_t)F * i;
        for (int k = 0; k < F; ++k) out[k] = 0.0;
        if (!cand[i]) continue;
        const double* g = grad2d + 9 * slot_of[i];
        const uint32_t fl = flags[i];
        /* ---- forward recomputation ---- */
        const double mu[3] = {means[3 * i], means[3 * i + 1], means[3 * i + 2]};
        double p[3];
        for (int r = 0; r < 3; ++r) p[r] = Rc[3 * r] * mu[0] + Rc[3 * r + 1] * mu[1] + Rc[3 * r + 2] * mu[2] + tc[r];
        const double px = p[0], py = p[1], pz = p[2];
        double s[3];
        for (int k = 0; k < 3; ++k) s[k] = exp(log_scales[3 * i + k]);
        const double* q = quats + 4 * i;
        const double qn = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
        const double w = q[0] / qn, x = q[1] / qn, y = q[2] / qn, z = q[3] / qn;
        double Rq[3][3];
        Rq[0][0] = 1 - 2 * (y * y + z * z); Rq[0][1] = 2 * (x * y - w * z); Rq[0][2] = 2 * (x * z + w * y);
        Rq[1][0] = 2 * (x * y + w * z); Rq[1][1] = 1 - 2 * (x * x + z * z); Rq[1][2] = 2 * (y * z - w * x);
        Rq[2][0] = 2 * (x * z - w * y); Rq[2][1] = 2 * (y * z + w * x); Rq[2][2] = 1 - 2 * (x * x + y * y);
        double M[3][3], Sg[3][3];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) M[r][c] = Rq[r][c] * s[c];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) Sg[r][c] = M[r][0] * M[c][0] + M[r][1] * M[c][1] + M[r][2] * M[c][2];
        const double u = px / pz, v = py / pz;
        const int clx = (fl & GSO_FLAG_CLAMP_UX) != 0, cly = (fl & GSO_FLAG_CLAMP_UY) != 0;
        const double ux = clx ? (u < 0 ? -limx : limx) : u;
        const double uy = cly ? (v < 0 ? -limy : limy) : v;
        const double J00 = fx / pz, J02 = -fx * ux / pz, J11 = fy / pz, J12 = -fy * uy / pz;
        double T[2][3], U[2][3];
        for (int c = 0; c < 3; ++c) {
            T[0][c] = J00 * Rc[c] + J02 * Rc[6 + c];
            T[1][c] = J11 * Rc[3 + c] + J12 * Rc[6 + c];
        }
        for (int a = 0; a < 2; ++a)
            for (int c = 0; c < 3; ++c) U[a][c] = T[a][0] * Sg[0][c] + T[a][1] * Sg[1][c] + T[a][2] * Sg[2][c];
        const double a = U[0][0] * T[0][0] + U[0][1] * T[0][1] + U[0][2] * T[0][2] + 0.3;
        const double b = U[0][0] * T[1][0] + U[0][1] * T[1][1] + U[0][2] * T[1][2];
        const double c = U[1][0] * T[1][0] + U[1][1] * T[1][1] + U[1][2] * T[1][2] + 0.3;
        const double det = a * c - b * b;
        const double o = 1.0 / (1.0 + exp(-logits[i]));
        const double vdir[3] = {mu[0] - cc[0], mu[1] - cc[1], mu[2] - cc[2]};
        const double vn = sqrt(vdir[0] * vdir[0] + vdir[1] * vdir[1] + vdir[2] * vdir[2]);
        const double d[3] = {vdir[0] / vn, vdir[1] / vn, vdir[2] / vn};
        double Y[16];
        sh_eval_f64(deg, d[0], d[1], d[2], Y);

        /* ---- chain rule ---- */
        const double dxm = g[0], dym = g[1], dA = g[2], dB = g[3], dC = g[4], dop = g[5];
        double dp[3] = {0, 0, 0};
        /* mean2d = (fx u + cx, fy v + cy), u = px/pz, v = py/pz */
        const double du = fx * dxm, dv = fy * dym;
        dp[0] += du / pz;
        dp[1] += dv / pz;
        dp[2] += -(du * u + dv * v) / pz;
        /* conic = (c, -b, a)/det */
        const double det2 = det * det;
        const double da = (-c * c * dA + b * c * dB - b * b * dC) / det2;
        const double db = (2 * b * c * dA - (a * c + b * b) * dB + 2 * a * b * dC) / det2;
        const double dc = (-b * b * dA + a * b * dB - a * a * dC) / det2;
        const double dS2[2][2] = {{da, db}, {0.0, dc}};   /* entries (0,0), (0,1), (1,1) are used */
        double dU[2][3] = {{0}}, dT[2][3] = {{0}}, dSg[3][3] = {{0}};
        for (int aa = 0; aa < 2; ++aa)
            for (int bb = 0; bb < 2; ++bb)
                for (int k = 0; k < 3; ++k) {
                    dU[aa][k] += dS2[aa][bb] * T[bb][k];
                    dT[bb][k] += dS2[aa][bb] * U[aa][k];
                }
        for (int aa = 0; aa < 2; ++aa)
            for (int k = 0; k < 3; ++k)
                for (int cidx = 0; cidx < 3; ++cidx) {
                    dSg[k][cidx] += T[aa][k] * dU[aa][cidx];
                    dT[aa][k] += dU[aa][cidx] * Sg[k][cidx];
                }
        double dJ00 = 0, dJ02 = 0, dJ11 = 0, dJ12 = 0;
        for (int k = 0; k < 3; ++k) {
            dJ00 += dT[0][k] * Rc[k];
            dJ02 += dT[0][k] * Rc[6 + k];
            dJ11 += dT[1][k] * Rc[3 + k];
            dJ12 += dT[1][k] * Rc[6 + k];
        }
        dp[2] += -fx / (pz * pz) * dJ00 + fx * ux / (pz * pz) * dJ02 - fy / (pz * pz) * dJ11
                 + fy * uy / (pz * pz) * dJ12;
        const double dux = -fx / pz * dJ02, duy = -fy / pz * dJ12;
        if (!clx) { dp[0] += dux / pz; dp[2] += -dux * u / pz; }
        if (!cly) { dp[1] += duy / pz; dp[2] += -duy * v / pz; }
        /* Sigma = M M^T */
        double dM[3][3];
        for (int r = 0; r < 3; ++r)
            for (int cidx = 0; cidx < 3; ++cidx) {
                double acc = 0.0;
                for (int k = 0; k < 3; ++k) acc += (dSg[r][k] + dSg[k][r]) * M[k][cidx];
                dM[r][cidx] = acc;
            }
        double dRq[3][3], ds[3] = {0, 0, 0};
        for (int r = 0; r < 3; ++r)
            for (int cidx = 0; cidx < 3; ++cidx) {
                dRq[r][cidx] = dM[r][cidx] * s[cidx];
                ds[cidx] += dM[r][cidx] * Rq[r][cidx];
            }
        for (int k = 0; k < 3; ++k) out[3 + k] = ds[k] * s[k];
        /* rotation matrix of the unit quaternion (w, x, y, z) */
        double dw = 0, dx = 0, dy = 0, dz = 0;
        dy += -4 * y * dRq[0][0]; dz += -4 * z * dRq[0][0];
        dx += 2 * y * dRq[0][1]; dy += 2 * x * dRq[0][1]; dw += -2 * z * dRq[0][1]; dz += -2 * w * dRq[0][1];
        dx += 2 * z * dRq[0][2]; dz += 2 * x * dRq[0][2]; dw += 2 * y * dRq[0][2]; dy += 2 * w * dRq[0][2];
        dx += 2 * y * dRq[1][0]; dy += 2 * x * dRq[1][0]; dw += 2 * z * dRq[1][0]; dz += 2 * w * dRq[1][0];
        dx += -4 * x * dRq[1][1]; dz += -4 * z * dRq[1][1];
        dy += 2 * z * dRq[1][2]; dz += 2 * y * dRq[1][2]; dw += -2 * x * dRq[1][2]; dx += -2 * w * dRq[1][2];
        dx += 2 * z * dRq[2][0]; dz += 2 * x * dRq[2][0]; dw += -2 * y * dRq[2][0]; dy += -2 * w * dRq[2][0];
        dy += 2 * z * dRq[2][1]; dz += 2 * y * dRq[2][1]; dw += 2 * x * dRq[2][1]; dx += 2 * w * dRq[2][1];
        dx += -4 * x * dRq[2][2]; dy += -4 * y * dRq[2][2];
        const double dot = w * dw + x * dx + y * dy + z * dz;
        out[6] = (dw - w * dot) / qn;
        out[7] = (dx - x * dot) / qn;
        out[8] = (dy - y * dot) / qn;
        out[9] = (dz - z * dot) / qn;
        out[10] = dop * o * (1.0 - o);
        /* colour from SH along the view direction */
        double Dy[48];
        sh_grad_dir(deg, d[0], d[1], d[2], Dy);
        double dd[3] = {0, 0, 0};
        const double* shi = sh + (int64_t)3 * K * i;
        for (int ch = 0; ch < 3; ++ch) {
            if (fl & (GSO_FLAG_CLAMP_R << ch)) continue;
            const double gr = g[6 + ch];
            for (int k = 0; k < K; ++k) {
                out[11 + 3 * k + ch] = Y[k] * gr;
                for (int e = 0; e < 3; ++e) dd[e] += shi[3 * k + ch] * gr * Dy[3 * k + e];
            }
        }
        const double ddot = d[0] * dd[0] + d[1] * dd[1] + d[2] * dd[2];
        double dmu[3];
        for (int e = 0; e < 3; ++e) dmu[e] = (dd[e] - d[e] * ddot) / vn;
        /* p = R mu + t */
        for (int e = 0; e < 3; ++e) dmu[e] += Rc[e] * dp[0] + Rc[3 + e] * dp[1] + Rc[6 + e] * dp[2];
        out[0] = dmu[0]; out[1] = dmu[1]; out[2] = dmu[2];
    }
}

/* ---------------------------------------------------------------------- */
/* Leaf planner (integer).  BoundedGS page, "01": regions are split by their
 * actual load, estimated from overlap counts, pixels and buffer layout, so
 * that dense regions become smaller; Fig. 3 B->C: regions over the budget
 * are subdivided further.  Reading: load estimate
 *   est = bI * I + bC * Cb + bP * P + bT * T + b0
 * (I = Gaussian-tile overlaps in the region, Cb = pairs (candidate,
 * super-cell) over the image-aligned 8x8-tile super-cells the region meets,
 * where a candidate meets a super-cell when its tile rectangle does,
 * P = the region's pixels inside the image, T = its tiles); a region is kept
 * when est <= budget or it is one tile, otherwise its longer side (in tiles,
 * ties -> x) is halved at floor(len/2) and the halves are planned in order. */
uint64_t gso_leaf_estimate(int32_t W, int32_t H, gso_rect r, uint64_t n_isect, uint64_t n_cells,
                           const gso_cost* cost)
{
    const int64_t x1 = (int64_t)r.tx1 * 16 < W ? (int64_t)r.tx1 * 16 : W;
    const int64_t y1 = (int64_t)r.ty1 * 16 < H ? (int64_t)r.ty1 * 16 : H;
    const uint64_t P = (uint64_t)(x1 - (int64_t)r.tx0 * 16) * (uint64_t)(y1 - (int64_t)r.ty0 * 16);
    const uint64_t T = (uint64_t)(r.tx1 - r.tx0) * (uint64_t)(r.ty1 - r.ty0);
    return cost->b_isect * n_isect + cost->b_cell * n_cells + cost->b_pixel * P + cost->b_tile * T +
           cost->b_const;
}

typedef struct {
    int32_t W, H, TW, SW;
    const uint64_t* sat;    /* (TH+1) x (TW+1), tile counts */
    const uint64_t* sat8;   /* (SH+1) x (SW+1), super-cell counts */
    uint64_t budget;
    const gso_cost* cost;
    gso_leaf* out;
    int32_t max_leaves, count;
} plan_ctx;

static uint64_t rect_sum(const uint64_t* sat, int64_t S, int32_t x0, int32_t y0, int32_t x1, int32_t y1)
{
    return sat[(int64_t)y1 * S + x1] - sat[(int64_t)y0 * S + x1] - sat[(int64_t)y1 * S + x0] +
           sat[(int64_t)y0 * S + x0];
}

static void plan_rec(plan_ctx* pc, gso_rect r)
{
    const uint64_t I = rect_sum(pc->sat, pc->TW + 1, r.tx0, r.ty0, r.tx1, r.ty1);
    const uint64_t Cb = rect_sum(pc->sat8, pc->SW + 1, r.tx0 / 8, r.ty0 / 8, (r.tx1 - 1) / 8 + 1,
                                 (r.ty1 - 1) / 8 + 1);
    const uint64_t est = gso_leaf_estimate(pc->W, pc->H, r, I, Cb, pc->cost);
    const int32_t w = r.tx1 - r.tx0, h = r.ty1 - r.ty0;
    if (est <= pc->budget || (w == 1 && h == 1)) {
        if (pc->count < pc->max_leaves) {
            gso_leaf* L = pc->out + pc->count;
            L->tx0 = r.tx0; L->ty0 = r.ty0; L->tx1 = r.tx1; L->ty1 = r.ty1;
            L->est_bytes = est;
            L->over_budget = est > pc->budget;
            L->pad = 0;
        }
        pc->count += 1;
        return;
    }
    gso_rect a = r, b = r;
    if (w >= h) { a.tx1 = r.tx0 + w / 2; b.tx0 = a.tx1; }
    else        { a.ty1 = r.ty0 + h / 2; b.ty0 = a.ty1; }
    plan_rec(pc, a);
    plan_rec(pc, b);
}

/* summed-area table (rows+1) x (cols+1) of a count grid rows x cols */
static void make_sat(const uint64_t* cnt, int32_t rows, int32_t cols, uint64_t* sat)
{
    const int64_t S = cols + 1;
    for (int64_t k = 0; k < S * (rows + 1); ++k) sat[k] = 0;
    for (int32_t y = 0; y < rows; ++y)
        for (int32_t x = 0; x < cols; ++x)
            sat[(int64_t)(y + 1) * S + x + 1] = cnt[(int64_t)y * cols + x] + sat[(int64_t)y * S + x + 1]
                                                + sat[(int64_t)(y + 1) * S + x] - sat[(int64_t)y * S + x];
}

int32_t gso_plan_leaves(int32_t W, int32_t H, int64_t n_cand, const int32_t* rect,
                        uint64_t budget, const gso_cost* cost, gso_leaf* out,
                        int32_t max_leaves, uint64_t* sat_out)
{
    return gso_replan_leaves(W, H, n_cand, rect, budget, cost, NULL, 0, out, max_leaves, sat_out);
}

/* The re-check of a cached layout before it is executed (BoundedGS "02 /
 * method": the region plan is checked against the current load before a
 * view runs).  Reading: each cached leaf, in the given order, is kept when
 * its estimate under the current candidates is within the budget and is
 * otherwise split by the same rule as a fresh plan; leaves are never merged.
 * roots = NULL: the whole tile grid, i.e. a fresh plan. */
int32_t gso_replan_leaves(int32_t W, int32_t H, int64_t n_cand, const int32_t* rect,
                          uint64_t budget, const gso_cost* cost, const gso_rect* roots,
                          int32_t n_roots, gso_leaf* out, int32_t max_leaves, uint64_t* sat_out)
{
    const int32_t TW = (W + 15) / 16, TH = (H + 15) / 16;
    const int32_t SW = (TW + 7) / 8, SH = (TH + 7) / 8;
    uint64_t* cnt = (uint64_t*)calloc((size_t)TW * TH, sizeof(uint64_t));
    uint64_t* cnt8 = (uint64_t*)calloc((size_t)SW * SH, sizeof(uint64_t));
    uint64_t* sat = sat_out ? sat_out : (uint64_t*)malloc(sizeof(uint64_t) * (TW + 1) * (TH + 1));
    uint64_t* sat8 = (uint64_t*)malloc(sizeof(uint64_t) * (SW + 1) * (SH + 1));
    for (int64_t j = 0; j < n_cand; ++j) {
        const int32_t* r = rect + 4 * j;
        for (int32_t ty = r[1]; ty < r[3]; ++ty)
            for (int32_t tx = r[0]; tx < r[2]; ++tx) cnt[(int64_t)ty * TW + tx] += 1;
        if (r[0] < r[2] && r[1] < r[3])
            for (int32_t sy = r[1] / 8; sy <= (r[3] - 1) / 8; ++sy)
                for (int32_t sx = r[0] / 8; sx <= (r[2] - 1) / 8; ++sx) cnt8[(int64_t)sy * SW + sx] += 1;
    }
    make_sat(cnt, TH, TW, sat);
    make_sat(cnt8, SH, SW, sat8);
    plan_ctx pc = {W, H, TW, SW, sat, sat8, budget, cost, out, max_leaves, 0};
    if (roots) {
        for (int32_t k = 0; k < n_roots; ++k) plan_rec(&pc, roots[k]);
    } else {
        gso_rect all = {0, 0, TW, TH};
        plan_rec(&pc, all);
    }
    free(cnt);
    free(cnt8);
    free(sat8);
    if (!sat_out) free(sat);
    return pc.count;
}

/* ---------------------------------------------------------------------- */
/* Adam (Kingma & Ba), one step t with bias correction; the pages (SkipGS
 * notes, "loss function") name Adam; BoundedGS "01": one update per view. */
void gso_adam(int64_t n, const double* grad, double* param, double* m, double* v,
              int32_t step, double lr, double beta1, double beta2, double eps)
{
    const double bc1 = 1.0 - pow(beta1, step), bc2 = 1.0 - pow(beta2, step);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = beta1 * m[i] + (1.0 - beta1) * grad[i];
        v[i] = beta2 * v[i] + (1.0 - beta2) * grad[i] * grad[i];
        const double mh = m[i] / bc1, vh = v[i] / bc2;
        param[i] -= lr * mh / (sqrt(vh) + eps);
    }
}
