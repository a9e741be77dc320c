/*
 * gso.h -- CPU oracle for one training view of differentiable tile-based 3D
 * Gaussian splatting with load-budgeted leaf regions (BoundedGS).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, constant or table with the GPU library: both sides are written
 * independently against the same arithmetic specification.
 *
 * What it computes (sources are the pages' own sections):
 *   - BoundedGS project page, "01 / problem and insight" and "02 / method"
 *     (Fig. 3, A->B->C->D->E): one view is rendered leaf by leaf with the
 *     full camera and the global model; each leaf runs rasterize -> loss ->
 *     backward; 2D (projected-attribute) gradients are collected first and
 *     the projection backward runs once afterwards; leaves are split until
 *     their estimated load (overlaps, pixels, buffers) fits a byte budget.
 *   - SkipGS notes, "loss function / training strategy": the loss
 *     (1-lambda)*L1 + lambda*(1-SSIM) with lambda = 0.2, gradients flowing
 *     through the 2D projected covariance and the transmittance chain to the
 *     means, quaternions, scales, opacities and SH coefficients, then Adam.
 * The pages never write the rasterizer's equations.  The standard EWA
 * splatting reading used here, with every constant and the exact f32
 * operation order, is the one the GPU side implements independently.
 *
 * Precision: the pages fix none.  Every floating-point result that decides
 * an integer (candidate set, tile rectangles, depth keys, which Gaussians a
 * pixel includes, where compositing stops, the sign of the L1 residual) is
 * taken in f32, the precision the GPU kernels compute in, with a fixed
 * operation order (functions suffixed _f32).  Everything that does not
 * decide an integer -- losses, all gradients, Adam -- is computed in f64.
 * The _f64 variants run the same steps entirely in f64 (libm exp) and serve
 * to pin the f32 path and for finite differences.
 *
 * Conventions: images are CHW f32 [3][H][W]; pixel (u, v) has centre
 * (u + 0.5, v + 0.5); tiles are 16x16, tile (tx, ty) has global id
 * ty * TW + tx with TW = ceil(W / 16); tile rectangles are half-open.
 * Per-candidate 2D gradient layout (9 values):
 *   d/d(mean2d.x), d/d(mean2d.y), d/dA, d/dB, d/dC, d/d(opacity), d/d(r,g,b)
 * where the conic (A, B, C) enters the exponent as
 *   power = -0.5*(A*dx*dx + C*dy*dy) - B*dx*dy.
 * Per-Gaussian 3D gradient layout (F = 11 + 3K values, K = (deg+1)^2):
 *   mean[3], log_scale[3], quat[4] (w,x,y,z), opacity_logit[1], sh[K][3].
 */
#ifndef GSO_H
#define GSO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    float R[9];          /* world->camera rotation, row-major: p = R*mu + t */
    float t[3];
    float fx, fy, cx, cy;
    float near_z;        /* Gaussians with camera z <= near_z are not candidates */
    float bg[3];         /* background colour */
    int32_t width, height;
} gso_camera;

typedef struct { int32_t tx0, ty0, tx1, ty1; } gso_rect;        /* half-open tiles */

typedef struct {
    int32_t tx0, ty0, tx1, ty1;
    uint64_t est_bytes;
    int32_t over_budget;  /* 1 when a single tile alone exceeds the budget */
    int32_t pad;
} gso_leaf;

typedef struct {          /* leaf load model: bytes = bI*I + bP*P + bT*T + b0 + bC*Cb */
    uint64_t b_isect, b_pixel, b_tile, b_const;
    uint64_t b_cell;      /* per candidate-(8x8-tile super-cell) pair of the region, counted
                             over the image-aligned super-cells the region meets */
} gso_cost;

/* flag bits written by the projection */
#define GSO_FLAG_CLAMP_R  1u
#define GSO_FLAG_CLAMP_G  2u
#define GSO_FLAG_CLAMP_B  4u
#define GSO_FLAG_CLAMP_UX 8u
#define GSO_FLAG_CLAMP_UY 16u

/* exp by Cody-Waite reduction + degree-7 Taylor/Horner (f32, as specified) */
float gso_exp_cw(float x);
void  gso_exp_cw_array(const float* x, float* y, int64_t n);
/* exp of the Gaussian falloff in alpha (f32 pass of the rasterizer): the
 * argument clamped into [-6, 0], one-constant reduction, degree-6 minimax */
float gso_exp_falloff(float x);
void  gso_exp_falloff_array(const float* x, float* y, int64_t n);
/* real orthonormal SH basis (no Condon-Shortley phase), order l then m=-l..l */
void  gso_sh_basis_f32(int deg, const float* dirs, float* Y, int64_t n);
void  gso_sh_basis_f64(int deg, const double* dirs, double* Y, int64_t n);

/* Projection of every Gaussian (dense outputs, index = Gaussian id). */
void gso_project_f32(const gso_camera* cam, int64_t n, int sh_degree,
                     const float* means, const float* log_scales, const float* quats,
                     const float* logits, const float* sh,
                     uint8_t* cand, int32_t* rect, float* xy, float* conic, float* depth,
                     float* radius, float* opacity, float* rgb, uint32_t* flags);
void gso_project_f64(const gso_camera* cam, int64_t n, int sh_degree,
                     const double* means, const double* log_scales, const double* quats,
                     const double* logits, const double* sh,
                     uint8_t* cand, int32_t* rect, double* xy, double* conic, double* depth,
                     double* radius, double* opacity, double* rgb, uint32_t* flags);

/* Binning of the candidates over one tile rectangle.  rect/depth are compact
 * (index = slot).  Returns the number of intersections.  counts [T_L],
 * offsets [T_L+1] (leaf-local row-major tiles) are always written; values
 * and keys (nullable) are written when values != NULL and cap >= result.
 * Sorted by (global tile id, depth, slot); key = (tile << 32) | depth_bits. */
int64_t gso_bin(int32_t tiles_x, gso_rect leaf, int64_t n_cand, const int32_t* rect,
                const double* depth, const uint32_t* depth_bits,
                uint32_t* counts, uint64_t* offsets, uint32_t* values, uint64_t* keys,
                int64_t cap);

/* Forward compositing of the pixels of a leaf.  Compact state by slot;
 * image [3][H][W], t_final [H][W], last [H][W] are full-size, only the leaf's
 * pixels are written.  *q_eval receives the evaluated (pixel, entry) pairs. */
void gso_render_fwd_f32(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                        const uint32_t* values, const float* xy, const float* conic,
                        const float* opacity, const float* rgb,
                        float* image, float* t_final, int32_t* last, int64_t* q_eval);
void gso_render_fwd_f64(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                        const uint32_t* values, const double* xy, const double* conic,
                        const double* opacity, const double* rgb,
                        double* image, double* t_final, int32_t* last, int64_t* q_eval);

/* L1 over the leaf's pixels with the full-image normaliser 1/(3WH).
 * Returns the partial loss; dloss [3][H][W] gets sgn(out - tgt)/(3WH) there. */
double gso_loss_l1(int32_t W, int32_t H, gso_rect leaf, const double* image,
                   const float* target, double* dloss);
/* (1-lambda)*L1 + lambda*(1 - SSIM_11x11) over the full image, and its gradient. */
double gso_loss_ssim(int32_t W, int32_t H, const double* image, const float* target,
                     double lambda, double* dloss, double* ssim_out);

/* Raster backward of a leaf: replays each pixel's forward decisions (taken
 * in f32 from the f32 state, or in f64 from the value state) and walks them
 * in reverse in f64.  grad2d [n_cand][9] is accumulated (+=). */
void gso_render_bwd_f32dec(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                           const uint32_t* values,
                           const float* xy32, const float* conic32, const float* opacity32,
                           const double* xy, const double* conic, const double* opacity,
                           const double* rgb, const double* dloss, double* grad2d,
                           int64_t* q_bwd, uint64_t* signature);
void gso_render_bwd_f64dec(const gso_camera* cam, gso_rect leaf, const uint64_t* offsets,
                           const uint32_t* values,
                           const double* xy, const double* conic, const double* opacity,
                           const double* rgb, const double* dloss, double* grad2d,
                           int64_t* q_bwd, uint64_t* signature);

/* Projection backward in f64 (dense grad3d [n][F], zero for non-candidates).
 * flags/cand are the decisions of the projection the forward used. */
void gso_project_bwd(const gso_camera* cam, int64_t n, int sh_degree,
                     const double* means, const double* log_scales, const double* quats,
                     const double* logits, const double* sh,
                     const uint8_t* cand, const uint32_t* flags, const int64_t* slot_of,
                     const double* grad2d, double* grad3d);

/* Leaf planner: per-tile counts and per-super-cell counts (8x8 tiles,
 * image-aligned) from candidate rects, their summed-area tables, recursive
 * bisection of the longer side until est <= budget or one tile.  Leaves are
 * written in depth-first order; returns their number (entries beyond
 * max_leaves are counted but not written).  sat (nullable) gets the
 * (TH+1) x (TW+1) table of the tile counts. */
int32_t gso_plan_leaves(int32_t W, int32_t H, int64_t n_cand, const int32_t* rect,
                        uint64_t budget, const gso_cost* cost, gso_leaf* out,
                        int32_t max_leaves, uint64_t* sat);
/* The same bisection started from cached leaves (roots, in order) instead of
 * the whole grid: a root within the budget is kept, one over it is split;
 * leaves are never merged.  roots = NULL: a fresh plan. */
int32_t gso_replan_leaves(int32_t W, int32_t H, int64_t n_cand, const int32_t* rect,
                          uint64_t budget, const gso_cost* cost, const gso_rect* roots,
                          int32_t n_roots, gso_leaf* out, int32_t max_leaves, uint64_t* sat_out);
/* est of a region with n_isect overlaps and n_cells candidate-super-cell
 * pairs over the super-cells it meets */
uint64_t gso_leaf_estimate(int32_t W, int32_t H, gso_rect r, uint64_t n_isect, uint64_t n_cells,
                           const gso_cost* cost);

/* Adam, elementwise in f64: m, v, param updated in place. */
void gso_adam(int64_t n, const double* grad, double* param, double* m, double* v,
              int32_t step, double lr, double beta1, double beta2, double eps);

#ifdef __cplusplus
}
#endif
#endif
