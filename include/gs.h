/*
 * gs.h -- C ABI of the MI355X (gfx950) library for one training view of
 * differentiable tile-based 3D Gaussian splatting with load-budgeted leaf
 * regions (BoundedGS).  Library: libgsmi.so.
 *
 * What a view computes (the pages' own sections):
 *   BoundedGS project page, "01 / problem and insight": within one view the
 *     Gaussian parameters are fixed; a local region that has finished its
 *     rasterization, loss and backward merges its gradient contribution and
 *     frees its local buffers before the next region; regions are sized by
 *     their actual load (overlap count, pixels, buffer layout), cover the
 *     whole image with the same camera and global model, and the gradient of
 *     the whole view is summed before a single parameter update.
 *   BoundedGS "02 / method", Fig. 3: A->B runs the rasterization backward
 *     first, collects the gradients of the projected attributes, then runs
 *     the projection backward; B->C splits the image into leaves under a load
 *     budget, subdividing regions over it; C->D->E keeps projected state and
 *     gradients only for candidate Gaussians.  "384 MiB" is the local
 *     rasterization budget, not a process limit.
 *   SkipGS notes, "loss function / training strategy": loss
 *     (1 - lambda) L1 + lambda (1 - SSIM), lambda = 0.2; gradients flow
 *     through the 2D projected covariance and the transmittance chain to the
 *     means, rotations, scales, opacities and SH coefficients; Adam.
 * The pages give no equations for the rasterizer; the library implements the
 * standard EWA-splatting reading with a fixed f32 operation order (one
 * specification, shared in writing with an independent CPU checker).
 *
 * Conventions
 *   - All functions return gs_status; GS_OK = 0.  On error the message is
 *     available from gs_last_error(ctx), every temporary of the failed call
 *     is released, and outputs are left untouched unless stated otherwise.
 *     No C++ exception crosses this boundary.
 *   - "device" pointers are GPU global memory (hipMalloc / torch tensors on
 *     the context's device); "host" pointers are CPU memory.  Caller-owned
 *     device buffers are never freed nor retained by the library.
 *   - Work is enqueued on the context's stream (asynchronous) unless the
 *     function says it synchronises (those returning counts on the host).
 *   - Images are f32 CHW [3][H][W].  Tiles are 16x16 pixels; tile (tx, ty)
 *     has global id ty * TW + tx, TW = ceil(W/16), TH = ceil(H/16).  Pixel
 *     (u, v) has centre (u + 0.5, v + 0.5).
 *   - Parameters (device, f32, row-major): means [N][3], log_scales [N][3],
 *     quats [N][4] (w, x, y, z; normalised inside), opacity_logits [N],
 *     sh [N][K][3] with K = (sh_degree + 1)^2, sh_degree in 0..3.
 *   - Per-candidate 2D gradients grad2d [n_cand][9] (f32):
 *       d/d mean2d.x, d/d mean2d.y, d/dA, d/dB, d/dC, d/d opacity, d/d rgb
 *     where the conic (A, B, C) enters the exponent as
 *       power = -0.5 (A dx^2 + C dy^2) - B dx dy.
 *   - Per-candidate 3D gradients grad3d [n_cand][F] (f32), F = 11 + 3K:
 *       mean[3], log_scale[3], quat[4], opacity_logit[1], sh[K][3].
 *   - One context per host thread; a context is not thread-safe.
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARG = 1,   /* a precondition on the arguments failed          */
    GS_ERR_OOM = 2,           /* the allocator returned NULL                     */
    GS_ERR_DEVICE = 3,        /* a HIP runtime call failed                       */
    GS_ERR_OVERFLOW = 4,      /* a count exceeds the index widths (see below)    */
    GS_ERR_BUDGET = 5,        /* strict planning: a single tile exceeds budget   */
    GS_ERR_STATE = 6          /* a handle belongs to another context / view      */
} gs_status;

typedef struct gs_ctx gs_ctx;
typedef struct gs_proj gs_proj;       /* projected candidate state of one view  */
typedef struct gs_bins gs_bins;       /* sorted per-tile lists of one leaf       */
typedef struct gs_raster gs_raster;   /* per-pixel forward state of one leaf     */

/* Device allocator callbacks.  alloc returns device memory of at least
 * `bytes` usable in stream order on `stream` (NULL on failure); free returns
 * it.  Both are called from the thread that called the gs_* function. */
typedef void* (*gs_alloc_fn)(void* user, size_t bytes, void* stream);
typedef void (*gs_free_fn)(void* user, void* ptr, size_t bytes, void* stream);

typedef struct {
    float R[9];          /* world->camera rotation, row-major: p = R mu + t   */
    float t[3];
    float fx, fy, cx, cy;
    float near_z;        /* camera z <= near_z: not a candidate (0.2 usual)   */
    float bg[3];         /* background colour                                  */
    int32_t width, height;
} gs_camera;

typedef struct {
    int64_t n;           /* number of Gaussians N (>= 0)                       */
    int32_t sh_degree;   /* 0..3                                               */
    int32_t pad;
    const float* means;
    const float* log_scales;
    const float* quats;
    const float* opacity_logits;
    const float* sh;
} gs_params;

typedef struct {         /* mutable parameter (or moment) arrays, same layout */
    float* means;
    float* log_scales;
    float* quats;
    float* opacity_logits;
    float* sh;
} gs_param_ptrs;

typedef struct { int32_t tx0, ty0, tx1, ty1; } gs_tile_rect;   /* half-open tiles */

typedef struct {
    int32_t tx0, ty0, tx1, ty1;   /* half-open tile rectangle                  */
    uint64_t est_bytes;           /* cost-model estimate of its raster buffers */
    int32_t over_budget;          /* 1: a single tile whose estimate > budget  */
    int32_t pad;
} gs_leaf;

/* Leaf load model:
 *   est = b_isect * I + b_cell * Cb + b_pixel * P + b_tile * T + b_const,
 * I = Gaussian-tile overlaps of the leaf, Cb = (candidate, super-cell) pairs
 * over the image-aligned super-cells of 8 x 8 tiles that the leaf meets (a
 * candidate meets a super-cell when its tile rectangle does; an upper bound
 * of the coarse pairs the leaf's binning sorts), P = its pixels inside the
 * image, T = its tiles.  gs_default_cost_model() returns the library's own
 * allocation sizes, which make est an upper bound of the bytes that
 * gs_bin_sort + gs_render_fwd allocate for a planned leaf (L1 loss inline).
 * gs_train_cost_model() bounds what gs_train_view allocates for a planned
 * leaf of an L1 view, whose fused raster walks the leaf's super-tile groups
 * and holds no per-tile lists or per-pixel state: b_isect = b_pixel = 0,
 * b_cell for the coarse sort, b_tile for the group offsets. */
typedef struct { uint64_t b_isect, b_pixel, b_tile, b_const, b_cell; } gs_cost_model;

enum { GS_MEM_PROJ = 0, GS_MEM_RASTER = 1, GS_MEM_GRAD = 2, GS_MEM_LOSS = 3, GS_MEM_SCRATCH = 4,
       GS_MEM_NCAT = 5 };

typedef struct {
    uint64_t live_bytes, peak_bytes;                 /* all categories        */
    uint64_t live_by_cat[GS_MEM_NCAT];
    uint64_t peak_by_cat[GS_MEM_NCAT];               /* per-category peaks    */
    uint64_t n_alloc, n_free;
} gs_mem_stats;

/* ---- context ----------------------------------------------------------- */

/* Create a context bound to the current HIP device and `stream` (a
 * hipStream_t; NULL = the null stream).  alloc/free NULL: stream-ordered
 * hipMallocAsync/hipFreeAsync.  *out receives the context. */
gs_status gs_ctx_create(gs_ctx** out, void* stream, gs_alloc_fn alloc, gs_free_fn free_fn, void* user);
void gs_ctx_destroy(gs_ctx* ctx);
const char* gs_last_error(const gs_ctx* ctx);
gs_status gs_mem_stats_get(const gs_ctx* ctx, gs_mem_stats* out);
gs_status gs_mem_reset_peak(gs_ctx* ctx);
/* Enable (1) / disable (0) per-kernel HIP-event timing on the context stream. */
gs_status gs_set_timing(gs_ctx* ctx, int32_t on);
/* Accumulated timing of kernel `name` since timing was enabled/reset:
 * total milliseconds and number of launches (synchronises). */
gs_status gs_kernel_time(gs_ctx* ctx, const char* name, double* total_ms, int64_t* launches);
gs_status gs_reset_timing(gs_ctx* ctx);
/* Restrict timing to the kernels timed under `name` (NULL: all kernels), so
 * that a measured run carries events around one kernel only. */
gs_status gs_set_timing_only(gs_ctx* ctx, const char* name);
gs_cost_model gs_default_cost_model(void);
gs_cost_model gs_train_cost_model(void);

/* ---- the six calls of one view ----------------------------------------- */

/* Projection + candidate compaction.  BoundedGS page, Fig. 3 C->D->E
 * (candidate-index projection) and the SkipGS notes' gradient chain through
 * the 2D projected covariance.  Per Gaussian: camera transform, culling,
 * EWA 2D covariance + 0.3 px^2 low-pass, conic, radius, tile rectangle,
 * opacity = sigmoid(logit), rgb = SH(view direction) + 0.5 clamped at 0.
 * Candidates (z > near, det > 0, finite, non-empty rectangle) are stored in
 * ascending Gaussian order.  params: device arrays (caller-owned).
 * *out: new handle (free with gs_release).  *n_cand (host): number of
 * candidates.  Synchronises.  Errors: INVALID_ARG (sh_degree, sizes,
 * NULL), OVERFLOW (n >= 2^31), OOM, DEVICE. */
gs_status gs_project(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, gs_proj** out,
                     int64_t* n_cand);

/* A fixed grid layout, the fixed-block baselines of BoundedGS "03 /
 * results" (Fig. 5: blocks 2K pixels wide; Fig. 6: 1 x 1, 2 x 2, 4 x 4):
 * nx x ny blocks of the tiles_x x tiles_y tile grid; block (i, j) spans tiles
 * [floor(i tiles_x / nx), floor((i + 1) tiles_x / nx)) x [floor(j tiles_y /
 * ny), floor((j + 1) tiles_y / ny)) and is written at out[j nx + i] (host,
 * nx * ny entries; est_bytes 0).  Host only, no context.  Errors:
 * GS_ERR_INVALID_ARG unless out != NULL, 1 <= nx <= tiles_x and
 * 1 <= ny <= tiles_y. */
gs_status gs_grid_leaves(int32_t tiles_x, int32_t tiles_y, int32_t nx, int32_t ny, gs_leaf* out);

/* Leaf planning.  BoundedGS page, "01": regions sized by load estimated from
 * overlap counts, pixels and buffer layout; Fig. 3 B->C: regions over the
 * budget are subdivided.  Per-tile overlap counts of all candidates ->
 * summed-area table -> starting from the whole tile grid, a region is kept
 * when its estimate <= budget_bytes or it is a single tile, otherwise its
 * longer side (ties: x) is halved at floor(len/2); leaves are returned in
 * depth-first order (first half first).  The plan (with, for each leaf, the
 * candidates whose rectangle meets it) is attached to `proj`, so that
 * gs_bin_sort of a planned leaf visits only those candidates; a new plan
 * replaces it.  cost: NULL = default.
 * leaves: host array of max_leaves entries; *n_leaves (host) = number of
 * leaves (entries beyond max_leaves are counted, not written; call again
 * with a larger array).  strict != 0: GS_ERR_BUDGET if any single tile
 * exceeds the budget (leaves are still written).  Synchronises. */
gs_status gs_plan_leaves(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, uint64_t budget_bytes,
                         const gs_cost_model* cost, int32_t strict, gs_leaf* leaves, int32_t max_leaves,
                         int32_t* n_leaves);

/* Re-check of a cached leaf layout before it is executed (BoundedGS page,
 * "02 / method": a region plan is checked against the current load before
 * it runs), e.g. the leaves of this view from an earlier round after the
 * model has changed.  cached (host, n_cached >= 1) must tile the tile grid
 * exactly (else GS_ERR_INVALID_ARG).  Each cached leaf, in order, is kept as
 * it is when its estimate under proj's candidates is within budget_bytes and
 * is otherwise split by the halving rule of gs_plan_leaves (depth-first);
 * leaves are never merged.  Output, errors, strict mode and the plan groups
 * attached to proj as for gs_plan_leaves.  Synchronises. */
gs_status gs_replan_leaves(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, uint64_t budget_bytes,
                           const gs_cost_model* cost, int32_t strict, const gs_leaf* cached, int32_t n_cached,
                           gs_leaf* leaves, int32_t max_leaves, int32_t* n_leaves);

/* Binning of one leaf (tile rectangle inside the grid).  BoundedGS page,
 * "01": raster buffers grow with the overlaps of Gaussians and image tiles.
 * One entry per (candidate, tile of its rectangle inside the leaf), sorted by
 * (tile, depth, candidate slot) -- a unique order.  The sort key of an entry
 * is (global tile id << 32) | f32 bits of its depth.  *out: new handle with
 * per-tile offsets [T_L + 1] (u64, leaf-local row-major tiles) and sorted
 * slots [n_isect] (u32).  *n_isect (host).  Synchronises.
 * Errors: INVALID_ARG (leaf outside the grid or empty), OOM, DEVICE. */
gs_status gs_bin_sort(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, gs_tile_rect leaf,
                      gs_bins** out, int64_t* n_isect);

/* Forward compositing of one leaf.  SkipGS notes, "loss function":
 * transmittance accumulation; BoundedGS Fig. 3 A: raster state is kept until
 * the backward.  Per pixel, front to back over its tile's list:
 * alpha = min(0.99, opacity * exp(power)); entries with power > 0 or
 * alpha < 1/255 are skipped; compositing stops before an entry that would
 * take T below 1e-4; out = C + T bg.  Keeps, per pixel, T_final and the
 * end of its walk over the list: the position of the entry before which
 * compositing stopped, else the list length (no entry from there on is
 * included; the backward starts there).
 * target: device full image [3][H][W] or NULL.  With a target the L1 term
 * is fused: sum |out - target| over the leaf is added to *loss_accum
 * (device, one double, may be NULL) and dL/dout = sgn(out - target)/(3WH)
 * is kept in the raster handle for gs_render_bwd.  image_out: device full
 * image [3][H][W] or NULL; the leaf's pixels are written.  stats: device
 * u64 [4] or NULL; when given, [0] the (pixel, entry) pairs examined, [1]
 * the pairs included, [2] the sum over pixels of the end of the walk, [3]
 * the pairs gs_render_bwd revisits (those examined), are added to it
 * (a separately compiled, slightly slower kernel).  *out: new handle.
 * Asynchronous. */
gs_status gs_render_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                        const float* target, double* loss_accum, float* image_out, uint64_t* stats,
                        gs_raster** out);

/* Raster backward of one leaf, accumulated into grad2d.  BoundedGS Fig. 3
 * A->B (rasterization backward collects the projected attributes'
 * gradients); SkipGS notes (backward = gradient propagation with atomic
 * accumulation).  Per pixel, walks its included entries back to front,
 * recovering T, and forms the 9 partials of each entry; the partials of one
 * entry are summed over a wavefront before one atomic add per value.
 * dl_dimage: device full image [3][H][W] of dL/dout, or NULL to use the L1
 * gradient fused by gs_render_fwd (then a target must have been given).
 * grad2d: device [n_cand][9], accumulated (+=); caller zero-fills it once
 * per view.  Asynchronous. */
gs_status gs_render_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                        const gs_raster* raster, const float* dl_dimage, float* grad2d);

/* Projection backward into compact per-candidate gradients.  BoundedGS
 * Fig. 3 A->B (projection backward after the raster backward) and C->D->E
 * (compact gradients); SkipGS notes (gradients through the 2D covariance to
 * means, rotations, scales, opacities, SH).  grad2d: device [n_cand][9];
 * grad3d: device [n_cand][F] (overwritten).  Asynchronous. */
gs_status gs_project_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, const gs_proj* proj,
                         const float* grad2d, float* grad3d);

/* ---- extras ------------------------------------------------------------ */

/* Full-image loss (1 - lambda) L1 + lambda (1 - SSIM) (SkipGS notes, "loss
 * function"); SSIM with an 11x11 Gaussian window (sigma 1.5), K1 = 0.01,
 * K2 = 0.03, zero padding, mean over channels and pixels.  image, target:
 * device [3][H][W]; dl_dimage: device [3][H][W] (overwritten);
 * loss, ssim: host (nullable).  Synchronises when loss or ssim is given. */
gs_status gs_loss_ssim(gs_ctx* ctx, int32_t width, int32_t height, const float* image, const float* target,
                       float lambda, float* dl_dimage, double* loss, double* ssim);

/* gs_loss_ssim that allocates nothing, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments, results and kernels as gs_loss_ssim, with its
 * work buffers (the 9 per-pixel partial maps and the per-workgroup sums) in a
 * static device array of the library instead of allocated ones.  The array
 * (about 78 MiB: GS_SSIM_STATIC_MAX_PIXELS pixels' maps and the sums of the
 * largest grid such an image takes) exists once on each device the library
 * runs on and is held until the process ends; its address is looked up per
 * device when a context is created.  Every call on a device uses that
 * device's array and overwrites it: calls that overlap on one device (two
 * streams, two host threads) race and must not be issued.  Nothing carries
 * over from one call to the next.  Errors: GS_ERR_INVALID_ARG (sizes < 1,
 * NULL image / target / dl_dimage), GS_ERR_OVERFLOW (width x height above
 * GS_SSIM_STATIC_MAX_PIXELS), GS_ERR_DEVICE.  Asynchronous when loss and
 * ssim are both NULL (the gradient only), else synchronises. */
#define GS_SSIM_STATIC_MAX_PIXELS (1 << 21)   /* 2,097,152: a 1920 x 1080 image fits */
gs_status gs_loss_ssim_static(gs_ctx* ctx, int32_t width, int32_t height, const float* image, const float* target,
                              float lambda, float* dl_dimage, double* loss, double* ssim);

/* One Adam step (beta1, beta2, eps, bias correction at `step` >= 1) over all
 * N x F parameters; Gaussians that are not candidates get a zero gradient.
 * BoundedGS page "01": one update per view after the whole view's gradient.
 * params, m, v: device arrays (in/out); grad3d: device [n_cand][F]. */
gs_status gs_adam_step(gs_ctx* ctx, const gs_proj* proj, int64_t n, int32_t sh_degree,
                       const gs_param_ptrs* params, const gs_param_ptrs* m, const gs_param_ptrs* v,
                       const float* grad3d, int32_t step, float lr, float beta1, float beta2, float eps);

/* Release a gs_proj / gs_bins / gs_raster handle (NULL is a no-op).  Its
 * memory returns to the allocator in stream order. */
void gs_release(gs_ctx* ctx, void* handle);

/* ---- inspection (copies into caller-owned device buffers, asynchronous) --- */

enum {
    GS_PROJ_IDS = 0,      /* u32 [n_cand]      Gaussian id of each slot             */
    GS_PROJ_RECT = 1,     /* i32 [n_cand][4]   tx0, ty0, tx1, ty1                   */
    GS_PROJ_XY = 2,       /* f32 [n_cand][2]   mean2d                               */
    GS_PROJ_CONIC = 3,    /* f32 [n_cand][3]   A, B, C                              */
    GS_PROJ_DEPTH = 4,    /* f32 [n_cand]                                           */
    GS_PROJ_RADIUS = 5,   /* f32 [n_cand]                                           */
    GS_PROJ_OPACITY = 6,  /* f32 [n_cand]                                           */
    GS_PROJ_RGB = 7,      /* f32 [n_cand][3]                                        */
    GS_PROJ_FLAGS = 8,    /* u32 [n_cand]  bit0-2 rgb clamped, bit3/4 x/y clamped   */
    GS_PROJ_SLOT_OF = 9,  /* i32 [N]       slot of each Gaussian or -1              */
    GS_BINS_OFFSETS = 20, /* u64 [T_L + 1]                                          */
    GS_BINS_VALUES = 21,  /* u32 [n_isect] sorted slots                             */
    GS_BINS_KEYS = 22,    /* u64 [n_isect] (global tile << 32) | depth bits         */
    GS_RASTER_TFINAL = 30,/* f32 [P_L]  leaf-local row-major pixels                 */
    GS_RASTER_LAST = 31   /* u32 [P_L]                                              */
};
/* Copy field `field` of handle into dst (device, dst_bytes >= its size). */
gs_status gs_export(gs_ctx* ctx, const void* handle, int32_t field, void* dst, size_t dst_bytes);
/* Size in bytes of a field (host). */
gs_status gs_export_size(gs_ctx* ctx, const void* handle, int32_t field, size_t* bytes);

/* The f32 exp of the projection (scales, sigmoid of the opacity logit):
 * Cody-Waite reduction + degree-7 Taylor polynomial, 0 below -87, +inf above
 * 88.7; on n device floats, for bit-exactness checks. */
gs_status gs_util_exp(gs_ctx* ctx, const float* x, float* y, int64_t n);

/* The f32 exp of the Gaussian falloff in the compositing alpha of
 * gs_render_fwd (SkipGS notes, "loss function": transmittance accumulation;
 * alpha = min(0.99, o exp(power))): the argument is clamped into [-6, 0] (below -6,
 * alpha < 1/255 for every opacity, so the entry is skipped whichever value is
 * used), then one-constant Cody-Waite reduction and the degree-7 Taylor
 * polynomial; within 1 ulp of exp on [-6, 0].  On n finite device floats
 * (NaN gives an unspecified value), for bit-exactness checks.  Errors:
 * GS_ERR_INVALID_ARG for n < 0 or null pointers with n > 0. */
gs_status gs_util_exp_falloff(gs_ctx* ctx, const float* x, float* y, int64_t n);

/* ---- SkipGS backward gate ------------------------------------------------ */
/* Host-side state of a sequence of training views (SkipGS notes, "key
 * design" items 1-3; the "worked example" is its test).  Per view v the gate
 * keeps an EMA of v's forward loss.  At step t with view v and loss L:
 *   score = L / (EMA_v + eps), +inf for a view never seen;
 *   a backward is proposed iff score > 1;
 *   EMA_v = beta EMA_v + (1 - beta) L whatever the decision (a view's first
 *   loss starts its EMA);
 *   steps 1..warmup always run their backward and count the proposals of
 *   views that had an EMA; at step warmup + 1 the floor rho_min = rho_lo +
 *   (1 - rho_lo) rho_hat is fixed, rho_hat = proposed / counted (0 if none);
 *   after that a proposed skip is overridden (forced = 1) while
 *   rho_cum = backwards so far / max(t - 1, 1) < rho_min.
 * All arithmetic in double, in that order.  The notes' values: warmup 500,
 * beta 0.95, rho_lo 0.5, eps 1e-8. */
typedef struct gs_gate gs_gate;
typedef struct {
    int32_t backward;   /* 1: run this view's backward and update            */
    int32_t forced;     /* 1: a proposed skip overridden by the floor         */
    double score;       /* L / (EMA + eps), +inf for a first visit            */
    double rho_cum;     /* backwards / max(t - 1, 1) before this step          */
} gs_gate_decision;
typedef struct {
    int64_t steps, backwards, warmup_counted, warmup_proposed;
    int32_t calibrated, pad;
    double rho_min;     /* valid once calibrated                              */
} gs_gate_stats;
/* n_views >= 1, warmup >= 0, 0 <= beta < 1, 0 <= rho_lo <= 1, eps > 0, else
 * GS_ERR_INVALID_ARG; GS_ERR_OOM.  *out owned by the caller
 * (gs_gate_destroy). */
gs_status gs_gate_create(int32_t n_views, int32_t warmup, double beta, double rho_lo, double eps, gs_gate** out);
void gs_gate_destroy(gs_gate* gate);
/* One step of the sequence: view in [0, n_views), loss finite (else
 * GS_ERR_INVALID_ARG, state unchanged). */
gs_status gs_gate_step(gs_gate* gate, int32_t view, double loss, gs_gate_decision* decision);
gs_status gs_gate_get_stats(const gs_gate* gate, gs_gate_stats* stats);

/* ---- one whole view ---------------------------------------------------- */

typedef struct {
    uint64_t budget_bytes;       /* 0: one leaf = the whole tile grid          */
    int32_t loss_kind;           /* 0: L1, 1: (1-l) L1 + l (1 - SSIM)          */
    float ssim_lambda;           /* 0.2 usual                                  */
    int32_t adam_step;           /* 0: no update; >= 1: one Adam step          */
    float lr, beta1, beta2, eps;
    int32_t strict_budget;
    int32_t max_leaves;          /* capacity of leaves_out (may be 0)          */
    gs_leaf* leaves_out;         /* host, nullable                             */
    const gs_cost_model* cost;   /* NULL: default                              */
    float* image_out;            /* device [3][H][W], nullable                 */
    float* grad3d_out;           /* device [N][F] dense (zero for non-         */
                                 /* candidates), nullable                      */
    gs_param_ptrs* params_rw;    /* required when adam_step >= 1 (in/out)      */
    gs_param_ptrs* adam_m;
    gs_param_ptrs* adam_v;
    int64_t adam_chunk;          /* with Adam and no grad3d_out: 0 fuses the   */
                                 /* projection backward with the update (no    */
                                 /* gradient array); > 0 runs them as two      */
                                 /* kernels per chunk of that many candidate   */
                                 /* slots (gradient buffer adam_chunk x F)     */
    const gs_leaf* leaves_in;    /* host, nullable: a layout to use instead of */
    int32_t n_leaves_in;         /* planning afresh.  budget_bytes > 0: it is  */
                                 /* re-checked as by gs_replan_leaves (e.g.    */
                                 /* this view's leaves_out of an earlier       */
                                 /* round); budget_bytes = 0: it is rendered   */
                                 /* as given (e.g. a gs_grid_leaves layout)    */
    int32_t leaves_in_partial;   /* 1: leaves_in need not cover the grid (no   */
                                 /* overlaps): only those leaves are rendered, */
                                 /* loss and gradients are those of their      */
                                 /* pixels (normaliser still 1/(3WH)); L1 only */
    gs_gate* gate;               /* nullable: SkipGS gate of the sequence; the */
    int32_t gate_view;           /* view's forward loss over all leaves goes   */
                                 /* to gs_gate_step(gate, gate_view, loss) and */
                                 /* the backward, projection backward and      */
                                 /* update run only when it says so            */
    int32_t serial_leaves;       /* 1: render one leaf at a time; 0: a planned */
                                 /* leaf's fused raster may start while the    */
                                 /* previous one ends (two leaves' slot arrays */
                                 /* held at once)                              */
    int32_t target_host;         /* 1: target is host memory [3][H][W] (page-  */
                                 /* locked, e.g. hipHostMalloc, for the copies */
                                 /* to overlap the rendering): each leaf's     */
                                 /* pixels (with the SSIM halo) are copied to  */
                                 /* a device slice before that leaf is         */
                                 /* rendered, so the image is never resident   */
                                 /* whole; 0: target is device memory          */
    uint64_t* leaf_bytes_out;    /* host, nullable, max_leaves entries: per    */
                                 /* leaf (same order as leaves_out) the high-  */
                                 /* water mark of the library bytes that leaf  */
                                 /* held: its binning buffers, slot array,     */
                                 /* target slice and SSIM buffers; to compare  */
                                 /* with its est_bytes (BoundedGS "02 /        */
                                 /* method": the budget bounds each local      */
                                 /* raster's buffers)                          */
    double* loss_out;            /* device, nullable: the view's loss is       */
                                 /* written there, stream-ordered, instead of  */
                                 /* being read back, so the call returns with  */
                                 /* the view's last kernels still queued (a    */
                                 /* training loop reads its losses when it     */
                                 /* needs them); result->loss is then NaN.     */
                                 /* Same bits as the read-back value.  Not     */
                                 /* with a gate, whose decision needs the loss */
                                 /* on the host: GS_ERR_INVALID_ARG            */
} gs_view_opts;

typedef struct {
    double loss;
    int64_t n_cand, n_isect;     /* n_isect summed over leaves                 */
    int32_t n_leaves;
    int32_t groups_walked;       /* 1: the L1 rasters walked the super-tile    */
                                 /* groups (coverage rule), 0: per-tile lists  */
    uint64_t peak_bytes;         /* library high-water mark during the view    */
                                 /* (a device-resident target not included)    */
    int32_t gate_backward;       /* with a gate: the decision (else 0)         */
    int32_t gate_forced;
    double gate_score;
} gs_view_result;

/* One training view: gs_project -> gs_plan_leaves -> for each leaf
 * (gs_bin_sort, gs_render_fwd, loss, gs_render_bwd, release) ->
 * gs_project_bwd -> optional gs_adam_step; for an L1 view of planned leaves
 * the binning stops at the coarse level (emission, the super-tile sort and
 * its group offsets) and one fused kernel per leaf renders, takes the L1
 * loss and runs the raster backward, each tile walking its super-tile's
 * group and taking the entries that cover it (the same entries in the same
 * order as its gs_bin_sort list, so the same values).  The 2D gradients of all leaves are
 * summed in one buffer before the single projection backward (BoundedGS
 * page "01", Fig. 3, Fig. 5 conclusion).  With Adam and no grad3d_out the
 * projection backward and the update run as one fused pass over the
 * Gaussians (adam_chunk 0), or chunk by chunk of candidate slots; both give
 * the result of gs_project_bwd followed by gs_adam_step.  With more than
 * one planned leaf, the binning of each next leaf (L1: its coarse level)
 * runs on a second stream of the library (default priority, created on first use)
 * while the current leaf is rendered, ordered by events; not while every
 * kernel is timed (gs_set_timing on, no gs_set_timing_only); and, for L1
 * views unless serial_leaves, each leaf's fused raster runs on one of two
 * render streams so that it can start while the previous leaf's last tiles
 * are still being rendered (the previous leaf's coarse buffers are released
 * after its raster ends).  With a gate
 * (SkipGS notes, "key design"): first the forward and the loss of every
 * leaf, then gs_gate_step; when it asks for the backward the leaves are
 * binned and rendered again with their backward (the leaves' buffers are
 * bounded, so they are not kept between the two passes), then the projection
 * backward and the update; otherwise the view ends after its forward
 * (gradients and parameters untouched).  SSIM (loss_kind 1; SkipGS notes,
 * "loss function"): each leaf's tile rectangle grown by one tile on each
 * side inside the grid is binned and rendered, so that the 11 x 11 windows
 * centred within 5 pixels of the leaf see the whole image's pixels; the leaf
 * sums the terms of the centres it owns and runs the raster backward with
 * the exact gradient of its own pixels, so loss and gradients equal the
 * whole image's for any layout (the BoundedGS page, "02 / method", notes
 * that leaf-local windows would differ at the leaf edges).  Per leaf it
 * holds 18 floats per pixel of the grown rectangle (image, gradient, target
 * slice, 9 partial maps) on top of the binning.  The leaves are not binned
 * ahead for SSIM; with a host target each next leaf's slice is copied on the
 * second stream while the current leaf is rendered.  When opts->cost is
 * NULL the plan uses gs_default_cost_model() with these 18 floats added to
 * b_pixel (SSIM), or gs_train_cost_model() with a host target's 3-float
 * slice as b_pixel (L1; with overlapped leaves up to three slices are held
 * at once).  target: device [3][H][W], or host memory with
 * target_host (BoundedGS page, "02 / method": bounded image feeding).
 * Errors: INVALID_ARG, OOM, BUDGET (strict planning), OVERFLOW, DEVICE.  On
 * error the parameters and moments are untouched (everything the view
 * allocates is allocated before its update is queued), but image_out and
 * grad3d_out may hold a partial result: the leaves are rendered one after
 * another in bounded memory, so a failure at a later leaf comes after the
 * earlier leaves wrote their pixels.
 * Synchronises. */
gs_status gs_train_view(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, const float* target,
                        const gs_view_opts* opts, gs_view_result* result);

#ifdef __cplusplus
}
#endif
#endif
