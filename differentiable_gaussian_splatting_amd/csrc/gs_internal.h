// gs_internal.h -- host-side internals of libgsmi: context, handles,
// allocation accounting, kernel timing and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/gs.h"

struct GsAlloc {
    void* ptr = nullptr;
    size_t bytes = 0;
    int cat = GS_MEM_SCRATCH;
    int32_t tag = -1;              // leaf of the view it belongs to, or -1
};

struct GsTimerRec {
    const char* name;
    hipEvent_t start, stop;
};

struct gs_ctx {
    int device = 0;
    hipStream_t stream = nullptr;
    gs_alloc_fn alloc = nullptr;
    gs_free_fn free_fn = nullptr;
    void* user = nullptr;
    std::string err;
    uint64_t live = 0, peak = 0, n_alloc = 0, n_free = 0;
    uint64_t live_cat[GS_MEM_NCAT] = {0}, peak_cat[GS_MEM_NCAT] = {0};
    // per-leaf accounting of a view: allocations made while tag >= 0 count
    // for that leaf (live and high-water bytes per leaf index)
    int32_t tag = -1;
    std::vector<uint64_t> tag_live, tag_peak;
    bool timing = false;
    std::string timing_only;       // time only kernels of this name (empty: all)
    std::vector<GsTimerRec> timers;
    std::vector<hipEvent_t> event_pool;
    void* pinned = nullptr;        // small pinned host buffer for count read-backs
    // second stream (default priority, non-blocking) on which gs_train_view
    // bins the next leaf while the current one is rendered, and its events
    hipStream_t side = nullptr;
    hipEvent_t ev_alloc = nullptr, ev_done[2] = {nullptr, nullptr};
    hipEvent_t ev_rectd = nullptr;   // a projection's depth order and rect_d written (on the second stream)
    hipEvent_t ev_counts = nullptr;  // its per-tile counts made (on render stream 0)
    hipEvent_t ev_toff = nullptr;    // a plan's tile offsets and launch order made (render stream 0)
    hipEvent_t ev_written = nullptr; // its compact state written (on the main stream)
    // two render streams: consecutive leaves' fused rasters overlap, the
    // next one filling the compute units the current one's last tiles leave
    hipStream_t rstream[2] = {nullptr, nullptr};
    hipEvent_t ev_ready[2] = {nullptr, nullptr}, ev_rendered[2] = {nullptr, nullptr};
    bool walk_guess = true;        // the last L1 view's raster choice (gs_train_view)
    int num_cu = 256;
    size_t max_lds = 65536;
};

constexpr uint32_t kMagicProj = 0x9a0c0001u, kMagicBins = 0x9a0c0002u, kMagicRaster = 0x9a0c0003u;

struct GsHandle {
    uint32_t magic = 0;
    gs_ctx* ctx = nullptr;
    std::vector<GsAlloc> allocs;
};

struct gs_proj : GsHandle {
    int64_t n = 0, n_cand = 0;
    int sh_degree = 0;
    int W = 0, H = 0, TW = 0, TH = 0;
    uint32_t* ids = nullptr;      // [n_cand] Gaussian id of each slot
    int4* rect = nullptr;         // [n_cand] tx0, ty0, tx1, ty1
    float4* g0 = nullptr;         // [n_cand] x, y, -A/2, -B
    float4* g1 = nullptr;         // [n_cand] -C/2, opacity, r, g
    float4* g2 = nullptr;         // [n_cand] b, depth, radius, flags (bits)
    int32_t* slot_of = nullptr;   // [n] slot or -1
    uint32_t* order = nullptr;    // [n_cand] slots sorted by (depth, slot)
    uint2* rect_d = nullptr;      // [n_cand] rect of order[k] at k, packed (gsd::rect_pack)
    mutable bool rect_d_pending = false;   // order, rect_d written on the second stream: wait for ctx->ev_rectd
    mutable std::vector<GsAlloc> deferred;  // the depth sort's buffers, released after that wait
    int32_t* tile_cnt = nullptr;  // [TH][TW] candidates per tile (made on first use)
    mutable bool tile_cnt_pending = false;   // tile_cnt made on render stream 0: wait for ctx->ev_counts
    // leaf plan of the view (set by gs_plan_leaves): the candidates whose
    // rectangle meets each leaf, so that binning a leaf visits only those
    std::vector<gs_leaf> plan;
    std::vector<uint64_t> plan_off;   // host copy of the group offsets [plan.size() + 1]
    std::vector<uint64_t> plan_cells; // per leaf: (super-tile, candidate) pairs of its coarse level
    std::vector<uint32_t> plan_cbase; // per leaf: value of plan_coff at its first group entry
    std::vector<uint64_t> plan_tbase; // per leaf: start of its tile offsets in plan_toff
    std::vector<uint64_t> plan_isect; // per leaf: intersections
    uint32_t* plan_coff = nullptr;    // device [entries + 1] scan of the entries' coarse pair counts
    uint64_t* plan_toff = nullptr;    // device: per leaf, its tile offsets [T_L + 1]
    uint32_t* plan_order = nullptr;   // device: per leaf at plan_tbase, its tiles longest list first [T_L]
    std::vector<GsAlloc> plan_retired; // earlier plans (bins may still point into them)
    uint32_t* plan_cands = nullptr;   // device [plan_off.back()] depth positions (indices into order), ascending per group
    std::vector<GsAlloc> plan_allocs;
    gs_cost_model plan_cost{};        // cost model the plan was made with
};

struct gs_bins : GsHandle {
    const gs_proj* proj = nullptr;
    gs_tile_rect leaf{};
    int64_t n_tiles = 0, n_isect = 0;
    int TWL = 0, THL = 0;
    uint64_t* offsets = nullptr;  // [n_tiles + 1]
    uint32_t* values = nullptr;   // [n_isect]
    const uint32_t* order = nullptr;   // [n_tiles] launch order of the fused raster (plan memory) or null
};

struct gs_raster : GsHandle {
    const gs_bins* bins = nullptr;
    int64_t n_pix = 0;
    int px0 = 0, py0 = 0, WL = 0, HL = 0;
    float* tfinal = nullptr;      // [n_pix]
    uint32_t* last = nullptr;     // [n_pix]
    uint8_t* sgn = nullptr;       // [n_pix] L1 residual signs (2 bits per channel) or null
    double* l1_part = nullptr;    // [n_tiles * 4]
};

// ---- error plumbing --------------------------------------------------------
gs_status gs_fail(gs_ctx* ctx, gs_status st, const char* fmt, ...);
#define GS_HIP(ctx, call)                                                                       \
    do {                                                                                        \
        hipError_t e_ = (call);                                                                 \
        if (e_ != hipSuccess) return gs_fail((ctx), GS_ERR_DEVICE, "%s failed: %s (%s:%d)", #call, \
                                             hipGetErrorString(e_), __FILE__, __LINE__);         \
    } while (0)

// ---- memory -----------------------------------------------------------------
void* gs_malloc(gs_ctx* ctx, size_t bytes, int cat, std::vector<GsAlloc>* owner);
void gs_free_all(gs_ctx* ctx, std::vector<GsAlloc>* owner);
void gs_free_one(gs_ctx* ctx, std::vector<GsAlloc>* owner, void* ptr);

// Allocations made while a LeafTag is alive count for leaf `t` of the view.
struct LeafTag {
    gs_ctx* ctx;
    int32_t prev;
    LeafTag(gs_ctx* c, int32_t t) : ctx(c), prev(c->tag) { ctx->tag = t; }
    ~LeafTag() { ctx->tag = prev; }
};

// ---- timing -----------------------------------------------------------------
struct GsTimerScope {
    gs_ctx* ctx;
    const char* name;
    hipEvent_t stop = nullptr;
    GsTimerScope(gs_ctx* c, const char* n);
    ~GsTimerScope();
};

// ---- launchers (defined in the .hip files) ------------------------------------
// scan.hip: exclusive scans; out has n + 1 entries, out[n] = total.
gs_status launch_scan_u32_to_u64(gs_ctx* ctx, const uint32_t* in, uint64_t* out, int64_t n);
gs_status launch_scan_u32_to_u32(gs_ctx* ctx, const uint32_t* in, uint32_t* out, int64_t n);
gs_status launch_fill_u32(gs_ctx* ctx, uint32_t* p, uint32_t v, int64_t n);
gs_status launch_fill_f32(gs_ctx* ctx, float* p, float v, int64_t n);
// 2D inclusive prefix over an int32 grid [rows][cols] (rows, then columns)
gs_status launch_prefix2d_i32(gs_ctx* ctx, int32_t* grid, int rows, int cols);
gs_status launch_prefix2d_u64(gs_ctx* ctx, uint64_t* grid, int rows, int cols);

// project.hip
// flags and their exclusive scan (the slots) of all N Gaussians; dkey
// (optional): their depth bits
gs_status launch_project(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, gs_proj* proj,
                         uint32_t* flag_scratch, uint32_t* slot_scratch, uint32_t* dkey = nullptr);
// compact gradient rows of slots [s0, s1) into grad3d (row s - s0)
gs_status launch_project_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, const gs_proj* proj,
                             const float* grad2d, int64_t s0, int64_t s1, float* grad3d);
gs_status launch_export_proj(gs_ctx* ctx, const gs_proj* proj, int field, void* dst);
gs_status launch_exp(gs_ctx* ctx, const float* x, float* y, int64_t n, bool falloff);

// binning.hip
// list: candidate slots to visit (NULL: all n_cand), n_list entries
gs_status launch_rect_diff(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                           int64_t n_list, int32_t* diff);
// super-tiles (8 x 8 tiles, aligned to the image) meeting a leaf
constexpr int kSuperShift = 3;
// coarse key: bits [0, kCellBits) the leaf's super-tile, above them the
// entry's rectangle inside that super-tile (x0, x1 - 1, y0, y1 - 1 in its
// 8 x 8 local tiles, 3 bits each)
constexpr int kCellBits = 20;
int super_cols(gs_tile_rect leaf);
int super_rows(gs_tile_rect leaf);
int64_t super_cells(gs_tile_rect leaf);
int super_shift();
uint32_t super_key_mask();      // bits of a coarse key that hold the super-tile
int64_t super_cells_max();      // super-tiles a leaf may have
// per listed candidate: super-tiles of the leaf its rectangle meets.  Here
// and in launch_emit_cells, list holds positions in the depth order
// (indices into proj->order and proj->rect_d), NULL: every candidate.
gs_status launch_count_cells(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                             int64_t n_list, uint32_t* cnt);
// per-tile candidate counts of the leaf (row-major in the leaf) from proj->tile_cnt
gs_status launch_leaf_counts(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, uint32_t* out);
// (super-tile, slot) pairs at the offsets eoff - ebase (exclusive scan of the counts)
// bst (optional, emit_blocks(total) u32 of scratch): each emission block's
// first candidate is precomputed there instead of searched by the block
gs_status launch_emit_cells(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint32_t* list,
                            int64_t n_list, const uint32_t* eoff, uint32_t ebase, uint64_t total, uint32_t* keys,
                            uint32_t* vals, uint32_t* bst = nullptr);
int64_t emit_blocks(uint64_t total);
// per-tile lists from the super-tile groups (soff: group offsets, toff: tile offsets)
// Work items of the fine level (segments of the super-tile groups), an upper
// bound for n_cells coarse pairs; scratch: item_sc u32 [items], ioff u32
// [n_super + 1], pos u32 [items * 64]
int64_t fine_items_bound(gs_tile_rect leaf, uint64_t n_cells);
// group: slots by super-tile; gkey: their sorted coarse keys (super-tile id
// and the rectangle inside the super-tile)
gs_status launch_fine_lists(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                            const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint64_t* toff,
                            uint32_t* item_sc, uint32_t* ioff, uint32_t* pos, uint64_t n_values, uint32_t* values);
// the two halves of launch_fine_lists: items, counts and write positions;
// then the slot array
gs_status launch_fine_prepare(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                              const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint64_t* toff,
                              uint32_t* item_sc, uint32_t* ioff, uint32_t* pos);
gs_status launch_fine_write(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, const uint64_t* soff,
                            const uint32_t* group, const uint32_t* gkey, uint64_t n_cells, const uint32_t* item_sc,
                            const uint32_t* ioff, uint32_t* pos, uint64_t n_values, uint32_t* values);
gs_status launch_seg_offsets(gs_ctx* ctx, const uint32_t* sorted_keys, int64_t n, int64_t n_seg, uint32_t kmask,
                             uint64_t* offsets);
// the depth sort's input over all n Gaussians: at each candidate's slot s,
// (its depth bits, s)
gs_status launch_depth_pairs(gs_ctx* ctx, int64_t n, const uint32_t* flag, const uint32_t* slot, const uint32_t* dkey,
                             uint32_t* keys, uint32_t* vals);
// rect_d[k] = the packed rectangle of slot order[k]
gs_status launch_rect_depth(gs_ctx* ctx, const gs_proj* proj, const uint32_t* order, uint2* rect_d);
gs_status launch_export_keys(gs_ctx* ctx, const gs_bins* bins, uint64_t* keys);
int bits_for(int64_t n_keys);

// radix.hip: stable sort of (u32 key, u32 value) pairs on the low key_bits bits
gs_status launch_radix_sort(gs_ctx* ctx, uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, int64_t n,
                            int key_bits, bool* in_second, uint64_t* digit_off = nullptr, int64_t n_seg = 0,
                            bool* off_written = nullptr, uint32_t* scratch = nullptr);
int64_t radix_scratch_words(int64_t n);

// Where pixel (px, py) of channel c of an image buffer lives:
// c * plane + (py - oy) * stride + (px - ox).  The whole image is
// {0, 0, W, W * H}; a device slice of a rectangle starting at (x0, y0) and
// w pixels wide is {x0, y0, w, w * h}.
struct PixFrame {
    int32_t ox, oy;
    int64_t stride, plane;
};
inline PixFrame full_frame(int W, int H) { return PixFrame{0, 0, W, (int64_t)W * H}; }

// raster.hip
gs_status launch_raster_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            gs_raster* r, const float* target, PixFrame tf, float* image_out, PixFrame imf,
                            double* loss_accum, uint64_t* stats);
// forward + L1 + backward of one leaf in one launch (no per-pixel state in
// memory); l1_part receives 4 doubles per tile of the leaf
gs_status launch_raster_fused(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                              const float* target, PixFrame tf, float* image_out, double* l1_part, float* grad2d,
                              bool backward);
// The fused raster walking super-tile groups: soff = group offsets of the
// leaf's super-tiles [super_cells(leaf) + 1], group / gkey = the sorted slots
// and coarse keys, order = the plan's tile order (required).
gs_status launch_raster_groups(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, gs_tile_rect leaf,
                               const uint64_t* soff, const uint32_t* group, const uint32_t* gkey,
                               const uint32_t* order, const float* target, PixFrame tf, float* image_out,
                               double* l1_part, float* grad2d, bool backward);
// tiles of each of n_sets offset arrays (set L at base[L], base[L + 1] - base[L]
// - 1 tiles; hleaves: the sets' leaves on the host, for the grid) in the
// fused raster's launch order, written at the same bases
gs_status launch_tile_order_sets(gs_ctx* ctx, int32_t n_sets, const gs_leaf* hleaves, const uint64_t* base,
                                 const uint64_t* offsets, uint32_t* order);
// the same for base = null: one set of n1 tiles at 0 (hleaves[0] its extent)
gs_status launch_tile_order(gs_ctx* ctx, int32_t n_sets, const gs_leaf* hleaves, const uint64_t* base, int64_t n1,
                            const uint64_t* offsets, uint32_t* order);
gs_status launch_raster_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            const gs_raster* r, const float* dl_dimage, PixFrame dlf, float* grad2d);

// planner.hip
// candidates per tile of the whole grid ([TH][TW], from the rectangles)
gs_status launch_tile_counts(gs_ctx* ctx, const gs_proj* proj, int32_t* grid);
// leaf plan; sat: scratch for the table of proj->tile_cnt, which must be
// there when cost->b_isect != 0 (else NULL: the tile counts are not read)
gs_status launch_plan(gs_ctx* ctx, const gs_proj* proj, uint64_t* sat, uint64_t budget, const gs_cost_model* cost,
                      const gs_leaf* roots_dev, int32_t n_roots, gs_leaf* leaves_dev, int32_t max_leaves,
                      int32_t* count_dev, int32_t* over_dev, uint64_t* totals_dev = nullptr);

// leaf -> candidate groups (planner.hip)
// hleaves: the same leaves on the host (their sizes shape the launch grids)
gs_status launch_leaf_map(gs_ctx* ctx, const gs_leaf* leaves_dev, const gs_leaf* hleaves, int32_t n_leaves, int TW,
                          int TH, int32_t* lot);
gs_status launch_leaf_pairs(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, int32_t n_leaves,
                            const int32_t* lot, uint32_t* cnt, const uint64_t* off, uint32_t* keys, uint32_t* vals);
// Per-view offsets of a plan, in three parts:
// - launch_leaf_toff: per leaf the exclusive scan of its tile counts
//   (proj->tile_cnt) at toff + toff_base[L] (T_L + 1 entries);
// - launch_plan_offsets: per grouped entry (sorted by leaf) its coarse pair
//   count and their exclusive scan (u32, modulo 2^32);
// - launch_leaf_bounds: per leaf the scan value at its first entry and its
//   pair count (leaf_cells [2 * n_leaves]) and its intersections (the last of
//   its tile offsets).
gs_status launch_leaf_toff(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, const gs_leaf* hleaves,
                           int32_t n_leaves, const uint64_t* toff_base, uint64_t* toff);
// the leaves' bases in the tile-offset arrays (n_leaves + 1 entries: the sums
// of T_L + 1 over the leaves before)
gs_status launch_tile_bases(gs_ctx* ctx, const gs_leaf* leaves_dev, int32_t n_leaves, uint64_t* base);
gs_status launch_plan_offsets(gs_ctx* ctx, const gs_proj* proj, const gs_leaf* leaves_dev, int64_t n_entries,
                              const uint32_t* leaf_of, const uint32_t* slot, uint32_t* cell_cnt, uint32_t* cell_off);
gs_status launch_leaf_bounds(gs_ctx* ctx, const gs_leaf* leaves_dev, int32_t n_leaves, const uint64_t* group_off,
                             const uint32_t* cell_off, const uint64_t* toff_base, const uint64_t* toff,
                             uint32_t* leaf_cells, uint64_t* leaf_isect);

// loss.hip
// L1 + SSIM over a W x H buffer (image, target, dl_dimage [3][H][W]) that is
// the whole image or a rectangle of it: the windows are zero-padded at the
// buffer's edges, the loss partials sum the centres in the owned rectangle
// [ox0, ox1) x [oy0, oy1) (buffer coordinates), dl_dimage is written there
// and zero elsewhere, and inv is 1 / (3 x the whole image's pixel count).
gs_status launch_ssim(gs_ctx* ctx, int W, int H, int ox0, int oy0, int ox1, int oy1, float inv, const float* image,
                      const float* target, float lambda, float* dl_dimage, double* partials /*[n_blocks*2]*/,
                      int64_t n_blocks, float* scratch /*[9][H][W] */);
int64_t ssim_partial_blocks(int W, int H);
// out = (accumulate ? out : 0) + sum of n values in[k * stride] in a fixed
// order; chunk_sums: 256 doubles of device scratch for long inputs (null:
// allocated and released by the call)
gs_status launch_sum_f64(gs_ctx* ctx, const double* in, int64_t n, int stride, double* out, int accumulate,
                         double* chunk_sums = nullptr);
// A view's loss on the device: kind 0 (L1) from the sum of |x - y| at
// sums[0]; kind 1 (L1 + SSIM) from the sums of S and |x - y| at sums[0],
// sums[1]; normalised by 3 P, in the host's double operations.
gs_status launch_view_loss(gs_ctx* ctx, int kind, const double* sums, int64_t P, double lambda, double* out);
// The static work buffers of gs_loss_ssim_static on the context's device:
// ssim_static_init (called by gs_ctx_create with the device current) looks up
// their address once per device; ssim_static_buffers hands out the parts for
// a W x H image (GS_ERR_OVERFLOW beyond their capacity).
struct SsimStatic {
    float* maps;     // [9][W H]
    double* part;    // [2 x ssim_partial_blocks]
    double* chunk;   // [256]
    double* sums;    // [2]: SSIM and L1 totals
};
gs_status ssim_static_init(gs_ctx* ctx);
gs_status ssim_static_buffers(gs_ctx* ctx, int W, int H, SsimStatic* out);

// adam.hip
// Adam over the Gaussians whose candidates are the slots [s0, s1), with their
// gradient rows in grad3d (row s - s0); [0, n_cand) covers every Gaussian
gs_status launch_adam(gs_ctx* ctx, const gs_proj* proj, int64_t n, int sh_degree, const gs_param_ptrs* p,
                      const gs_param_ptrs* m, const gs_param_ptrs* v, const float* grad3d, int64_t s0, int64_t s1,
                      int32_t step, float lr, float b1, float b2, float eps);
gs_status launch_scatter_grad3d(gs_ctx* ctx, const gs_proj* proj, int F, const float* grad3d, float* dense);
// projection backward of the candidates fused with one Adam step over all N
// Gaussians (no gradient array); p: the parameters the backward reads, pr /
// m / v: the parameters and moments Adam updates (pr may equal p's arrays)
gs_status launch_bwd_adam(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, const gs_proj* proj,
                          const float* grad2d, const gs_param_ptrs* pr, const gs_param_ptrs* m, const gs_param_ptrs* v,
                          int32_t step, float lr, float b1, float b2, float eps);

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
