// gs_api.cpp -- the C ABI of libgsmi (declared in include/gs.h): context,
// allocation accounting, kernel timing, handles, argument checking and the
// whole-view driver.  Every numeric step runs in the HIP kernels of the .hip
// files; this file only allocates, launches, synchronises and checks.
#include <cstdarg>
#include <cstring>
#include <limits>
#include <algorithm>
#include <cmath>
#include <new>

#include "gs_internal.h"

gs_status launch_project_write(gs_ctx* ctx, const gs_camera* cam, const gs_params* p, gs_proj* proj,
                               const uint32_t* flag, const uint32_t* slot);

// ---------------------------------------------------------------------------
// errors

gs_status gs_fail(gs_ctx* ctx, gs_status st, const char* fmt, ...)
{
    if (ctx) {
        char buf[1024];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof(buf), fmt, ap);
        va_end(ap);
        ctx->err = buf;
    }
    return st;
}

// ---------------------------------------------------------------------------
// memory

void* gs_malloc(gs_ctx* ctx, size_t bytes, int cat, std::vector<GsAlloc>* owner)
{
    bytes = (bytes + 255) & ~(size_t)255;
    if (bytes == 0) bytes = 256;
    void* p = nullptr;
    if (ctx->alloc) {
        p = ctx->alloc(ctx->user, bytes, (void*)ctx->stream);
    } else if (hipMallocAsync(&p, bytes, ctx->stream) != hipSuccess) {
        p = nullptr;
    }
    if (!p) {
        gs_fail(ctx, GS_ERR_OOM, "allocation of %zu bytes failed", bytes);
        return nullptr;
    }
    ctx->live += bytes;
    ctx->live_cat[cat] += bytes;
    ctx->peak = std::max(ctx->peak, ctx->live);
    ctx->peak_cat[cat] = std::max(ctx->peak_cat[cat], ctx->live_cat[cat]);
    ctx->n_alloc += 1;
    const int32_t tag = ctx->tag >= 0 && (size_t)ctx->tag < ctx->tag_live.size() ? ctx->tag : -1;
    if (tag >= 0) {
        ctx->tag_live[tag] += bytes;
        ctx->tag_peak[tag] = std::max(ctx->tag_peak[tag], ctx->tag_live[tag]);
    }
    owner->push_back(GsAlloc{p, bytes, cat, tag});
    return p;
}

static void release_alloc(gs_ctx* ctx, const GsAlloc& a)
{
    if (ctx->free_fn) ctx->free_fn(ctx->user, a.ptr, a.bytes, (void*)ctx->stream);
    else (void)hipFreeAsync(a.ptr, ctx->stream);
    ctx->live -= a.bytes;
    ctx->live_cat[a.cat] -= a.bytes;
    if (a.tag >= 0 && (size_t)a.tag < ctx->tag_live.size()) ctx->tag_live[a.tag] -= a.bytes;
    ctx->n_free += 1;
}

void gs_free_all(gs_ctx* ctx, std::vector<GsAlloc>* owner)
{
    for (const GsAlloc& a : *owner) release_alloc(ctx, a);
    owner->clear();
}

void gs_free_one(gs_ctx* ctx, std::vector<GsAlloc>* owner, void* ptr)
{
    for (size_t k = 0; k < owner->size(); ++k)
        if ((*owner)[k].ptr == ptr) {
            release_alloc(ctx, (*owner)[k]);
            owner->erase(owner->begin() + (long)k);
            return;
        }
}

// ---------------------------------------------------------------------------
// timing

static hipEvent_t take_event(gs_ctx* ctx)
{
    if (!ctx->event_pool.empty()) {
        hipEvent_t e = ctx->event_pool.back();
        ctx->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

GsTimerScope::GsTimerScope(gs_ctx* c, const char* n) : ctx(c), name(n)
{
    if (!ctx->timing) return;
    if (!ctx->timing_only.empty() && ctx->timing_only != name) return;
    hipEvent_t s = take_event(ctx);
    stop = take_event(ctx);
    if (!s || !stop) {
        stop = nullptr;
        return;
    }
    (void)hipEventRecord(s, ctx->stream);
    ctx->timers.push_back(GsTimerRec{name, s, stop});
}

GsTimerScope::~GsTimerScope()
{
    if (stop) (void)hipEventRecord(stop, ctx->stream);
}

// ---------------------------------------------------------------------------
// handles

template <typename H>
static H* new_handle(gs_ctx* ctx, uint32_t magic)
{
    H* h = new (std::nothrow) H();
    if (!h) return nullptr;
    h->magic = magic;
    h->ctx = ctx;
    return h;
}

static bool handle_ok(const gs_ctx* ctx, const void* h, uint32_t magic)
{
    if (!h) return false;
    const GsHandle* g = static_cast<const GsHandle*>(h);
    return g->magic == magic && g->ctx == ctx;
}

static void destroy_handle(gs_ctx* ctx, GsHandle* h)
{
    // the other streams may still write a projection's rect_d and tile counts
    if (h->magic == kMagicProj && static_cast<gs_proj*>(h)->rect_d_pending)
        (void)hipStreamWaitEvent(ctx->stream, ctx->ev_rectd, 0);
    if (h->magic == kMagicProj && static_cast<gs_proj*>(h)->tile_cnt_pending)
        (void)hipStreamWaitEvent(ctx->stream, ctx->ev_counts, 0);
    gs_free_all(ctx, &h->allocs);
    if (h->magic == kMagicProj) {
        gs_free_all(ctx, &static_cast<gs_proj*>(h)->deferred);
        gs_free_all(ctx, &static_cast<gs_proj*>(h)->plan_allocs);
        gs_free_all(ctx, &static_cast<gs_proj*>(h)->plan_retired);
    }
    const uint32_t magic = h->magic;
    h->magic = 0;
    // delete through the concrete type
    if (magic == kMagicProj) delete static_cast<gs_proj*>(h);
    else if (magic == kMagicBins) delete static_cast<gs_bins*>(h);
    else if (magic == kMagicRaster) delete static_cast<gs_raster*>(h);
    else delete h;
}

// ---------------------------------------------------------------------------
// read-back helper: copy `bytes` device bytes to the pinned buffer and wait

static gs_status readback(gs_ctx* ctx, const void* dev, size_t bytes, void* host)
{
    GS_HIP(ctx, hipMemcpyAsync(ctx->pinned, dev, bytes, hipMemcpyDeviceToHost, ctx->stream));
    GS_HIP(ctx, hipStreamSynchronize(ctx->stream));
    std::memcpy(host, ctx->pinned, bytes);
    return GS_OK;
}

static gs_status check_camera(gs_ctx* ctx, const gs_camera* cam)
{
    if (!cam) return gs_fail(ctx, GS_ERR_INVALID_ARG, "camera is NULL");
    if (cam->width < 1 || cam->height < 1 || cam->width > (1 << 20) || cam->height > (1 << 20))
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "image size %d x %d out of range", cam->width, cam->height);
    const int64_t tiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
    if (tiles >= (1ll << 31)) return gs_fail(ctx, GS_ERR_OVERFLOW, "too many tiles");
    if (!(cam->fx > 0.0f) || !(cam->fy > 0.0f) || !std::isfinite(cam->fx) || !std::isfinite(cam->fy))
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "focal lengths must be positive and finite");
    return GS_OK;
}

static gs_status check_params(gs_ctx* ctx, const gs_params* p)
{
    if (!p) return gs_fail(ctx, GS_ERR_INVALID_ARG, "params is NULL");
    if (p->n < 0) return gs_fail(ctx, GS_ERR_INVALID_ARG, "negative Gaussian count");
    if (p->n >= (1ll << 31)) return gs_fail(ctx, GS_ERR_OVERFLOW, "at most 2^31 - 1 Gaussians");
    if (p->sh_degree < 0 || p->sh_degree > 3) return gs_fail(ctx, GS_ERR_INVALID_ARG, "sh_degree must be 0..3");
    if (p->n > 0 && (!p->means || !p->log_scales || !p->quats || !p->opacity_logits || !p->sh))
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "a parameter pointer is NULL");
    return GS_OK;
}

// A projection's depth order and rect_d are written on the second stream,
// beside the per-tile counts and the plan; the first reader of either on
// ctx->stream waits for them there (later readers are ordered after it),
// and the sort's buffers are released after that wait.
static gs_status rect_d_ready(gs_ctx* ctx, const gs_proj* proj)
{
    if (!proj->rect_d_pending) return GS_OK;
    GS_HIP(ctx, hipStreamWaitEvent(ctx->stream, ctx->ev_rectd, 0));
    proj->rect_d_pending = false;
    gs_free_all(ctx, &proj->deferred);
    return GS_OK;
}

// leaf -> candidate groups of a plan (leaves on the device), attached to
// proj; every group keeps the candidates' (depth, slot) order
// Candidates per tile of the whole grid, made once per projection.
static gs_status ensure_tile_counts(gs_ctx* ctx, gs_proj* proj)
{
    if (proj->tile_cnt) {
        if (proj->tile_cnt_pending) {
            GS_HIP(ctx, hipStreamWaitEvent(ctx->stream, ctx->ev_counts, 0));
            proj->tile_cnt_pending = false;
        }
        return GS_OK;
    }
    int32_t* g = (int32_t*)gs_malloc(ctx, sizeof(int32_t) * (int64_t)proj->TW * proj->TH, GS_MEM_PROJ, &proj->allocs);
    if (!g) return GS_ERR_OOM;
    const gs_status st = launch_tile_counts(ctx, proj, g);
    if (st != GS_OK) {
        gs_free_one(ctx, &proj->allocs, g);
        return st;
    }
    proj->tile_cnt = g;
    return GS_OK;
}

static gs_status ensure_side(gs_ctx* ctx);

// The per-tile counts of a projection on render stream 0 (idle outside a
// view's rasters), launched by a plan that does not price intersections
// once its own kernels are queued, so that they run beside the plan's
// read-back and the leaf groups: only the leaves' tile offsets (and a plan
// that prices intersections) read them, through ensure_tile_counts, which
// makes ctx->stream wait for them.
static gs_status tile_counts_beside(gs_ctx* ctx, gs_proj* proj)
{
    int32_t* g = (int32_t*)gs_malloc(ctx, sizeof(int32_t) * (int64_t)proj->TW * proj->TH, GS_MEM_PROJ, &proj->allocs);
    if (!g) return GS_ERR_OOM;
    GS_HIP(ctx, hipEventRecord(ctx->ev_alloc, ctx->stream));
    GS_HIP(ctx, hipStreamWaitEvent(ctx->rstream[0], ctx->ev_alloc, 0));
    hipStream_t main = ctx->stream;
    ctx->stream = ctx->rstream[0];
    gs_status st = launch_tile_counts(ctx, proj, g);
    ctx->stream = main;
    // the grid is attached even on failure, so that its release waits
    proj->tile_cnt = g;
    if (st == GS_OK && hipEventRecord(ctx->ev_counts, ctx->rstream[0]) != hipSuccess)
        st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
    if (st != GS_OK) {
        (void)hipStreamSynchronize(ctx->rstream[0]);
        return st;
    }
    proj->tile_cnt_pending = true;
    return GS_OK;
}

static void clear_plan(gs_ctx* ctx, gs_proj* proj, bool retire)
{
    // bins of an earlier plan may still point at its tile offsets: keep its
    // memory until the projection is released
    if (retire)
        for (auto& a : proj->plan_allocs) proj->plan_retired.push_back(a);
    else
        gs_free_all(ctx, &proj->plan_allocs);
    proj->plan_allocs.clear();
    proj->plan.clear();
    proj->plan_off.clear();
    proj->plan_cells.clear();
    proj->plan_cbase.clear();
    proj->plan_tbase.clear();
    proj->plan_isect.clear();
    proj->plan_cands = nullptr;
    proj->plan_coff = nullptr;
    proj->plan_toff = nullptr;
    proj->plan_order = nullptr;
}

// Groups the candidates by planned leaf and precomputes, for the whole view,
// what binning a planned leaf needs besides its own kernels: the leaf's
// candidates in depth order (as positions in proj->order), the offsets of
// their coarse pairs and the leaf's tile offsets.
static gs_status build_plan_groups(gs_ctx* ctx, gs_proj* proj, const gs_leaf* ldev, const gs_leaf* hleaves,
                                   int32_t nl)
{
    clear_plan(ctx, proj, true);
    const int64_t T = (int64_t)proj->TW * proj->TH;
    const int64_t nc = proj->n_cand;
    std::vector<GsAlloc> tmp;
    gs_status st = GS_OK;
    std::vector<gs_leaf> plan(hleaves, hleaves + nl);
    std::vector<uint64_t> hoff(nl + 1, 0), hcells(nl, 0), tbase(nl + 1, 0);
    std::vector<uint32_t> cbase(nl, 0);
    std::vector<uint64_t> hisect(nl, 0);
    // per-leaf results read back together: group offsets [nl + 1], then
    // intersections [nl] (u64), then (first coarse offset, pairs) [2 nl] (u32)
    std::vector<unsigned char> hres(sizeof(uint64_t) * (2 * (size_t)nl + 1) + sizeof(uint32_t) * 2 * (size_t)nl);
    uint64_t* lisect = nullptr;
    uint64_t G = 0;
    bool second = false;
    uint32_t *k0 = nullptr, *k1 = nullptr, *v0 = nullptr, *v1 = nullptr, *ccnt = nullptr, *coff = nullptr;
    uint32_t* lcells = nullptr;
    uint64_t *segoff = nullptr, *dtbase = nullptr, *toff = nullptr;
    uint32_t* torder = nullptr;
    hipError_t e;
    // the leaves' tile offsets and launch order need only the plan and the
    // per-tile counts: with the streams in use they run on render stream 0
    // (behind the counts) beside the leaf groups, and join before the leaf
    // bounds
    const bool toff_beside = !(ctx->timing && ctx->timing_only.empty()) && ensure_side(ctx) == GS_OK;
    bool toff_queued = false;
    hipStream_t main = ctx->stream;
    int32_t* lot = (int32_t*)gs_malloc(ctx, sizeof(int32_t) * T, GS_MEM_SCRATCH, &tmp);
    uint32_t* cnt = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<int64_t>(nc, 1), GS_MEM_SCRATCH, &tmp);
    uint64_t* goff = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (nc + 1), GS_MEM_SCRATCH, &tmp);
    for (int32_t L = 0; L < nl; ++L)
        tbase[L + 1] = tbase[L] + (uint64_t)(plan[L].tx1 - plan[L].tx0) * (uint64_t)(plan[L].ty1 - plan[L].ty0) + 1;
    dtbase = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (nl + 1), GS_MEM_SCRATCH, &tmp);
    toff = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * tbase[nl], GS_MEM_PROJ, &proj->plan_allocs);
    torder = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * tbase[nl], GS_MEM_PROJ, &proj->plan_allocs);
    if (!lot || !cnt || !goff || !dtbase || !toff || !torder) { st = GS_ERR_OOM; goto out; }
    if (toff_beside) {
        if (!proj->tile_cnt && (st = tile_counts_beside(ctx, proj)) != GS_OK) goto out;
        if (hipEventRecord(ctx->ev_alloc, main) != hipSuccess) {
            st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
            goto out;
        }
    }
    if ((st = launch_leaf_map(ctx, ldev, plan.data(), nl, proj->TW, proj->TH, lot)) != GS_OK) goto out;
    if ((st = rect_d_ready(ctx, proj)) != GS_OK) goto out;
    if ((st = launch_leaf_pairs(ctx, proj, ldev, nl, lot, cnt, nullptr, nullptr, nullptr)) != GS_OK) goto out;
    if ((st = launch_scan_u32_to_u64(ctx, cnt, goff, nc)) != GS_OK) goto out;
    if (toff_beside) {
        // queued after the leaf pairs' count so that the GPU starts on those
        // first; the render stream waits only for the allocations above
        if (hipStreamWaitEvent(ctx->rstream[0], ctx->ev_alloc, 0) != hipSuccess) {
            st = gs_fail(ctx, GS_ERR_DEVICE, "stream ordering failed");
            goto out;
        }
        ctx->stream = ctx->rstream[0];
        toff_queued = true;
        st = launch_tile_bases(ctx, ldev, nl, dtbase);
        if (st == GS_OK) st = launch_leaf_toff(ctx, proj, ldev, plan.data(), nl, dtbase, toff);
        if (st == GS_OK) st = launch_tile_order_sets(ctx, nl, plan.data(), dtbase, toff, torder);
        ctx->stream = main;
        if (st == GS_OK && hipEventRecord(ctx->ev_toff, ctx->rstream[0]) != hipSuccess)
            st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
        if (st != GS_OK) goto out;
    }
    if ((st = readback(ctx, goff + nc, sizeof(uint64_t), &G)) != GS_OK) goto out;
    k0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(G, 1), GS_MEM_SCRATCH, &tmp);
    k1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(G, 1), GS_MEM_SCRATCH, &tmp);
    v0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(G, 1), GS_MEM_PROJ, &proj->plan_allocs);
    v1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(G, 1), GS_MEM_PROJ, &proj->plan_allocs);
    segoff = (uint64_t*)gs_malloc(ctx, hres.size(), GS_MEM_SCRATCH, &tmp);
    ccnt = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(G, 1), GS_MEM_SCRATCH, &tmp);
    coff = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * (G + 1), GS_MEM_PROJ, &proj->plan_allocs);
    if (!k0 || !k1 || !v0 || !v1 || !segoff || !ccnt || !coff) {
        st = GS_ERR_OOM;
        goto out;
    }
    lisect = segoff + (nl + 1);
    lcells = (uint32_t*)(lisect + nl);
    if ((st = launch_leaf_pairs(ctx, proj, ldev, nl, lot, cnt, goff, k0, v0)) != GS_OK) goto out;
    if ((st = launch_radix_sort(ctx, k0, v0, k1, v1, (int64_t)G, bits_for(nl), &second)) != GS_OK) goto out;
    if ((st = launch_seg_offsets(ctx, second ? k1 : k0, (int64_t)G, nl, 0xFFFFFFFFu, segoff)) != GS_OK) goto out;
    if ((st = launch_plan_offsets(ctx, proj, ldev, (int64_t)G, second ? k1 : k0, second ? v1 : v0, ccnt, coff)) !=
        GS_OK)
        goto out;
    if (toff_beside) {
        if (hipStreamWaitEvent(main, ctx->ev_toff, 0) != hipSuccess) {
            st = gs_fail(ctx, GS_ERR_DEVICE, "stream wait failed");
            goto out;
        }
    } else {
        // on this stream: the counts, the tile offsets, the launch order
        if ((st = ensure_tile_counts(ctx, proj)) != GS_OK) goto out;
        if ((st = launch_tile_bases(ctx, ldev, nl, dtbase)) != GS_OK) goto out;
        if ((st = launch_leaf_toff(ctx, proj, ldev, plan.data(), nl, dtbase, toff)) != GS_OK) goto out;
        if ((st = launch_tile_order_sets(ctx, nl, plan.data(), dtbase, toff, torder)) != GS_OK) goto out;
    }
    if ((st = launch_leaf_bounds(ctx, ldev, nl, segoff, coff, dtbase, toff, lcells, lisect)) != GS_OK) goto out;
    e = hipMemcpyAsync(hres.data(), segoff, hres.size(), hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) { st = gs_fail(ctx, GS_ERR_DEVICE, "plan copy failed: %s", hipGetErrorString(e)); goto out; }
    {
        const uint64_t* r64 = (const uint64_t*)hres.data();
        const uint32_t* r32 = (const uint32_t*)(r64 + 2 * (size_t)nl + 1);
        for (int32_t L = 0; L <= nl; ++L) hoff[L] = r64[L];
        for (int32_t L = 0; L < nl; ++L) {
            hisect[L] = r64[nl + 1 + L];
            cbase[L] = r32[2 * (size_t)L];
            hcells[L] = r32[2 * (size_t)L + 1];
        }
    }
    gs_free_one(ctx, &proj->plan_allocs, second ? v0 : v1);
    proj->plan_cands = second ? v1 : v0;
    proj->plan_coff = coff;
    proj->plan_toff = toff;
    proj->plan_order = torder;
    proj->plan.swap(plan);
    proj->plan_off.swap(hoff);
    proj->plan_cells.swap(hcells);
    proj->plan_cbase.swap(cbase);
    proj->plan_tbase.swap(tbase);
    proj->plan_isect.swap(hisect);
out:
    // render stream 0 may still use the plan's buffers on an error
    if (st != GS_OK && toff_queued) (void)hipStreamSynchronize(ctx->rstream[0]);
    gs_free_all(ctx, &tmp);
    if (st != GS_OK) clear_plan(ctx, proj, false);
    return st;
}

// What binning a leaf of the current plan can take from it; found = false
// when the leaf is not part of the plan.
struct PlanLeaf {
    bool found = false;
    const uint32_t* list = nullptr;   // candidates meeting the leaf: depth positions, ascending
    int64_t n = 0;
    int64_t isect = -1;               // from the plan's tile offsets
    int64_t cells = 0;                // coarse pairs
    const uint32_t* eoff = nullptr;   // their offsets (subtract ebase)
    uint32_t ebase = 0;
    uint64_t* toff = nullptr;         // tile offsets [T_L + 1]
    const uint32_t* order = nullptr;  // tiles longest list first [T_L]
};

static PlanLeaf plan_leaf(const gs_proj* proj, gs_tile_rect leaf)
{
    PlanLeaf r;
    if (!proj->plan_cands) return r;
    for (size_t k = 0; k < proj->plan.size(); ++k) {
        const gs_leaf& L = proj->plan[k];
        if (L.tx0 == leaf.tx0 && L.ty0 == leaf.ty0 && L.tx1 == leaf.tx1 && L.ty1 == leaf.ty1) {
            r.found = true;
            r.list = proj->plan_cands + proj->plan_off[k];
            r.n = (int64_t)(proj->plan_off[k + 1] - proj->plan_off[k]);
            r.cells = (int64_t)proj->plan_cells[k];
            r.eoff = proj->plan_coff + proj->plan_off[k];
            r.ebase = proj->plan_cbase[k];
            r.toff = proj->plan_toff + proj->plan_tbase[k];
            r.order = proj->plan_order + proj->plan_tbase[k];
            r.isect = (int64_t)proj->plan_isect[k];
            return r;
        }
    }
    return r;
}

extern "C" {

// ---------------------------------------------------------------------------
// context

gs_status gs_ctx_create(gs_ctx** out, void* stream, gs_alloc_fn alloc, gs_free_fn free_fn, void* user)
{
    if (!out) return GS_ERR_INVALID_ARG;
    *out = nullptr;
    if ((alloc == nullptr) != (free_fn == nullptr)) return GS_ERR_INVALID_ARG;
    gs_ctx* c = new (std::nothrow) gs_ctx();
    if (!c) return GS_ERR_OOM;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        return GS_ERR_DEVICE;
    }
    c->stream = (hipStream_t)stream;
    c->alloc = alloc;
    c->free_fn = free_fn;
    c->user = user;
    if (hipHostMalloc(&c->pinned, 256, hipHostMallocDefault) != hipSuccess) {
        delete c;
        return GS_ERR_DEVICE;
    }
    // the device address of the static SSIM work buffers, once per device
    if (ssim_static_init(c) != GS_OK) {
        (void)hipHostFree(c->pinned);
        delete c;
        return GS_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, c->device) == hipSuccess) {
        c->num_cu = prop.multiProcessorCount;
        c->max_lds = prop.sharedMemPerBlock;
    }
    *out = c;
    return GS_OK;
}

void gs_ctx_destroy(gs_ctx* ctx)
{
    if (!ctx) return;
    (void)hipStreamSynchronize(ctx->stream);
    if (ctx->side) {
        (void)hipStreamSynchronize(ctx->side);
        (void)hipStreamDestroy(ctx->side);
    }
    if (ctx->ev_alloc) (void)hipEventDestroy(ctx->ev_alloc);
    if (ctx->ev_rectd) (void)hipEventDestroy(ctx->ev_rectd);
    if (ctx->ev_counts) (void)hipEventDestroy(ctx->ev_counts);
    if (ctx->ev_toff) (void)hipEventDestroy(ctx->ev_toff);
    if (ctx->ev_written) (void)hipEventDestroy(ctx->ev_written);
    for (hipEvent_t e : ctx->ev_done)
        if (e) (void)hipEventDestroy(e);
    for (int k = 0; k < 2; ++k) {
        if (ctx->rstream[k]) {
            (void)hipStreamSynchronize(ctx->rstream[k]);
            (void)hipStreamDestroy(ctx->rstream[k]);
        }
        if (ctx->ev_ready[k]) (void)hipEventDestroy(ctx->ev_ready[k]);
        if (ctx->ev_rendered[k]) (void)hipEventDestroy(ctx->ev_rendered[k]);
    }
    for (auto& t : ctx->timers) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
    if (ctx->pinned) (void)hipHostFree(ctx->pinned);
    delete ctx;
}

const char* gs_last_error(const gs_ctx* ctx) { return ctx ? ctx->err.c_str() : "no context"; }

gs_status gs_mem_stats_get(const gs_ctx* ctx, gs_mem_stats* out)
{
    if (!ctx || !out) return GS_ERR_INVALID_ARG;
    out->live_bytes = ctx->live;
    out->peak_bytes = ctx->peak;
    for (int k = 0; k < GS_MEM_NCAT; ++k) {
        out->live_by_cat[k] = ctx->live_cat[k];
        out->peak_by_cat[k] = ctx->peak_cat[k];
    }
    out->n_alloc = ctx->n_alloc;
    out->n_free = ctx->n_free;
    return GS_OK;
}

gs_status gs_mem_reset_peak(gs_ctx* ctx)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    ctx->peak = ctx->live;
    for (int k = 0; k < GS_MEM_NCAT; ++k) ctx->peak_cat[k] = ctx->live_cat[k];
    return GS_OK;
}

gs_status gs_set_timing(gs_ctx* ctx, int32_t on)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    ctx->timing = on != 0;
    return GS_OK;
}

gs_status gs_set_timing_only(gs_ctx* ctx, const char* name)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    ctx->timing_only = name ? name : "";
    return GS_OK;
}

gs_status gs_reset_timing(gs_ctx* ctx)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    GS_HIP(ctx, hipStreamSynchronize(ctx->stream));
    for (auto& t : ctx->timers) {
        ctx->event_pool.push_back(t.start);
        ctx->event_pool.push_back(t.stop);
    }
    ctx->timers.clear();
    return GS_OK;
}

gs_status gs_kernel_time(gs_ctx* ctx, const char* name, double* total_ms, int64_t* launches)
{
    if (!ctx || !name || !total_ms || !launches) return GS_ERR_INVALID_ARG;
    GS_HIP(ctx, hipStreamSynchronize(ctx->stream));
    double tot = 0.0;
    int64_t cnt = 0;
    for (auto& t : ctx->timers)
        if (std::strcmp(t.name, name) == 0) {
            float ms = 0.0f;
            GS_HIP(ctx, hipEventElapsedTime(&ms, t.start, t.stop));
            tot += ms;
            cnt += 1;
        }
    *total_ms = tot;
    *launches = cnt;
    return GS_OK;
}

gs_cost_model gs_default_cost_model(void)
{
    // Upper bounds of the bytes the library allocates for a planned leaf,
    // all of a leaf's buffers counted as held at once:
    //   coarse sort of the C coarse pairs (C <= Cb): keys u32 x 2 and slots
    //     u32 x 2 (ping-pong) + the digit histogram of a single 10-bit pass
    //     (1024 u32 per 2048 pairs) -> 18 B per pair;
    //   fine lists: per work item (at most one per super-tile, so per tile,
    //     plus one per 512 pairs) 64 u32 positions, its super-tile and
    //     offsets -> 0.5 B per pair (19 B per pair in all), 272 B per tile;
    //     the slots u32 per intersection -> 4 B per intersection;
    //   rasterization (gs_render_fwd): T_final f32 + last u32 + L1 signs u8
    //     per pixel, 4 f64 L1 partials per tile -> 9 B, 32 B;
    //   constant: scan block sums, digit totals, allocation rounding.
    // The fused forward + L1 + backward of gs_train_view allocates no
    // per-pixel state, so for it the 9 B per pixel are slack.
    gs_cost_model c;
    c.b_isect = 4;
    c.b_cell = 19;
    c.b_pixel = 9;
    c.b_tile = 320;
    c.b_const = 1u << 20;
    return c;
}

gs_cost_model gs_train_cost_model(void)
{
    // Upper bounds of the bytes gs_train_view allocates for a planned leaf of
    // an L1 view (the fused raster walks the super-tile groups):
    //   coarse sort of the C coarse pairs (C <= Cb): keys u32 x 2 and slots
    //     u32 x 2 (ping-pong) + the digit counts of a single 10-bit pass
    //     (1024 u32 per 2048 pairs) -> 18 B per pair;
    //   group offsets: a u64 per super-tile, at most one per tile -> 8 B;
    //   constant: digit totals, allocation rounding.
    // No per-tile list, no per-intersection and no per-pixel buffer.
    gs_cost_model c;
    c.b_isect = 0;
    c.b_cell = 19;
    c.b_pixel = 0;
    c.b_tile = 8;
    c.b_const = 1u << 20;
    return c;
}

// ---------------------------------------------------------------------------
// projection

gs_status gs_project(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, gs_proj** out, int64_t* n_cand)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (!out || !n_cand) return gs_fail(ctx, GS_ERR_INVALID_ARG, "out / n_cand is NULL");
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if ((st = check_params(ctx, params)) != GS_OK) return st;
    gs_proj* p = new_handle<gs_proj>(ctx, kMagicProj);
    if (!p) return gs_fail(ctx, GS_ERR_OOM, "host allocation failed");
    p->n = params->n;
    p->sh_degree = params->sh_degree;
    p->W = cam->width;
    p->H = cam->height;
    p->TW = (cam->width + 15) / 16;
    p->TH = (cam->height + 15) / 16;
    std::vector<GsAlloc> tmp;
    // flags, slots and depth keys of all N Gaussians, and the depth sort's
    // keys and spare value buffer: the second stream reads them, so with it
    // in use they are released by rect_d_ready (or with the projection)
    std::vector<GsAlloc> sortbuf;
    bool side_used = false;
    bool second = false;
    const int64_t n = params->n;
    const bool beside = !(ctx->timing && ctx->timing_only.empty()) && ensure_side(ctx) == GS_OK;
    hipStream_t main = ctx->stream;
    uint32_t* flag = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<int64_t>(n, 1), GS_MEM_SCRATCH, &sortbuf);
    uint32_t* slot = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * (n + 1), GS_MEM_SCRATCH, &sortbuf);
    uint32_t* dkey = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<int64_t>(n, 1), GS_MEM_SCRATCH, &sortbuf);
    uint32_t *k0 = nullptr, *k1 = nullptr, *v0 = nullptr, *v1 = nullptr;
    uint32_t cnt = 0;
    if (!flag || !slot || !dkey) { st = GS_ERR_OOM; goto fail; }
    if ((st = launch_project(ctx, cam, params, p, flag, slot, dkey)) != GS_OK) goto fail;
    if ((st = readback(ctx, slot + n, sizeof(uint32_t), &cnt)) != GS_OK) goto fail;
    p->n_cand = cnt;
    {
        const int64_t nc = std::max<int64_t>(cnt, 1);
        p->ids = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_PROJ, &p->allocs);
        p->rect = (int4*)gs_malloc(ctx, sizeof(int4) * nc, GS_MEM_PROJ, &p->allocs);
        p->g0 = (float4*)gs_malloc(ctx, sizeof(float4) * nc, GS_MEM_PROJ, &p->allocs);
        p->g1 = (float4*)gs_malloc(ctx, sizeof(float4) * nc, GS_MEM_PROJ, &p->allocs);
        p->g2 = (float4*)gs_malloc(ctx, sizeof(float4) * nc, GS_MEM_PROJ, &p->allocs);
        p->slot_of = (int32_t*)gs_malloc(ctx, sizeof(int32_t) * std::max<int64_t>(n, 1), GS_MEM_PROJ, &p->allocs);
        k0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_SCRATCH, &sortbuf);
        k1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_SCRATCH, &sortbuf);
        v0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_PROJ, &p->allocs);
        v1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_PROJ, &p->allocs);
        p->rect_d = (uint2*)gs_malloc(ctx, sizeof(uint2) * nc, GS_MEM_PROJ, &p->allocs);
        if (!p->ids || !p->rect || !p->g0 || !p->g1 || !p->g2 || !p->slot_of || !k0 || !k1 || !v0 || !v1 ||
            !p->rect_d) {
            st = GS_ERR_OOM;
            goto fail;
        }
    }
    // Candidates in (depth, slot) order: a stable radix sort of the depth
    // bits (kept per Gaussian by the flag pass) over slots in ascending
    // order, on the second stream while this one writes the compact state
    // (queued first, so that it runs while the host queues the sort); then,
    // once that is written, the rectangles in that order (rect_d).  This
    // stream goes on (a view plans its leaves meanwhile); readers of the
    // order and of rect_d wait for the second stream first (rect_d_ready).
    // With every kernel timed, all of it runs on this stream.
    if (beside && hipEventRecord(ctx->ev_alloc, main) != hipSuccess) {
        st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
        goto fail;
    }
    if ((st = launch_project_write(ctx, cam, params, p, flag, slot)) != GS_OK) goto fail;
    if (beside) {
        if (hipEventRecord(ctx->ev_written, main) != hipSuccess ||
            hipStreamWaitEvent(ctx->side, ctx->ev_alloc, 0) != hipSuccess) {
            st = gs_fail(ctx, GS_ERR_DEVICE, "stream ordering failed");
            goto fail;
        }
        ctx->stream = ctx->side;
        side_used = true;
    }
    st = launch_depth_pairs(ctx, n, flag, slot, dkey, k0, v0);
    if (st == GS_OK) st = launch_radix_sort(ctx, k0, v0, k1, v1, (int64_t)cnt, 32, &second);
    if (st == GS_OK && beside && hipStreamWaitEvent(ctx->side, ctx->ev_written, 0) != hipSuccess)
        st = gs_fail(ctx, GS_ERR_DEVICE, "stream ordering failed");
    if (st == GS_OK) st = launch_rect_depth(ctx, p, second ? v1 : v0, p->rect_d);
    ctx->stream = main;
    if (beside && st == GS_OK && hipEventRecord(ctx->ev_rectd, ctx->side) != hipSuccess)
        st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
    if (st != GS_OK) goto fail;
    // the spare value buffer joins the sort's keys
    for (size_t k = 0; k < p->allocs.size(); ++k)
        if (p->allocs[k].ptr == (second ? (void*)v0 : (void*)v1)) {
            sortbuf.push_back(p->allocs[k]);
            p->allocs.erase(p->allocs.begin() + (long)k);
            break;
        }
    p->order = second ? v1 : v0;
    if (beside) {
        p->deferred.swap(sortbuf);   // released by rect_d_ready or with the projection
        p->rect_d_pending = true;
    } else {
        gs_free_all(ctx, &sortbuf);
        // the per-tile counts (with the streams in use they are launched by
        // the first plan, beside it, or made on first use)
        if ((st = ensure_tile_counts(ctx, p)) != GS_OK) goto fail;
    }
    gs_free_all(ctx, &tmp);
    *out = p;
    *n_cand = (int64_t)cnt;
    return GS_OK;
fail:
    // nothing is released while the second stream may still use it
    ctx->stream = main;
    if (side_used) (void)hipStreamSynchronize(ctx->side);
    gs_free_all(ctx, &sortbuf);
    gs_free_all(ctx, &tmp);
    destroy_handle(ctx, p);
    return st;
}

// ---------------------------------------------------------------------------
// planning

// A fresh plan (roots null) or the re-check of a cached layout: roots (host)
// must tile the grid exactly (partial: must not overlap); each is kept when
// within the budget and split by the halving rule otherwise.
static gs_status plan_impl(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, uint64_t budget_bytes,
                           const gs_cost_model* cost, int32_t strict, const gs_leaf* roots, int32_t n_roots,
                           gs_leaf* leaves, int32_t max_leaves, int32_t* n_leaves, bool partial = false,
                           uint64_t* totals = nullptr)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if (!handle_ok(ctx, proj, kMagicProj)) return gs_fail(ctx, GS_ERR_STATE, "invalid projection handle");
    if (proj->W != cam->width || proj->H != cam->height)
        return gs_fail(ctx, GS_ERR_STATE, "camera does not match the projection");
    if (budget_bytes == 0) return gs_fail(ctx, GS_ERR_INVALID_ARG, "budget must be > 0");
    if (!n_leaves || (max_leaves > 0 && !leaves) || max_leaves < 0)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "leaves / n_leaves");
    const gs_cost_model cm = cost ? *cost : gs_default_cost_model();
    const int64_t T = (int64_t)proj->TW * proj->TH;
    const int32_t cap = (int32_t)std::min<int64_t>(std::max<int32_t>(max_leaves, 1), T);
    if (n_roots > 0) {
        // the cached leaves must cover every tile of the grid exactly once
        if (!roots || n_roots > T) return gs_fail(ctx, GS_ERR_INVALID_ARG, "cached leaves: %d for %lld tiles",
                                                  (int)n_roots, (long long)T);
        std::vector<uint8_t> cover((size_t)T, 0);
        for (int32_t k = 0; k < n_roots; ++k) {
            const gs_leaf& R = roots[k];
            if (R.tx0 < 0 || R.ty0 < 0 || R.tx1 > proj->TW || R.ty1 > proj->TH || R.tx0 >= R.tx1 || R.ty0 >= R.ty1)
                return gs_fail(ctx, GS_ERR_INVALID_ARG, "cached leaf %d outside the tile grid or empty", (int)k);
            for (int32_t ty = R.ty0; ty < R.ty1; ++ty)
                for (int32_t tx = R.tx0; tx < R.tx1; ++tx) {
                    uint8_t& c = cover[(size_t)ty * proj->TW + tx];
                    if (c) return gs_fail(ctx, GS_ERR_INVALID_ARG, "cached leaves overlap at tile (%d, %d)", tx, ty);
                    c = 1;
                }
        }
        for (size_t t = 0; t < cover.size() && !partial; ++t)
            if (!cover[t]) return gs_fail(ctx, GS_ERR_INVALID_ARG, "cached leaves leave tile %zu uncovered", t);
    }
    std::vector<GsAlloc> tmp;
    // the tile counts only when the model prices intersections
    const bool priced = cm.b_isect != 0;
    if (priced && (st = ensure_tile_counts(ctx, const_cast<gs_proj*>(proj))) != GS_OK) return st;
    uint64_t* sat = priced ? (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (proj->TW + 1) * (int64_t)(proj->TH + 1),
                                                  GS_MEM_SCRATCH, &tmp)
                           : nullptr;
    // the leaf count and the over-budget flag (64 bytes), then the leaves:
    // read back together, the first kFirst leaves with the count
    constexpr int32_t kFirst = 128;
    unsigned char* blk = (unsigned char*)gs_malloc(ctx, 64 + sizeof(gs_leaf) * (size_t)cap, GS_MEM_SCRATCH, &tmp);
    int32_t* small = (int32_t*)blk;
    gs_leaf* ldev = (gs_leaf*)(blk + 64);
    gs_leaf* rdev = n_roots > 0 ? (gs_leaf*)gs_malloc(ctx, sizeof(gs_leaf) * n_roots, GS_MEM_SCRATCH, &tmp) : nullptr;
    int32_t hv[2] = {0, 0};
    std::vector<unsigned char> hblk(64 + sizeof(gs_leaf) * (size_t)std::min(cap, kFirst));
    std::vector<gs_leaf> hleaves;
    if ((priced && !sat) || !blk || (n_roots > 0 && !rdev)) {
        gs_free_all(ctx, &tmp);
        return GS_ERR_OOM;
    }
    if (n_roots > 0) {
        const hipError_t e = hipMemcpyAsync(rdev, roots, sizeof(gs_leaf) * n_roots, hipMemcpyHostToDevice, ctx->stream);
        if (e != hipSuccess) {
            gs_free_all(ctx, &tmp);
            return gs_fail(ctx, GS_ERR_DEVICE, "cached leaf copy failed: %s", hipGetErrorString(e));
        }
    }
    // header: leaf count, over-budget flag, then (u64 at byte 8) the whole
    // grid's intersections and (candidate, super-cell) pairs
    st = launch_plan(ctx, proj, sat, budget_bytes, &cm, rdev, n_roots, ldev, cap, small, small + 1,
                     (uint64_t*)(blk + 8));
    if (st == GS_OK && !proj->tile_cnt && !(ctx->timing && ctx->timing_only.empty()) && ensure_side(ctx) == GS_OK)
        st = tile_counts_beside(ctx, const_cast<gs_proj*>(proj));
    if (st == GS_OK) {
        hipError_t e = hipMemcpyAsync(hblk.data(), blk, hblk.size(), hipMemcpyDeviceToHost, ctx->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
        if (e != hipSuccess) st = gs_fail(ctx, GS_ERR_DEVICE, "plan read-back failed: %s", hipGetErrorString(e));
    }
    if (st == GS_OK) {
        std::memcpy(hv, hblk.data(), sizeof(hv));
        if (totals) std::memcpy(totals, hblk.data() + 8, 2 * sizeof(uint64_t));
        const int32_t nh = std::min(hv[0], cap);
        if (nh > 0) {
            hleaves.resize(nh);
            const int32_t n1 = std::min(nh, kFirst);
            std::memcpy(hleaves.data(), hblk.data() + 64, sizeof(gs_leaf) * n1);
            if (nh > n1) {
                hipError_t e = hipMemcpyAsync(hleaves.data() + n1, ldev + n1, sizeof(gs_leaf) * (nh - n1),
                                              hipMemcpyDeviceToHost, ctx->stream);
                if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
                if (e != hipSuccess) st = gs_fail(ctx, GS_ERR_DEVICE, "leaf copy failed: %s", hipGetErrorString(e));
            }
            if (st == GS_OK && max_leaves > 0)
                std::memcpy(leaves, hleaves.data(), sizeof(gs_leaf) * std::min(nh, max_leaves));
        }
    }
    // Attach the leaf -> candidate groups of this plan to the projection, so
    // that gs_bin_sort of a planned leaf visits only the candidates meeting it.
    if (st == GS_OK && hv[0] > 0 && hv[0] <= cap) {
        st = build_plan_groups(ctx, const_cast<gs_proj*>(proj), ldev, hleaves.data(), hv[0]);
        const_cast<gs_proj*>(proj)->plan_cost = cm;
    }
    gs_free_all(ctx, &tmp);
    if (st != GS_OK) return st;
    *n_leaves = hv[0];
    if (strict && hv[1]) return gs_fail(ctx, GS_ERR_BUDGET, "a single tile exceeds the budget");
    return GS_OK;
}

gs_status gs_grid_leaves(int32_t tiles_x, int32_t tiles_y, int32_t nx, int32_t ny, gs_leaf* out)
{
    if (!out || tiles_x < 1 || tiles_y < 1 || nx < 1 || ny < 1 || nx > tiles_x || ny > tiles_y)
        return GS_ERR_INVALID_ARG;
    for (int32_t j = 0; j < ny; ++j)
        for (int32_t i = 0; i < nx; ++i) {
            gs_leaf& L = out[(size_t)j * nx + i];
            L = gs_leaf{};
            L.tx0 = (int32_t)((int64_t)i * tiles_x / nx);
            L.tx1 = (int32_t)((int64_t)(i + 1) * tiles_x / nx);
            L.ty0 = (int32_t)((int64_t)j * tiles_y / ny);
            L.ty1 = (int32_t)((int64_t)(j + 1) * tiles_y / ny);
        }
    return GS_OK;
}

gs_status gs_plan_leaves(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, uint64_t budget_bytes,
                         const gs_cost_model* cost, int32_t strict, gs_leaf* leaves, int32_t max_leaves,
                         int32_t* n_leaves)
{
    return plan_impl(ctx, cam, proj, budget_bytes, cost, strict, nullptr, 0, leaves, max_leaves, n_leaves);
}

gs_status gs_replan_leaves(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, uint64_t budget_bytes,
                           const gs_cost_model* cost, int32_t strict, const gs_leaf* cached, int32_t n_cached,
                           gs_leaf* leaves, int32_t max_leaves, int32_t* n_leaves)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (!cached || n_cached < 1) return gs_fail(ctx, GS_ERR_INVALID_ARG, "no cached leaves");
    return plan_impl(ctx, cam, proj, budget_bytes, cost, strict, cached, n_cached, leaves, max_leaves, n_leaves);
}

// ---------------------------------------------------------------------------
// binning

// ---------------------------------------------------------------------------
// The coarse stage of a planned leaf, which is all the binning an L1 view's
// fused raster needs (it walks the super-tile groups itself), split so that
// gs_train_view can run it on a second stream for the next leaf while the
// current one is rendered:
//   coarse_alloc (main stream): every buffer the stage needs;
//   coarse_launch (any stream, allocates nothing): emission, the coarse sort
//     and the super-tile group offsets.
// The buffers stay until the leaf's raster has ended.  The same kernels and
// launch shapes as the first half of gs_bin_sort.
struct CoarseBins {
    gs_tile_rect leaf{};
    PlanLeaf pl{};
    int64_t n_super = 0;
    uint64_t C = 0, I = 0;
    uint32_t *k0 = nullptr, *v0 = nullptr, *k1 = nullptr, *v1 = nullptr, *scratch = nullptr;
    uint64_t* soff = nullptr;
    bool second = false;
    std::vector<GsAlloc> allocs;
};

static bool leaf_pipelinable(const gs_proj* proj, gs_tile_rect leaf)
{
    const PlanLeaf pl = plan_leaf(proj, leaf);
    return pl.found && pl.isect >= 0 && pl.order && super_cells(leaf) < super_cells_max() &&
           (uint64_t)pl.cells < (1ull << 32);
}

static gs_status coarse_alloc(gs_ctx* ctx, const gs_proj* proj, gs_tile_rect leaf, CoarseBins* cb)
{
    cb->leaf = leaf;
    cb->pl = plan_leaf(proj, leaf);
    cb->n_super = super_cells(leaf);
    cb->C = (uint64_t)cb->pl.cells;
    cb->I = (uint64_t)cb->pl.isect;
    const uint64_t nc = std::max<uint64_t>(cb->C, 1);
    auto get = [&](size_t bytes) { return gs_malloc(ctx, bytes, GS_MEM_RASTER, &cb->allocs); };
    cb->k0 = (uint32_t*)get(sizeof(uint32_t) * nc);
    cb->v0 = (uint32_t*)get(sizeof(uint32_t) * nc);
    cb->k1 = (uint32_t*)get(sizeof(uint32_t) * nc);
    cb->v1 = (uint32_t*)get(sizeof(uint32_t) * nc);
    cb->soff = (uint64_t*)get(sizeof(uint64_t) * (cb->n_super + 1));
    cb->scratch = (uint32_t*)get(sizeof(uint32_t) * radix_scratch_words((int64_t)cb->C));
    if (!cb->k0 || !cb->v0 || !cb->k1 || !cb->v1 || !cb->soff || !cb->scratch) {
        gs_free_all(ctx, &cb->allocs);
        return GS_ERR_OOM;
    }
    return GS_OK;
}

static gs_status coarse_launch(gs_ctx* ctx, const gs_proj* proj, CoarseBins* cb)
{
    gs_status st = rect_d_ready(ctx, proj);
    if (st != GS_OK) return st;
    // the radix scratch (idle until the sort) holds the emission's block starts
    st = launch_emit_cells(ctx, proj, cb->leaf, cb->pl.list, cb->pl.n, cb->pl.eoff, cb->pl.ebase, cb->C,
                           cb->k0, cb->v0, cb->scratch);
    if (st != GS_OK) return st;
    bool have_soff = false;
    if ((st = launch_radix_sort(ctx, cb->k0, cb->v0, cb->k1, cb->v1, (int64_t)cb->C, bits_for(cb->n_super),
                                &cb->second, cb->soff, cb->n_super, &have_soff, cb->scratch)) != GS_OK)
        return st;
    const uint32_t* gkey = cb->second ? cb->k1 : cb->k0;
    if (!have_soff &&
        (st = launch_seg_offsets(ctx, gkey, (int64_t)cb->C, cb->n_super, super_key_mask(), cb->soff)) != GS_OK)
        return st;
    return GS_OK;
}

static gs_status ensure_side(gs_ctx* ctx)
{
    if (ctx->side) return GS_OK;
    GS_HIP(ctx, hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_alloc, hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_rectd, hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_counts, hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_toff, hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_written, hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_done[0], hipEventDisableTiming));
    GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_done[1], hipEventDisableTiming));
    for (int k = 0; k < 2; ++k) {
        GS_HIP(ctx, hipStreamCreateWithFlags(&ctx->rstream[k], hipStreamNonBlocking));
        GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_ready[k], hipEventDisableTiming));
        GS_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_rendered[k], hipEventDisableTiming));
    }
    return GS_OK;
}

// stage one of leaf cb on the side stream, after everything the main stream
// has queued so far (its buffers may reuse memory the main stream freed)
static gs_status coarse_on_side(gs_ctx* ctx, const gs_proj* proj, CoarseBins* cb, hipEvent_t done)
{
    GS_HIP(ctx, hipEventRecord(ctx->ev_alloc, ctx->stream));
    GS_HIP(ctx, hipStreamWaitEvent(ctx->side, ctx->ev_alloc, 0));
    hipStream_t main = ctx->stream;
    ctx->stream = ctx->side;
    const gs_status st = coarse_launch(ctx, proj, cb);
    ctx->stream = main;
    if (st != GS_OK) return st;
    GS_HIP(ctx, hipEventRecord(done, ctx->side));
    return GS_OK;
}

gs_status gs_bin_sort(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, gs_tile_rect leaf, gs_bins** out,
                      int64_t* n_isect)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if (!handle_ok(ctx, proj, kMagicProj)) return gs_fail(ctx, GS_ERR_STATE, "invalid projection handle");
    if (!out || !n_isect) return gs_fail(ctx, GS_ERR_INVALID_ARG, "out / n_isect is NULL");
    if (leaf.tx0 < 0 || leaf.ty0 < 0 || leaf.tx1 > proj->TW || leaf.ty1 > proj->TH || leaf.tx0 >= leaf.tx1 ||
        leaf.ty0 >= leaf.ty1)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "leaf (%d,%d)-(%d,%d) is empty or outside the %d x %d tile grid",
                       leaf.tx0, leaf.ty0, leaf.tx1, leaf.ty1, proj->TW, proj->TH);
    gs_bins* b = new_handle<gs_bins>(ctx, kMagicBins);
    if (!b) return gs_fail(ctx, GS_ERR_OOM, "host allocation failed");
    b->proj = proj;
    b->leaf = leaf;
    b->TWL = leaf.tx1 - leaf.tx0;
    b->THL = leaf.ty1 - leaf.ty0;
    b->n_tiles = (int64_t)b->TWL * b->THL;
    std::vector<GsAlloc> tmp;
    uint64_t I = 0, C = 0;
    bool second = false;
    const int64_t n_super = super_cells(leaf);
    if (n_super >= super_cells_max()) {
        destroy_handle(ctx, b);
        return gs_fail(ctx, GS_ERR_OVERFLOW, "leaf meets %lld super-tiles (limit %lld)", (long long)n_super,
                       (long long)super_cells_max());
    }
    uint32_t *cnt = nullptr, *lc = nullptr, *k0 = nullptr, *k1 = nullptr, *v0 = nullptr, *v1 = nullptr;
    uint32_t* eoff_own = nullptr;
    uint32_t* rsc = nullptr;
    uint64_t* soff = nullptr;
    const PlanLeaf pl = plan_leaf(proj, leaf);
    const uint32_t* list = pl.found ? pl.list : nullptr;   // depth positions; not planned: every candidate
    if ((st = rect_d_ready(ctx, proj)) != GS_OK) {
        destroy_handle(ctx, b);
        return st;
    }
    const int64_t n_list = pl.found ? pl.n : proj->n_cand;
    const uint32_t* eoff = pl.eoff;
    const uint32_t ebase = pl.ebase;
    if (pl.found) {
        b->offsets = pl.toff;      // the plan's memory (kept until the projection is released)
        b->order = pl.order;
        C = (uint64_t)pl.cells;
    } else {
        if ((st = ensure_tile_counts(ctx, const_cast<gs_proj*>(proj))) != GS_OK) goto fail;
        // tile offsets: exclusive scan of the leaf's per-tile counts
        b->offsets = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (b->n_tiles + 1), GS_MEM_RASTER, &b->allocs);
        lc = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * b->n_tiles, GS_MEM_RASTER, &tmp);
        if (!b->offsets || !lc) { st = GS_ERR_OOM; goto fail; }
        if ((st = launch_leaf_counts(ctx, proj, leaf, lc)) != GS_OK) goto fail;
        if ((st = launch_scan_u32_to_u64(ctx, lc, b->offsets, b->n_tiles)) != GS_OK) goto fail;
        gs_free_one(ctx, &tmp, lc);
        // coarse pair offsets of the listed candidates
        cnt = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<int64_t>(n_list, 1), GS_MEM_RASTER, &tmp);
        eoff_own = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * (n_list + 1), GS_MEM_RASTER, &tmp);
        if (!cnt || !eoff_own) { st = GS_ERR_OOM; goto fail; }
        if ((st = launch_count_cells(ctx, proj, leaf, list, n_list, cnt)) != GS_OK) goto fail;
        if ((st = launch_scan_u32_to_u32(ctx, cnt, eoff_own, n_list)) != GS_OK) goto fail;
        gs_free_one(ctx, &tmp, cnt);   // stream-ordered: the scan has consumed it
        eoff = eoff_own;
        uint32_t hc = 0;
        if ((st = readback(ctx, eoff_own + n_list, sizeof(uint32_t), &hc)) != GS_OK) goto fail;
        C = hc;
    }
    if (pl.found && pl.isect >= 0) {
        I = (uint64_t)pl.isect;    // read back with the plan: no synchronisation here
    } else if ((st = readback(ctx, b->offsets + b->n_tiles, sizeof(uint64_t), &I)) != GS_OK) {
        goto fail;
    }
    if (I >= (1ull << 32) || C >= (1ull << 32)) {
        st = gs_fail(ctx, GS_ERR_OVERFLOW, "leaf has %llu intersections / %llu super-tile pairs (limit 2^32)",
                     (unsigned long long)I, (unsigned long long)C);
        goto fail;
    }
    b->n_isect = (int64_t)I;
    {
        const uint64_t nc = std::max<uint64_t>(C, 1);
        k0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_RASTER, &tmp);
        v0 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_RASTER, &tmp);
        // the sort's histogram, and before it the emission's block starts
        rsc = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * radix_scratch_words((int64_t)C), GS_MEM_SCRATCH, &tmp);
        if (!k0 || !v0 || !rsc) { st = GS_ERR_OOM; goto fail; }
    }
    if ((st = launch_emit_cells(ctx, proj, leaf, list, n_list, eoff, ebase, C, k0, v0, rsc)) != GS_OK) goto fail;
    if (eoff_own) gs_free_one(ctx, &tmp, eoff_own);
    {
        const uint64_t nc = std::max<uint64_t>(C, 1);
        k1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_RASTER, &tmp);
        v1 = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * nc, GS_MEM_RASTER, &tmp);
        if (!k1 || !v1) { st = GS_ERR_OOM; goto fail; }
    }
    soff = (uint64_t*)gs_malloc(ctx, sizeof(uint64_t) * (n_super + 1), GS_MEM_RASTER, &tmp);
    if (!soff) { st = GS_ERR_OOM; goto fail; }
    {
        // a single-pass sort writes the super-tile group offsets itself
        bool have_soff = false;
        if ((st = launch_radix_sort(ctx, k0, v0, k1, v1, (int64_t)C, bits_for(n_super), &second, soff, n_super,
                                    &have_soff, rsc)) != GS_OK)
            goto fail;
        if (!have_soff &&
            (st = launch_seg_offsets(ctx, second ? k1 : k0, (int64_t)C, n_super, super_key_mask(), soff)) != GS_OK)
            goto fail;
    }
    gs_free_one(ctx, &tmp, second ? k0 : k1);     // the sorted keys stay for the fine level
    gs_free_one(ctx, &tmp, second ? v0 : v1);
    // fine level: per-tile lists at the tile offsets
    {
        const int64_t items = fine_items_bound(leaf, C);
        b->values = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * std::max<uint64_t>(I, 1), GS_MEM_RASTER, &b->allocs);
        uint32_t* item_sc = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * items, GS_MEM_RASTER, &tmp);
        uint32_t* ioff = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * (n_super + 1), GS_MEM_RASTER, &tmp);
        uint32_t* pos = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * 64 * items, GS_MEM_RASTER, &tmp);
        if (!b->values || !item_sc || !ioff || !pos) { st = GS_ERR_OOM; goto fail; }
        if ((st = launch_fine_lists(ctx, proj, leaf, soff, second ? v1 : v0, second ? k1 : k0, C, b->offsets, item_sc,
                                    ioff, pos, I, b->values)) != GS_OK)
            goto fail;
    }
    gs_free_all(ctx, &tmp);
    *out = b;
    *n_isect = b->n_isect;
    return GS_OK;
fail:
    gs_free_all(ctx, &tmp);
    destroy_handle(ctx, b);
    return st;
}

// ---------------------------------------------------------------------------
// raster

// gs_render_fwd with an optional caller-owned destination for the per-tile
// L1 partials (l1_dst, 4 doubles per tile of the leaf): then the partials are
// left there for the caller to sum once for several leaves, and loss_accum is
// not touched; target and image_out may be slices (frames tf, imf).
static gs_status render_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                            const float* target, PixFrame tf, double* loss_accum, float* image_out, PixFrame imf,
                            uint64_t* stats, double* l1_dst, gs_raster** out)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if (!handle_ok(ctx, proj, kMagicProj)) return gs_fail(ctx, GS_ERR_STATE, "invalid projection handle");
    if (!handle_ok(ctx, bins, kMagicBins) || bins->proj != proj)
        return gs_fail(ctx, GS_ERR_STATE, "bins handle does not belong to this projection");
    if (!out) return gs_fail(ctx, GS_ERR_INVALID_ARG, "out is NULL");
    if (proj->W != cam->width || proj->H != cam->height)
        return gs_fail(ctx, GS_ERR_STATE, "camera does not match the projection");
    gs_raster* r = new_handle<gs_raster>(ctx, kMagicRaster);
    if (!r) return gs_fail(ctx, GS_ERR_OOM, "host allocation failed");
    r->bins = bins;
    r->px0 = bins->leaf.tx0 * 16;
    r->py0 = bins->leaf.ty0 * 16;
    r->WL = std::min(bins->leaf.tx1 * 16, cam->width) - r->px0;
    r->HL = std::min(bins->leaf.ty1 * 16, cam->height) - r->py0;
    r->n_pix = (int64_t)r->WL * r->HL;
    r->tfinal = (float*)gs_malloc(ctx, sizeof(float) * r->n_pix, GS_MEM_RASTER, &r->allocs);
    r->last = (uint32_t*)gs_malloc(ctx, sizeof(uint32_t) * r->n_pix, GS_MEM_RASTER, &r->allocs);
    if (target) {
        r->sgn = (uint8_t*)gs_malloc(ctx, r->n_pix, GS_MEM_RASTER, &r->allocs);
        r->l1_part = l1_dst ? l1_dst
                            : (double*)gs_malloc(ctx, sizeof(double) * 4 * bins->n_tiles, GS_MEM_RASTER, &r->allocs);
    }
    if (!r->tfinal || !r->last || (target && (!r->sgn || !r->l1_part))) {
        destroy_handle(ctx, r);
        return GS_ERR_OOM;
    }
    if ((st = launch_raster_fwd(ctx, cam, proj, bins, r, target, tf, image_out, imf, l1_dst ? nullptr : loss_accum,
                                stats)) != GS_OK) {
        destroy_handle(ctx, r);
        return st;
    }
    *out = r;
    return GS_OK;
}

gs_status gs_render_fwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                        const float* target, double* loss_accum, float* image_out, uint64_t* stats,
                        gs_raster** out)
{
    const PixFrame f = full_frame(cam->width, cam->height);
    return render_fwd(ctx, cam, proj, bins, target, f, loss_accum, image_out, f, stats, nullptr, out);
}

gs_status gs_render_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const gs_bins* bins,
                        const gs_raster* raster, const float* dl_dimage, float* grad2d)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if (!handle_ok(ctx, proj, kMagicProj) || !handle_ok(ctx, bins, kMagicBins) ||
        !handle_ok(ctx, raster, kMagicRaster) || bins->proj != proj || raster->bins != bins)
        return gs_fail(ctx, GS_ERR_STATE, "handles do not belong together");
    if (!grad2d && proj->n_cand > 0) return gs_fail(ctx, GS_ERR_INVALID_ARG, "grad2d is NULL");
    if (!dl_dimage && !raster->sgn)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "no dL/dimage given and no L1 target fused in the forward");
    return launch_raster_bwd(ctx, cam, proj, bins, raster, dl_dimage, full_frame(cam->width, cam->height), grad2d);
}

gs_status gs_project_bwd(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, const gs_proj* proj,
                         const float* grad2d, float* grad3d)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    gs_status st;
    if ((st = check_camera(ctx, cam)) != GS_OK) return st;
    if ((st = check_params(ctx, params)) != GS_OK) return st;
    if (!handle_ok(ctx, proj, kMagicProj)) return gs_fail(ctx, GS_ERR_STATE, "invalid projection handle");
    if (params->n != proj->n || params->sh_degree != proj->sh_degree)
        return gs_fail(ctx, GS_ERR_STATE, "params do not match the projection");
    if (proj->n_cand > 0 && (!grad2d || !grad3d)) return gs_fail(ctx, GS_ERR_INVALID_ARG, "grad2d / grad3d NULL");
    return launch_project_bwd(ctx, cam, params, proj, grad2d, 0, proj->n_cand, grad3d);
}

// ---------------------------------------------------------------------------
// extras

gs_status gs_loss_ssim(gs_ctx* ctx, int32_t width, int32_t height, const float* image, const float* target,
                       float lambda, float* dl_dimage, double* loss, double* ssim)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (width < 1 || height < 1 || !image || !target || !dl_dimage)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "gs_loss_ssim arguments");
    const int64_t P = (int64_t)width * height;
    const int64_t nb = ssim_partial_blocks(width, height);
    std::vector<GsAlloc> tmp;
    float* scratch = (float*)gs_malloc(ctx, sizeof(float) * 9 * P, GS_MEM_LOSS, &tmp);
    double* part = (double*)gs_malloc(ctx, sizeof(double) * (2 * nb + 2), GS_MEM_LOSS, &tmp);
    if (!scratch || !part) {
        gs_free_all(ctx, &tmp);
        return GS_ERR_OOM;
    }
    gs_status st = launch_ssim(ctx, width, height, 0, 0, width, height, (float)(1.0 / (3.0 * (double)P)), image,
                               target, lambda, dl_dimage, part, nb, scratch);
    if (st == GS_OK && (loss || ssim)) {
        st = launch_sum_f64(ctx, part, nb, 2, part + 2 * nb, 0);
        if (st == GS_OK) st = launch_sum_f64(ctx, part + 1, nb, 2, part + 2 * nb + 1, 0);
        double hv[2] = {0, 0};
        if (st == GS_OK) st = readback(ctx, part + 2 * nb, sizeof(hv), hv);
        if (st == GS_OK) {
            const double s = hv[0] / (3.0 * (double)P), l1 = hv[1] / (3.0 * (double)P);
            if (ssim) *ssim = s;
            if (loss) *loss = (1.0 - lambda) * l1 + lambda * (1.0 - s);
        }
    }
    gs_free_all(ctx, &tmp);
    return st;
}

gs_status gs_loss_ssim_static(gs_ctx* ctx, int32_t width, int32_t height, const float* image, const float* target,
                              float lambda, float* dl_dimage, double* loss, double* ssim)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (width < 1 || height < 1 || !image || !target || !dl_dimage)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "gs_loss_ssim_static arguments");
    SsimStatic sb;
    gs_status st = ssim_static_buffers(ctx, width, height, &sb);
    if (st != GS_OK) return st;
    const int64_t P = (int64_t)width * height;
    const int64_t nb = ssim_partial_blocks(width, height);
    // every map and block sum is written before it is read in this call
    st = launch_ssim(ctx, width, height, 0, 0, width, height, (float)(1.0 / (3.0 * (double)P)), image, target, lambda,
                     dl_dimage, sb.part, nb, sb.maps);
    if (st == GS_OK && (loss || ssim)) {
        st = launch_sum_f64(ctx, sb.part, nb, 2, sb.sums, 0, sb.chunk);
        if (st == GS_OK) st = launch_sum_f64(ctx, sb.part + 1, nb, 2, sb.sums + 1, 0, sb.chunk);
        double hv[2] = {0, 0};
        if (st == GS_OK) st = readback(ctx, sb.sums, sizeof(hv), hv);
        if (st == GS_OK) {
            const double s = hv[0] / (3.0 * (double)P), l1 = hv[1] / (3.0 * (double)P);
            if (ssim) *ssim = s;
            if (loss) *loss = (1.0 - lambda) * l1 + lambda * (1.0 - s);
        }
    }
    return st;
}

gs_status gs_adam_step(gs_ctx* ctx, const gs_proj* proj, int64_t n, int32_t sh_degree, const gs_param_ptrs* params,
                       const gs_param_ptrs* m, const gs_param_ptrs* v, const float* grad3d, int32_t step, float lr,
                       float beta1, float beta2, float eps)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (!handle_ok(ctx, proj, kMagicProj)) return gs_fail(ctx, GS_ERR_STATE, "invalid projection handle");
    if (n != proj->n || sh_degree != proj->sh_degree) return gs_fail(ctx, GS_ERR_STATE, "sizes do not match");
    if (!params || !m || !v || step < 1 || (proj->n_cand > 0 && !grad3d))
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "gs_adam_step arguments");
    return launch_adam(ctx, proj, n, sh_degree, params, m, v, grad3d, 0, proj->n_cand, step, lr, beta1, beta2, eps);
}

void gs_release(gs_ctx* ctx, void* handle)
{
    if (!ctx || !handle) return;
    GsHandle* h = static_cast<GsHandle*>(handle);
    if (h->ctx != ctx || (h->magic != kMagicProj && h->magic != kMagicBins && h->magic != kMagicRaster)) return;
    destroy_handle(ctx, h);
}

gs_status gs_export_size(gs_ctx* ctx, const void* handle, int32_t field, size_t* bytes)
{
    if (!ctx || !handle || !bytes) return GS_ERR_INVALID_ARG;
    const GsHandle* h = static_cast<const GsHandle*>(handle);
    if (h->ctx != ctx) return gs_fail(ctx, GS_ERR_STATE, "handle of another context");
    if (h->magic == kMagicProj) {
        const gs_proj* p = static_cast<const gs_proj*>(h);
        const size_t nc = (size_t)p->n_cand;
        switch (field) {
        case GS_PROJ_IDS: case GS_PROJ_DEPTH: case GS_PROJ_RADIUS: case GS_PROJ_OPACITY: case GS_PROJ_FLAGS:
            *bytes = 4 * nc; return GS_OK;
        case GS_PROJ_RECT: *bytes = 16 * nc; return GS_OK;
        case GS_PROJ_XY: *bytes = 8 * nc; return GS_OK;
        case GS_PROJ_CONIC: case GS_PROJ_RGB: *bytes = 12 * nc; return GS_OK;
        case GS_PROJ_SLOT_OF: *bytes = 4 * (size_t)p->n; return GS_OK;
        default: break;
        }
    } else if (h->magic == kMagicBins) {
        const gs_bins* b = static_cast<const gs_bins*>(h);
        switch (field) {
        case GS_BINS_OFFSETS: *bytes = 8 * (size_t)(b->n_tiles + 1); return GS_OK;
        case GS_BINS_VALUES: *bytes = 4 * (size_t)b->n_isect; return GS_OK;
        case GS_BINS_KEYS: *bytes = 8 * (size_t)b->n_isect; return GS_OK;
        default: break;
        }
    } else if (h->magic == kMagicRaster) {
        const gs_raster* r = static_cast<const gs_raster*>(h);
        if (field == GS_RASTER_TFINAL || field == GS_RASTER_LAST) {
            *bytes = 4 * (size_t)r->n_pix;
            return GS_OK;
        }
    }
    return gs_fail(ctx, GS_ERR_INVALID_ARG, "field %d does not belong to this handle", field);
}

gs_status gs_export(gs_ctx* ctx, const void* handle, int32_t field, void* dst, size_t dst_bytes)
{
    size_t need = 0;
    gs_status st = gs_export_size(ctx, handle, field, &need);
    if (st != GS_OK) return st;
    if (need == 0) return GS_OK;
    if (!dst || dst_bytes < need) return gs_fail(ctx, GS_ERR_INVALID_ARG, "destination too small (%zu < %zu)", dst_bytes, need);
    const GsHandle* h = static_cast<const GsHandle*>(handle);
    if (h->magic == kMagicProj) return launch_export_proj(ctx, static_cast<const gs_proj*>(h), field, dst);
    if (h->magic == kMagicBins) {
        const gs_bins* b = static_cast<const gs_bins*>(h);
        if (field == GS_BINS_KEYS) return launch_export_keys(ctx, b, (uint64_t*)dst);
        const void* src = field == GS_BINS_OFFSETS ? (const void*)b->offsets : (const void*)b->values;
        GS_HIP(ctx, hipMemcpyAsync(dst, src, need, hipMemcpyDeviceToDevice, ctx->stream));
        return GS_OK;
    }
    const gs_raster* r = static_cast<const gs_raster*>(h);
    const void* src = field == GS_RASTER_TFINAL ? (const void*)r->tfinal : (const void*)r->last;
    GS_HIP(ctx, hipMemcpyAsync(dst, src, need, hipMemcpyDeviceToDevice, ctx->stream));
    return GS_OK;
}

gs_status gs_util_exp(gs_ctx* ctx, const float* x, float* y, int64_t n)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (n < 0 || (n > 0 && (!x || !y))) return gs_fail(ctx, GS_ERR_INVALID_ARG, "gs_util_exp arguments");
    return launch_exp(ctx, x, y, n, false);
}

gs_status gs_util_exp_falloff(gs_ctx* ctx, const float* x, float* y, int64_t n)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (n < 0 || (n > 0 && (!x || !y))) return gs_fail(ctx, GS_ERR_INVALID_ARG, "gs_util_exp_falloff arguments");
    return launch_exp(ctx, x, y, n, true);
}

// ---------------------------------------------------------------------------
// one whole view

}  // extern "C"

// A device copy of the target over one pixel rectangle (a leaf's, or a
// leaf's with its SSIM halo), and the frame it is read through.
struct TargetSlice {
    float* ptr = nullptr;
    PixFrame f{};
    std::vector<GsAlloc> allocs;
};

// The pixel rectangle [x0, x0 + w) x [y0, y0 + h) of a tile rectangle,
// clipped to the image.
struct PixRect {
    int x0, y0, w, h;
};
static PixRect pix_rect(const gs_camera* cam, gs_tile_rect r)
{
    PixRect p;
    p.x0 = r.tx0 * 16;
    p.y0 = r.ty0 * 16;
    p.w = std::min(r.tx1 * 16, cam->width) - p.x0;
    p.h = std::min(r.ty1 * 16, cam->height) - p.y0;
    return p;
}

// Allocates (on the main stream) a slice for rectangle pr and copies the
// target's pixels there on stream s: from host memory (host != 0) or from the
// device-resident image.  The three channel planes are one 2D copy each.
static gs_status slice_target(gs_ctx* ctx, const gs_camera* cam, const float* target, bool host, PixRect pr,
                              TargetSlice* sl, hipStream_t s)
{
    const int64_t P = (int64_t)cam->width * cam->height, n = (int64_t)pr.w * pr.h;
    sl->ptr = (float*)gs_malloc(ctx, sizeof(float) * 3 * n, GS_MEM_LOSS, &sl->allocs);
    if (!sl->ptr) return GS_ERR_OOM;
    sl->f = PixFrame{pr.x0, pr.y0, pr.w, n};
    if (s != ctx->stream) {
        GS_HIP(ctx, hipEventRecord(ctx->ev_alloc, ctx->stream));
        GS_HIP(ctx, hipStreamWaitEvent(s, ctx->ev_alloc, 0));
    }
    for (int c = 0; c < 3; ++c)
        GS_HIP(ctx, hipMemcpy2DAsync(sl->ptr + c * n, sizeof(float) * pr.w,
                                     target + c * P + (int64_t)pr.y0 * cam->width + pr.x0,
                                     sizeof(float) * cam->width, sizeof(float) * pr.w, pr.h,
                                     host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice, s));
    return GS_OK;
}

// One leaf of an SSIM view: its tile rectangle grown by one tile (16 pixels,
// at least the 10 the 11 x 11 windows of its pixels' gradients reach) on each
// side inside the grid is binned and rendered into a buffer of that size;
// the SSIM terms of the centres inside the leaf and the gradient of its
// pixels are exactly the whole image's (see loss.hip); the raster backward
// runs with that gradient (zero on the halo).  The sums of S and |x - y|
// over the leaf are added to acc[0], acc[1]; the leaf's pixels of the image
// go to image_out when given.  `given`: the target over the grown
// rectangle, already copied (else it is sliced here when needed).
static gs_tile_rect ssim_grown(const gs_proj* proj, gs_tile_rect r)
{
    return gs_tile_rect{std::max(r.tx0 - 1, 0), std::max(r.ty0 - 1, 0), std::min(r.tx1 + 1, proj->TW),
                        std::min(r.ty1 + 1, proj->TH)};
}

static gs_status ssim_leaf(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const float* target,
                           bool target_host, const TargetSlice* given, const gs_view_opts* opts, gs_tile_rect r,
                           bool backward, float* grad2d, float* image_out, double* acc, int64_t* ni)
{
    gs_status st = GS_OK;
    const gs_tile_rect e = ssim_grown(proj, r);
    const PixRect ep = pix_rect(cam, e), op = pix_rect(cam, r);
    const int64_t n = (int64_t)ep.w * ep.h, P = (int64_t)cam->width * cam->height;
    const bool whole = ep.w == cam->width && ep.h == cam->height;
    const PixFrame ef{ep.x0, ep.y0, ep.w, n};
    gs_bins* bins = nullptr;
    gs_raster* ras = nullptr;
    TargetSlice ts;
    std::vector<GsAlloc> tmp;
    const float* tgt = target;
    float* image = whole && image_out ? image_out : nullptr;
    float* dl = nullptr;
    float* scratch = nullptr;
    double* part = nullptr;
    const int64_t nb = ssim_partial_blocks(ep.w, ep.h);
    if ((st = gs_bin_sort(ctx, cam, proj, e, &bins, ni)) != GS_OK) return st;
    if (given) {
        tgt = given->ptr;
    } else if (!whole || target_host) {
        if ((st = slice_target(ctx, cam, target, target_host, ep, &ts, ctx->stream)) != GS_OK) goto done;
        tgt = ts.ptr;
    }
    if (!image) image = (float*)gs_malloc(ctx, sizeof(float) * 3 * n, GS_MEM_LOSS, &tmp);
    dl = (float*)gs_malloc(ctx, sizeof(float) * 3 * n, GS_MEM_LOSS, &tmp);
    scratch = (float*)gs_malloc(ctx, sizeof(float) * 9 * n, GS_MEM_LOSS, &tmp);
    part = (double*)gs_malloc(ctx, sizeof(double) * 2 * nb, GS_MEM_LOSS, &tmp);
    if (!image || !dl || !scratch || !part) { st = GS_ERR_OOM; goto done; }
    if ((st = render_fwd(ctx, cam, proj, bins, nullptr, ef, nullptr, image, ef, nullptr, nullptr, &ras)) != GS_OK)
        goto done;
    if ((st = launch_ssim(ctx, ep.w, ep.h, op.x0 - ep.x0, op.y0 - ep.y0, op.x0 - ep.x0 + op.w, op.y0 - ep.y0 + op.h,
                          (float)(1.0 / (3.0 * (double)P)), image, tgt, opts->ssim_lambda, dl, part, nb, scratch)) !=
        GS_OK)
        goto done;
    if ((st = launch_sum_f64(ctx, part, nb, 2, acc, 1)) != GS_OK) goto done;
    if ((st = launch_sum_f64(ctx, part + 1, nb, 2, acc + 1, 1)) != GS_OK) goto done;
    if (backward && (st = launch_raster_bwd(ctx, cam, proj, bins, ras, dl, ef, grad2d)) != GS_OK) goto done;
    if (image_out && image != image_out)
        for (int c = 0; c < 3; ++c)
            if (hipMemcpy2DAsync(image_out + c * P + (int64_t)op.y0 * cam->width + op.x0, sizeof(float) * cam->width,
                                 image + c * n + (int64_t)(op.y0 - ep.y0) * ep.w + (op.x0 - ep.x0),
                                 sizeof(float) * ep.w, sizeof(float) * op.w, op.h, hipMemcpyDeviceToDevice,
                                 ctx->stream) != hipSuccess) {
                st = gs_fail(ctx, GS_ERR_DEVICE, "image copy failed");
                goto done;
            }
done:
    gs_release(ctx, ras);
    gs_release(ctx, bins);
    gs_free_all(ctx, &tmp);
    gs_free_all(ctx, &ts.allocs);
    return st;
}

// The leaves of one view: binning (the next leaf's on a second stream while
// the current one is rendered, when every leaf is planned and not every
// kernel is timed), then per leaf the fused forward + L1 (+ backward when
// `backward`), or for the SSIM loss the forward over the leaf with a halo,
// the loss and (when `backward`) the raster backward.  L1 partials go to
// l1_view (4 per tile, leaves side by side); SSIM sums are added to
// ssim_acc[0..1]; 2D gradients are added to grad2d.  A host target is copied
// leaf by leaf (for a binned-ahead leaf on the second stream, before its
// binning), each slice freed once its leaf's raster has ended.
static gs_status render_leaves(gs_ctx* ctx, const gs_camera* cam, const gs_proj* proj, const float* target,
                               const gs_view_opts* opts, const std::vector<gs_leaf>& leaves, bool backward,
                               float* grad2d, double* l1_view, float* image, double* ssim_acc, int64_t* isect_total,
                               bool walk, bool* walked)
{
    gs_status st = GS_OK;
    int64_t l1_off = 0;
    *isect_total = 0;
    const bool host = opts->target_host != 0;
    const PixFrame full = full_frame(cam->width, cam->height);
    CoarseBins cbs[3];   // leaf li uses cbs[li % 3]
    TargetSlice sl[3];   // leaf li uses sl[li % 3]
    int inflight[2] = {-1, -1};   // leaves on the render streams (their cbs and slices are held)
    // L1 views of planned leaves whose coverage calls for it (walk_rule):
    // the fused raster walks each leaf's super-tile groups (no per-tile
    // lists); overlapped unless every kernel is timed or there is a single
    // leaf
    bool groups = opts->loss_kind == 0 && walk;
    for (const gs_leaf& L : leaves)
        groups = groups && leaf_pipelinable(proj, gs_tile_rect{L.tx0, L.ty0, L.tx1, L.ty1});
    const bool pipe = groups && leaves.size() > 1 && !(ctx->timing && ctx->timing_only.empty());
    *walked = groups;
    if (opts->loss_kind == 1) {
        // a host target: each next leaf's slice is copied on the second
        // stream while the current leaf is rendered
        if ((st = launch_fill_u32(ctx, (uint32_t*)ssim_acc, 0u, 4)) != GS_OK) return st;
        auto grown = [&](size_t li) {
            const gs_leaf& L = leaves[li];
            return pix_rect(cam, ssim_grown(proj, gs_tile_rect{L.tx0, L.ty0, L.tx1, L.ty1}));
        };
        if (host) {
            if ((st = ensure_side(ctx)) != GS_OK) return st;
            LeafTag tag(ctx, 0);
            if ((st = slice_target(ctx, cam, target, true, grown(0), &sl[0], ctx->side)) == GS_OK &&
                hipEventRecord(ctx->ev_done[0], ctx->side) != hipSuccess)
                st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
        }
        for (size_t li = 0; li < leaves.size() && st == GS_OK; ++li) {
            const gs_leaf& L = leaves[li];
            int64_t ni = 0;
            if (host) {
                if (hipStreamWaitEvent(ctx->stream, ctx->ev_done[li & 1], 0) != hipSuccess) {
                    st = gs_fail(ctx, GS_ERR_DEVICE, "stream wait failed");
                    break;
                }
                if (li + 1 < leaves.size()) {
                    LeafTag tag(ctx, (int32_t)li + 1);
                    if ((st = slice_target(ctx, cam, target, true, grown(li + 1), &sl[(li + 1) % 3], ctx->side)) !=
                        GS_OK)
                        break;
                    if (hipEventRecord(ctx->ev_done[(li + 1) & 1], ctx->side) != hipSuccess) {
                        st = gs_fail(ctx, GS_ERR_DEVICE, "event record failed");
                        break;
                    }
                }
            }
            {
                LeafTag tag(ctx, (int32_t)li);
                st = ssim_leaf(ctx, cam, proj, target, host, host ? &sl[li % 3] : nullptr, opts,
                               gs_tile_rect{L.tx0, L.ty0, L.tx1, L.ty1}, backward, grad2d, image, ssim_acc, &ni);
            }
            *isect_total += ni;
            gs_free_all(ctx, &sl[li % 3].allocs);
        }
        if (host) (void)hipStreamSynchronize(ctx->side);
        for (TargetSlice& t : sl) gs_free_all(ctx, &t.allocs);
        return st;
    }
    if (pipe) {
        const gs_leaf& L = leaves[0];
        if ((st = ensure_side(ctx)) != GS_OK) return st;
        LeafTag tag(ctx, 0);
        if (host && (st = slice_target(ctx, cam, target, true, pix_rect(cam, gs_tile_rect{L.tx0, L.ty0, L.tx1, L.ty1}),
                                       &sl[0], ctx->side)) != GS_OK)
            goto done;
        if ((st = coarse_alloc(ctx, proj, gs_tile_rect{L.tx0, L.ty0, L.tx1, L.ty1}, &cbs[0])) != GS_OK) goto done;
        if ((st = coarse_on_side(ctx, proj, &cbs[0], ctx->ev_done[0])) != GS_OK) goto done;
    }
    for (size_t li = 0; li < leaves.size(); ++li) {
        const gs_leaf& L = leaves[li];
        int64_t ni = 0;
        gs_tile_rect r{L.tx0, L.ty0, L.tx1, L.ty1};
        TargetSlice& ts = sl[li % 3];
        CoarseBins& cb = cbs[li % 3];
        // the next leaf's coarse stage (and its target slice) on the side
        // stream, behind everything the main stream has queued so far
        auto stage_next = [&]() -> gs_status {
            if (li + 1 >= leaves.size()) return GS_OK;
            const gs_leaf& N = leaves[li + 1];
            const gs_tile_rect nr{N.tx0, N.ty0, N.tx1, N.ty1};
            CoarseBins& nx = cbs[(li + 1) % 3];
            LeafTag tag(ctx, (int32_t)li + 1);
            gs_status s2 = GS_OK;
            if (host) s2 = slice_target(ctx, cam, target, true, pix_rect(cam, nr), &sl[(li + 1) % 3], ctx->side);
            if (s2 == GS_OK && (s2 = coarse_alloc(ctx, proj, nr, &nx)) == GS_OK)
                s2 = coarse_on_side(ctx, proj, &nx, ctx->ev_done[(li + 1) & 1]);
            return s2;
        };
        if (!groups) {
            // lists per tile (gs_bin_sort), then the fused raster on the main
            // stream
            gs_bins* bins = nullptr;
            {
                LeafTag tag(ctx, (int32_t)li);
                if ((st = gs_bin_sort(ctx, cam, proj, r, &bins, &ni)) != GS_OK) goto done;
                if (host && (st = slice_target(ctx, cam, target, true, pix_rect(cam, r), &ts, ctx->stream)) != GS_OK) {
                    gs_release(ctx, bins);
                    goto done;
                }
                *isect_total += ni;
                st = launch_raster_fused(ctx, cam, proj, bins, host ? ts.ptr : target, host ? ts.f : full, image,
                                         l1_view + l1_off, backward ? grad2d : nullptr, backward);
            }
            l1_off += 4 * (int64_t)(L.tx1 - L.tx0) * (L.ty1 - L.ty0);
            gs_release(ctx, bins);
            gs_free_all(ctx, &ts.allocs);
            if (st != GS_OK) goto done;
            continue;
        }
        if (!pipe) {
            // every stage of the leaf on the main stream, in series
            LeafTag tag(ctx, (int32_t)li);
            if ((st = coarse_alloc(ctx, proj, r, &cb)) != GS_OK) goto done;
            if ((st = coarse_launch(ctx, proj, &cb)) != GS_OK) goto done;
            if (host && (st = slice_target(ctx, cam, target, true, pix_rect(cam, r), &ts, ctx->stream)) != GS_OK)
                goto done;
        }
        ni = (int64_t)cb.I;
        *isect_total += ni;
        const float* tgt = host ? ts.ptr : target;
        const PixFrame tf = host ? ts.f : full;
        if (pipe && !opts->serial_leaves) {
            // the fused raster of this leaf on render stream li & 1 once its
            // coarse stage (side stream) is done; the previous leaf's raster
            // may still run on the other render stream, and its coarse
            // buffers (and target slice) are released on the main stream
            // only after it has ended
            const int k = (int)(li & 1);
            hipStream_t main = ctx->stream;
            if (hipStreamWaitEvent(ctx->rstream[k], ctx->ev_done[li & 1], 0) != hipSuccess) {
                st = gs_fail(ctx, GS_ERR_DEVICE, "render stream ordering failed");
                goto done;
            }
            ctx->stream = ctx->rstream[k];
            {
                LeafTag tag(ctx, (int32_t)li);
                st = launch_raster_groups(ctx, cam, proj, r, cb.soff, cb.second ? cb.v1 : cb.v0,
                                          cb.second ? cb.k1 : cb.k0, cb.pl.order, tgt, tf, image, l1_view + l1_off,
                                          backward ? grad2d : nullptr, backward);
            }
            ctx->stream = main;
            if (st == GS_OK && hipEventRecord(ctx->ev_rendered[k], ctx->rstream[k]) != hipSuccess)
                st = gs_fail(ctx, GS_ERR_DEVICE, "render event failed");
            l1_off += 4 * (int64_t)(L.tx1 - L.tx0) * (L.ty1 - L.ty0);
            inflight[k] = (int)li;
            if (st != GS_OK) goto done;
            if ((st = stage_next()) != GS_OK) goto done;
            if (li >= 1 && inflight[k ^ 1] >= 0) {
                if (hipStreamWaitEvent(main, ctx->ev_rendered[k ^ 1], 0) != hipSuccess) {
                    st = gs_fail(ctx, GS_ERR_DEVICE, "render stream wait failed");
                    goto done;
                }
                gs_free_all(ctx, &cbs[inflight[k ^ 1] % 3].allocs);
                gs_free_all(ctx, &sl[inflight[k ^ 1] % 3].allocs);
                inflight[k ^ 1] = -1;
            }
            continue;
        }
        if (pipe) {
            // one leaf at a time on the main stream: this leaf's coarse
            // stage is done on the side stream, and the next leaf's is queued
            // before this raster, so that it runs beside it
            if (hipStreamWaitEvent(ctx->stream, ctx->ev_done[li & 1], 0) != hipSuccess) {
                st = gs_fail(ctx, GS_ERR_DEVICE, "stream wait failed");
                goto done;
            }
            if ((st = stage_next()) != GS_OK) goto done;
        }
        {
            LeafTag tag(ctx, (int32_t)li);
            st = launch_raster_groups(ctx, cam, proj, r, cb.soff, cb.second ? cb.v1 : cb.v0, cb.second ? cb.k1 : cb.k0,
                                      cb.pl.order, tgt, tf, image, l1_view + l1_off, backward ? grad2d : nullptr,
                                      backward);
        }
        l1_off += 4 * (int64_t)(L.tx1 - L.tx0) * (L.ty1 - L.ty0);
        gs_free_all(ctx, &cb.allocs);   // stream-ordered after the raster
        gs_free_all(ctx, &ts.allocs);
        if (st != GS_OK) goto done;
    }
done:
    if (pipe) {
        // the main stream follows the render streams before the last leaves'
        // buffers are released; nothing may be freed while the side stream
        // could still use it
        for (int k = 0; k < 2; ++k)
            if (inflight[k] >= 0 && hipStreamWaitEvent(ctx->stream, ctx->ev_rendered[k], 0) != hipSuccess) {
                (void)hipStreamSynchronize(ctx->rstream[k]);
                if (st == GS_OK) st = gs_fail(ctx, GS_ERR_DEVICE, "render stream wait failed");
            }
        (void)hipStreamSynchronize(ctx->side);
    }
    for (CoarseBins& c : cbs) gs_free_all(ctx, &c.allocs);
    for (TargetSlice& t : sl) gs_free_all(ctx, &t.allocs);
    return st;
}

// The view's loss: L1 from the per-tile partials (one sum, one read-back);
// L1 + SSIM from the sums of |x - y| and S over the leaves (ssim_acc).
static gs_status view_loss(gs_ctx* ctx, const gs_view_opts* opts, double* l1_view, int64_t l1_n, double* loss_dev,
                           const double* ssim_acc, int64_t P, double* loss, double* sum_chunks)
{
    gs_status st;
    if (opts->loss_kind == 0) {
        double s = 0.0;
        // the sum adds into loss_dev: start from zero (a gated view sums twice)
        if ((st = launch_fill_u32(ctx, (uint32_t*)loss_dev, 0u, 2)) != GS_OK) return st;
        if (l1_n > 0 && (st = launch_sum_f64(ctx, l1_view, l1_n, 1, loss_dev, 1, sum_chunks)) != GS_OK) return st;
        if (opts->loss_out) {
            // left on the device: the caller reads it when it needs it
            *loss = std::numeric_limits<double>::quiet_NaN();
            return launch_view_loss(ctx, 0, loss_dev, P, opts->ssim_lambda, opts->loss_out);
        }
        if ((st = readback(ctx, loss_dev, sizeof(double), &s)) != GS_OK) return st;
        *loss = s / (3.0 * (double)P);
    } else if (opts->loss_out) {
        *loss = std::numeric_limits<double>::quiet_NaN();
        return launch_view_loss(ctx, 1, ssim_acc, P, opts->ssim_lambda, opts->loss_out);
    } else {
        double hv[2] = {0.0, 0.0};
        if ((st = readback(ctx, ssim_acc, sizeof(hv), hv)) != GS_OK) return st;
        const double ssim = hv[0] / (3.0 * (double)P), l1 = hv[1] / (3.0 * (double)P);
        *loss = (1.0 - opts->ssim_lambda) * l1 + opts->ssim_lambda * (1.0 - ssim);
    }
    return GS_OK;
}

extern "C" {

// Which raster an L1 view of planned leaves takes.  Walking the super-tile
// groups visits, per tile, the entries of its super-tile's group; a tile's
// own list holds the fraction of them that covers it, I / (64 Cb) on average
// over the view (I intersections, Cb (candidate, super-cell) pairs).  When
// that coverage is at least 0.18 the walk pays for the per-tile lists it
// saves; below it the lists are built (gs_bin_sort) and walked.
static bool walk_rule(uint64_t I, uint64_t Cb) { return 100 * I >= 1152 * Cb; }

gs_status gs_train_view(gs_ctx* ctx, const gs_camera* cam, const gs_params* params, const float* target,
                        const gs_view_opts* opts, gs_view_result* result)
{
    if (!ctx) return GS_ERR_INVALID_ARG;
    if (!opts || !result || !target) return gs_fail(ctx, GS_ERR_INVALID_ARG, "opts / result / target is NULL");
    if (opts->loss_kind != 0 && opts->loss_kind != 1) return gs_fail(ctx, GS_ERR_INVALID_ARG, "loss_kind");
    if (opts->adam_step > 0 && (!opts->params_rw || !opts->adam_m || !opts->adam_v))
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "Adam needs params_rw, adam_m, adam_v");
    if (opts->gate && opts->loss_out)
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "a gated view needs its loss on the host (loss_out must be NULL)");
    std::memset(result, 0, sizeof(*result));
    gs_status st;
    gs_proj* proj = nullptr;
    int64_t n_cand = 0;
    const uint64_t live0 = ctx->live;
    const uint64_t peak_before = ctx->peak;
    ctx->peak = ctx->live;
    if ((st = gs_project(ctx, cam, params, &proj, &n_cand)) != GS_OK) return st;

    std::vector<gs_leaf> leaves;
    const int32_t TW = proj->TW, TH = proj->TH;
    bool walk = false;   // L1: the leaves' rasters walk their super-tile groups
    bool walk_used = false;
    if (opts->budget_bytes > 0 || opts->n_leaves_in > 0) {
        // a fresh plan, the re-check of the caller's cached layout, or (budget
        // 0) the caller's layout as it is
        const gs_leaf* roots = opts->n_leaves_in > 0 ? opts->leaves_in : nullptr;
        const int32_t nr = opts->n_leaves_in > 0 ? opts->n_leaves_in : 0;
        const uint64_t budget = opts->budget_bytes > 0 ? opts->budget_bytes : ~0ull;
        const bool partial = nr > 0 && opts->leaves_in_partial != 0;
        // Without a caller's model: for SSIM the default one plus 18 floats
        // per pixel of a leaf (image, gradient, target slice, 9 partial
        // maps); for L1 the model of the raster the view takes (walk_rule):
        // the group-walking bound, or the per-tile-list one, plus with a
        // host target its 3-float slice.  The planner reports the view's
        // totals the rule reads; an L1 view starts from the previous view's
        // choice and is planned again only when the rule picks the other.
        const bool l1_auto = !opts->cost && opts->loss_kind == 0;
        auto model = [&](bool w) {
            gs_cost_model c = opts->cost ? *opts->cost
                                         : (opts->loss_kind == 1 || !w ? gs_default_cost_model() : gs_train_cost_model());
            if (!opts->cost) c.b_pixel += opts->loss_kind == 1 ? 18 * 4 : (opts->target_host ? 3 * 4 : 0);
            return c;
        };
        uint64_t tot[2] = {0, 0};
        int32_t nl = 0;
        auto plan = [&](bool w) {
            const gs_cost_model cm = model(w);
            leaves.resize(4096);
            gs_status s2 = plan_impl(ctx, cam, proj, budget, &cm, opts->strict_budget, roots, nr, leaves.data(),
                                     (int32_t)leaves.size(), &nl, partial, tot);
            if (s2 == GS_OK && nl > (int32_t)leaves.size()) {
                leaves.resize(nl);
                s2 = plan_impl(ctx, cam, proj, budget, &cm, opts->strict_budget, roots, nr, leaves.data(), nl, &nl,
                               partial, tot);
            }
            return s2;
        };
        walk = ctx->walk_guess;
        st = plan(walk);
        if (st == GS_OK && opts->loss_kind == 0) {
            const bool want = walk_rule(tot[0], tot[1]);
            if (l1_auto && want != walk) st = plan(want);
            walk = want;
            if (l1_auto) ctx->walk_guess = want;
        }
        if (st != GS_OK) { gs_release(ctx, proj); return st; }
        leaves.resize(nl);
    } else {
        gs_leaf L{};
        L.tx0 = 0; L.ty0 = 0; L.tx1 = TW; L.ty1 = TH;
        leaves.push_back(L);
    }
    if (opts->loss_kind == 1 && opts->n_leaves_in > 0 && opts->leaves_in_partial) {
        gs_release(ctx, proj);
        return gs_fail(ctx, GS_ERR_INVALID_ARG, "the SSIM loss needs a layout that covers the image");
    }
    if (opts->leaves_out && opts->max_leaves > 0)
        std::memcpy(opts->leaves_out, leaves.data(), sizeof(gs_leaf) * std::min<size_t>(leaves.size(), opts->max_leaves));
    // per-leaf accounting: allocations made for leaf i count in slot i
    ctx->tag_live.assign(leaves.size(), 0);
    ctx->tag_peak.assign(leaves.size(), 0);

    const int K = (params->sh_degree + 1) * (params->sh_degree + 1);
    const int F = 11 + 3 * K;
    std::vector<GsAlloc> view;
    const int64_t nc = std::max<int64_t>(n_cand, 1);
    float* grad2d = (float*)gs_malloc(ctx, sizeof(float) * 9 * nc, GS_MEM_GRAD, &view);
    // loss_dev[0]: the L1 sum; loss_dev[1..2]: the SSIM view's sums of S and
    // |x - y|
    double* loss_dev = (double*)gs_malloc(ctx, 3 * sizeof(double), GS_MEM_SCRATCH, &view);
    // the loss sum's chunk sums, allocated here so that nothing is allocated
    // once the update has started
    double* sum_chunks = (double*)gs_malloc(ctx, 256 * sizeof(double), GS_MEM_SCRATCH, &view);
    const int64_t P = (int64_t)cam->width * cam->height;
    float* image = opts->image_out;
    double loss = 0.0;
    int64_t isect_total = 0;
    // L1: the per-tile partials of every leaf side by side, summed once
    int64_t l1_n = 0;
    for (const gs_leaf& L : leaves) l1_n += 4 * (int64_t)(L.tx1 - L.tx0) * (L.ty1 - L.ty0);
    double* l1_view = opts->loss_kind == 0 && l1_n > 0
                          ? (double*)gs_malloc(ctx, sizeof(double) * l1_n, GS_MEM_LOSS, &view)
                          : nullptr;
    if (!grad2d || !loss_dev || !sum_chunks || (opts->loss_kind == 0 && l1_n > 0 && !l1_view)) {
        st = GS_ERR_OOM;
        goto done;
    }
    if ((st = launch_fill_f32(ctx, grad2d, 0.0f, 9 * nc)) != GS_OK) goto done;
    if ((st = launch_fill_u32(ctx, (uint32_t*)loss_dev, 0u, 6)) != GS_OK) goto done;
    if (opts->gate) {
        // SkipGS gate: the forward and the loss of every leaf first, the
        // decision, then (when it asks for the backward) the full pass; the
        // leaves' buffers are not kept between the passes, so a view that
        // runs its backward renders twice
        if ((st = render_leaves(ctx, cam, proj, target, opts, leaves, false, grad2d, l1_view, image, loss_dev + 1,
                                &isect_total, walk, &walk_used)) != GS_OK)
            goto done;
        if ((st = view_loss(ctx, opts, l1_view, l1_n, loss_dev, loss_dev + 1, P, &loss, sum_chunks)) != GS_OK) goto done;
        gs_gate_decision d{};
        if ((st = gs_gate_step(opts->gate, opts->gate_view, loss, &d)) != GS_OK) {
            st = gs_fail(ctx, st, "gate step (view %d, loss %g)", (int)opts->gate_view, loss);
            goto done;
        }
        result->gate_backward = d.backward;
        result->gate_forced = d.forced;
        result->gate_score = d.score;
        if (!d.backward) goto finish;
    }
    if ((st = render_leaves(ctx, cam, proj, target, opts, leaves, true, grad2d, l1_view, image, loss_dev + 1,
                            &isect_total, walk, &walk_used)) != GS_OK)
        goto done;
    if (opts->grad3d_out || opts->adam_step <= 0) {
        float* grad3d = (float*)gs_malloc(ctx, sizeof(float) * (int64_t)F * nc, GS_MEM_GRAD, &view);
        if (!grad3d) { st = GS_ERR_OOM; goto done; }
        if ((st = gs_project_bwd(ctx, cam, params, proj, grad2d, grad3d)) != GS_OK) goto done;
        if (opts->grad3d_out && (st = launch_scatter_grad3d(ctx, proj, F, grad3d, opts->grad3d_out)) != GS_OK)
            goto done;
        if (opts->adam_step > 0 &&
            (st = gs_adam_step(ctx, proj, params->n, params->sh_degree, opts->params_rw, opts->adam_m, opts->adam_v,
                               grad3d, opts->adam_step, opts->lr, opts->beta1, opts->beta2, opts->eps)) != GS_OK)
            goto done;
    } else if (opts->adam_chunk <= 0) {
        // projection backward fused with the update over all Gaussians
        if (!opts->params_rw || !opts->adam_m || !opts->adam_v) {
            st = gs_fail(ctx, GS_ERR_INVALID_ARG, "Adam parameters / moments NULL");
            goto done;
        }
        if ((st = launch_bwd_adam(ctx, cam, params, proj, grad2d, opts->params_rw, opts->adam_m, opts->adam_v,
                                  opts->adam_step, opts->lr, opts->beta1, opts->beta2, opts->eps)) != GS_OK)
            goto done;
    } else {
        // Projection backward and Adam in chunks of candidate slots: the
        // compact gradient rows of one chunk at a time, each chunk's
        // Gaussians updated right after; same result as the whole
        // [n_cand][F] buffer followed by one Adam step.
        if (!opts->params_rw || !opts->adam_m || !opts->adam_v) {
            st = gs_fail(ctx, GS_ERR_INVALID_ARG, "Adam parameters / moments NULL");
            goto done;
        }
        // The slot ranges cover [0, n_cand) exactly; a view without
        // candidates runs one Adam launch over the empty range (0, 0), which
        // updates every Gaussian with a zero gradient and reads no slot.
        const int64_t chunk = std::max<int64_t>(1, std::min<int64_t>(nc, opts->adam_chunk));
        float* grad3d = (float*)gs_malloc(ctx, sizeof(float) * (int64_t)F * chunk, GS_MEM_GRAD, &view);
        if (!grad3d) { st = GS_ERR_OOM; goto done; }
        for (int64_t s0 = 0; s0 < n_cand || s0 == 0; s0 += chunk) {
            const int64_t s1 = std::min<int64_t>(n_cand, s0 + chunk);
            if ((st = launch_project_bwd(ctx, cam, params, proj, grad2d, s0, s1, grad3d)) != GS_OK) goto done;
            if ((st = launch_adam(ctx, proj, params->n, params->sh_degree, opts->params_rw, opts->adam_m,
                                  opts->adam_v, grad3d, s0, s1, opts->adam_step, opts->lr, opts->beta1, opts->beta2,
                                  opts->eps)) != GS_OK)
                goto done;
        }
    }
    if ((st = view_loss(ctx, opts, l1_view, l1_n, loss_dev, loss_dev + 1, P, &loss, sum_chunks)) != GS_OK) goto done;
finish:
    result->loss = loss;
    result->n_cand = n_cand;
    result->n_isect = isect_total;
    result->n_leaves = (int32_t)leaves.size();
    result->groups_walked = walk_used ? 1 : 0;
    result->peak_bytes = ctx->peak - live0;
    if (opts->leaf_bytes_out && opts->max_leaves > 0)
        std::memcpy(opts->leaf_bytes_out, ctx->tag_peak.data(),
                    sizeof(uint64_t) * std::min<size_t>(ctx->tag_peak.size(), opts->max_leaves));
done:
    gs_free_all(ctx, &view);
    gs_release(ctx, proj);
    ctx->peak = std::max(ctx->peak, peak_before);
    ctx->tag_live.clear();
    ctx->tag_peak.clear();
    return st;
}

}  // extern "C"
