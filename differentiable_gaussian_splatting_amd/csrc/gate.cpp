// gate.cpp -- the SkipGS backward gate (SkipGS notes, "key design" items 1-3
// and the "worked example"): host-side state of a training-view sequence
// that decides, from each view's forward loss, whether the view runs its
// backward and update.  Every value is a double computed in the order below,
// so the decisions are reproducible exactly.
#include <cmath>
#include <limits>
#include <new>
#include <vector>

#include "gs.h"

struct gs_gate {
    std::vector<double> ema;    // per view: loss EMA (valid where seen != 0)
    std::vector<uint8_t> seen;
    int32_t warmup = 500;
    double beta = 0.95, rho_lo = 0.5, eps = 1e-8;
    int64_t t = 0;              // steps taken
    int64_t b = 0;              // backwards run
    int64_t warm_n = 0;         // warm-up steps whose view already had an EMA
    int64_t warm_hits = 0;      // ... of which the score asked for a backward
    bool calibrated = false;
    double rho_min = 0.0;
};

extern "C" {

gs_status gs_gate_create(int32_t n_views, int32_t warmup, double beta, double rho_lo, double eps, gs_gate** out)
{
    if (!out || n_views < 1 || warmup < 0 || !(beta >= 0.0 && beta < 1.0) || !(rho_lo >= 0.0 && rho_lo <= 1.0) ||
        !(eps > 0.0))
        return GS_ERR_INVALID_ARG;
    gs_gate* g = new (std::nothrow) gs_gate;
    if (!g) return GS_ERR_OOM;
    try {
        g->ema.assign((size_t)n_views, 0.0);
        g->seen.assign((size_t)n_views, 0);
    } catch (...) {
        delete g;
        return GS_ERR_OOM;
    }
    g->warmup = warmup;
    g->beta = beta;
    g->rho_lo = rho_lo;
    g->eps = eps;
    *out = g;
    return GS_OK;
}

void gs_gate_destroy(gs_gate* g) { delete g; }

gs_status gs_gate_step(gs_gate* g, int32_t view, double loss, gs_gate_decision* d)
{
    if (!g || !d || view < 0 || (size_t)view >= g->ema.size() || !std::isfinite(loss)) return GS_ERR_INVALID_ARG;
    g->t += 1;
    const bool have = g->seen[(size_t)view] != 0;
    const double e = g->ema[(size_t)view];
    // item 1: the score against the view's own baseline; a view never seen
    // scores +inf so that it runs its backward
    const double score = have ? loss / (e + g->eps) : std::numeric_limits<double>::infinity();
    const bool proposed = score > 1.0;
    const double rho_cum = (double)g->b / (double)std::max<int64_t>(g->t - 1, 1);
    bool backward, forced = false;
    if (g->t <= g->warmup) {
        // item 3: the warm-up runs every backward and counts the proposals
        if (have) {
            g->warm_n += 1;
            g->warm_hits += proposed ? 1 : 0;
        }
        backward = true;
    } else {
        if (!g->calibrated) {
            const double rho_hat = g->warm_n > 0 ? (double)g->warm_hits / (double)g->warm_n : 0.0;
            g->rho_min = g->rho_lo + (1.0 - g->rho_lo) * rho_hat;
            g->calibrated = true;
        }
        backward = proposed;
        if (!proposed && rho_cum < g->rho_min) {   // the floor overrides the skip
            backward = true;
            forced = true;
        }
    }
    // item 2: the baseline follows the forward loss whatever the decision
    g->ema[(size_t)view] = have ? g->beta * e + (1.0 - g->beta) * loss : loss;
    g->seen[(size_t)view] = 1;
    if (backward) g->b += 1;
    d->backward = backward ? 1 : 0;
    d->forced = forced ? 1 : 0;
    d->score = score;
    d->rho_cum = rho_cum;
    return GS_OK;
}

gs_status gs_gate_get_stats(const gs_gate* g, gs_gate_stats* s)
{
    if (!g || !s) return GS_ERR_INVALID_ARG;
    s->steps = g->t;
    s->backwards = g->b;
    s->warmup_counted = g->warm_n;
    s->warmup_proposed = g->warm_hits;
    s->calibrated = g->calibrated ? 1 : 0;
    s->pad = 0;
    s->rho_min = g->rho_min;
    return GS_OK;
}

}  // extern "C"
