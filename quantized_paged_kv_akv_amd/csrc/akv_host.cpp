// akv_host.cpp -- status strings, thread-local errors, shape checks, split plan.
#include "akv_host.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

namespace akv {

static thread_local char g_err[512] = "";

akv_status fail(akv_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = '\0'; }

static thread_local hipEvent_t g_prof_start = nullptr;
static thread_local hipEvent_t g_prof_stop = nullptr;

void prof_begin(hipStream_t s) {
    if (g_prof_start) (void)hipEventRecord(g_prof_start, s);
}
void prof_end(hipStream_t s) {
    if (g_prof_stop) (void)hipEventRecord(g_prof_stop, s);
}

akv_status check_dims(const akv_dims* d) {
    if (!d) return fail(AKV_ERR_ARG, "dims is NULL");
    if (d->num_kv_heads < 1 || d->group < 1 || d->head_dim < 1 || d->page_size < 1)
        return fail(AKV_ERR_ARG, "dims must be positive (Hkv=%d G=%d D=%d P=%d)", d->num_kv_heads,
                    d->group, d->head_dim, d->page_size);
    if (d->head_dim != 256) return fail(AKV_ERR_UNSUPPORTED, "head_dim %d unsupported (256 only)", d->head_dim);
    if (d->page_size != 64) return fail(AKV_ERR_UNSUPPORTED, "page_size %d unsupported (64 only)", d->page_size);
    if (d->group > 8) return fail(AKV_ERR_UNSUPPORTED, "group %d unsupported (1..8)", d->group);
    return AKV_OK;
}

// Enough work-groups to cover the 256 compute units several times over, but
// at least 4 pages per work-group so the split partials (6 KB written per
// split) stay a few percent of the pages read.  AKV_PAGES_PER_SPLIT overrides
// the choice (for launch-shape sweeps).
SplitPlan plan_splits(const akv_dims* d, int batch, int max_pages) {
    SplitPlan p{1, 0};
    if (batch <= 0 || max_pages <= 0) return p;
    long long units = (long long)batch * d->num_kv_heads * max_pages;
    long long target_wgs = 1024;
    int pps = (int)std::max<long long>(4, (units + target_wgs - 1) / target_wgs);
    if (const char* e = getenv("AKV_PAGES_PER_SPLIT")) {
        int v = atoi(e);
        if (v > 0) pps = v;
    }
    pps = std::min(pps, max_pages);
    p.pages_per_split = pps;
    p.n_splits = (max_pages + pps - 1) / pps;
    return p;
}

// One wave per SIMD is resident (1024 on the chip); give each about an equal
// share of the page-heads, at least 2 pages so the per-wave set-up and the
// end-of-split merge stay small.  AKV_PAGES_PER_WAVE overrides (sweeps).
SplitPlan plan_int8_splits(const akv_dims* d, int batch, int max_pages) {
    SplitPlan p{1, 0};
    if (batch <= 0 || max_pages <= 0) return p;
    long long units = (long long)batch * d->num_kv_heads * max_pages;
    int ppw = (int)std::max<long long>(2, (units + 1023) / 1024);
    if (const char* e = getenv("AKV_PAGES_PER_WAVE")) {
        int v = atoi(e);
        if (v > 0) ppw = v;
    }
    ppw = std::min(std::min(ppw, max_pages), 64);  // a wave stages at most 64 page slots
    p.pages_per_split = ppw;
    p.n_splits = (max_pages + 4 * ppw - 1) / (4 * ppw);
    return p;
}

SplitPlan plan_window_splits(const akv_dims* d, int batch, int max_pages) {
    SplitPlan p{1, 0};
    if (batch <= 0 || max_pages <= 0) return p;
    long long units = (long long)batch * d->num_kv_heads * max_pages;
    int pps = (int)std::max<long long>(1, (units + 511) / 512);
    pps = std::min(pps, max_pages);
    p.pages_per_split = pps;
    p.n_splits = (max_pages + pps - 1) / pps;
    return p;
}

size_t partial_bytes(const akv_dims* d, int batch, int n_splits) {
    size_t rows = (size_t)batch * d->num_kv_heads * d->group;
    size_t o = rows * (size_t)n_splits * d->head_dim * sizeof(float);
    size_t l = rows * (size_t)n_splits * sizeof(float);
    return ((o + 255) / 256) * 256 + ((l + 255) / 256) * 256;
}

}  // namespace akv

extern "C" const char* akv_status_string(akv_status s) {
    switch (s) {
        case AKV_OK: return "AKV_OK";
        case AKV_ERR_ARG: return "AKV_ERR_ARG";
        case AKV_ERR_UNSUPPORTED: return "AKV_ERR_UNSUPPORTED";
        case AKV_ERR_ALIGN: return "AKV_ERR_ALIGN";
        case AKV_ERR_WORKSPACE: return "AKV_ERR_WORKSPACE";
        case AKV_ERR_BUDGET: return "AKV_ERR_BUDGET";
        case AKV_ERR_HIP: return "AKV_ERR_HIP";
        case AKV_ERR_STATE: return "AKV_ERR_STATE";
    }
    return "AKV_ERR_UNKNOWN";
}

extern "C" const char* akv_last_error(void) { return akv::g_err; }

extern "C" const char* akv_version(void) { return "akv 0.1.0 gfx950"; }

extern "C" akv_status akv_set_profile_events(void* start_event, void* stop_event) {
    akv::clear_error();
    if ((start_event == nullptr) != (stop_event == nullptr))
        return akv::fail(AKV_ERR_ARG, "set both profile events or neither");
    akv::g_prof_start = (hipEvent_t)start_event;
    akv::g_prof_stop = (hipEvent_t)stop_event;
    return AKV_OK;
}

extern "C" size_t akv_decode_workspace_bytes(const akv_dims* dims, int32_t batch, int32_t max_pages) {
    if (akv::check_dims(dims) != AKV_OK || batch <= 0 || max_pages <= 0) return 0;
    const akv::SplitPlan p = akv::plan_splits(dims, batch, max_pages);
    const akv::SplitPlan p8 = akv::plan_int8_splits(dims, batch, max_pages);
    return akv::partial_bytes(dims, batch, std::max(p.n_splits, p8.n_splits));
}

extern "C" size_t akv_decode_hybrid_workspace_bytes(const akv_dims* dims, int32_t batch, int32_t max_pages_int8,
                                                    int32_t max_pages_window) {
    if (akv::check_dims(dims) != AKV_OK || batch <= 0 || max_pages_int8 < 0 || max_pages_window < 0) return 0;
    if (max_pages_int8 + max_pages_window == 0) return 0;
    akv::SplitPlan p8 = akv::plan_int8_splits(dims, batch, max_pages_int8);
    akv::SplitPlan pw = akv::plan_window_splits(dims, batch, max_pages_window);
    return akv::partial_bytes(dims, batch, p8.n_splits + pw.n_splits);
}
