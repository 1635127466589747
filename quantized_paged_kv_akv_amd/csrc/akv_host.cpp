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
// launch-shape overrides of the calling thread (akv_set_launch_shape); 0 = planned
static thread_local akv_launch_shape g_shape = {0, 0, 0, 0, 0, 0};

hipEvent_t prof_start_event() { return g_prof_start; }
bool pv_fp16() { return g_shape.pv_fp16 != 0; }
int issue_priority() { return g_shape.issue_priority; }
hipEvent_t prof_stop_event() { return g_prof_stop; }

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
// split) stay a few percent of the pages read.  The thread's launch shape
// (akv_set_launch_shape) overrides the choice.
SplitPlan plan_splits(const akv_dims* d, int batch, int max_pages) {
    SplitPlan p{1, 0};
    if (batch <= 0 || max_pages <= 0) return p;
    long long units = (long long)batch * d->num_kv_heads * max_pages;
    long long target_wgs = 1024;
    int pps = (int)std::max<long long>(4, (units + target_wgs - 1) / target_wgs);
    if (g_shape.pages_per_split > 0) pps = g_shape.pages_per_split;
    pps = std::min(pps, max_pages);
    p.pages_per_split = pps;
    p.n_splits = (max_pages + pps - 1) / pps;
    return p;
}

// Two waves per SIMD are resident (2048 on the chip); give each about an equal
// share of the page-heads, at least min_ppw pages so the per-wave set-up, the
// first page's latency and the end-of-split merge stay small.  Measured at 32K
// (496 pages x 4 KV heads): the int8 call alone runs best with 2 pages per wave
// (19.2 us against 20.7 with 3 and 24.4 with 4), the hybrid call with 3.  A
// work-group is four waves, so it owns four waves' worth of consecutive pages.
// The thread's launch shape overrides the choice.
SplitPlan plan_int8_splits(const akv_dims* d, int batch, int max_pages, int min_ppw) {
    SplitPlan p{1, 0};
    if (batch <= 0 || max_pages <= 0) return p;
    long long units = (long long)batch * d->num_kv_heads * max_pages;
    int ppw = (int)std::max<long long>(min_ppw, (units + 2047) / 2048);
    if (g_shape.pages_per_wave > 0) ppw = g_shape.pages_per_wave;
    ppw = std::min(ppw, kMaxPagesPerWave);
    p.pages_per_split = std::min(4 * ppw, max_pages);
    p.n_splits = (max_pages + p.pages_per_split - 1) / p.pages_per_split;
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

int device_cu_count() {
    static thread_local int cached_dev = -1, cached_cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached_cus = cus;
        else
            (void)hipGetLastError();
        cached_dev = dev;
    }
    return cached_cus;
}

void plan_hybrid(const akv_dims* d, int batch, int max_pages_int8, int max_pages_window, SplitPlan* p8,
                 SplitPlan* pw) {
    *p8 = plan_int8_splits(d, batch, max_pages_int8, 3);
    *pw = plan_window_splits(d, batch, max_pages_window);
    if (batch <= 0 || max_pages_window <= 0 || max_pages_int8 <= 0) return;
    const long long units = (long long)batch * d->num_kv_heads;
    const long long slots = 2LL * device_cu_count();
    // A BF16 page is twice the bytes of an int8 page, and the exact body
    // streams more slowly per work-group (a barrier per page): window
    // work-groups of a sixth as many pages finish with the int8 ones
    // (measured at 32K, one request: 322 us per 16-layer step with two
    // window pages per work-group against 325 with three and 329 with one).
    int qw = std::max(1, std::min(p8->pages_per_split / 6, max_pages_window));
    long long nw = units * ((max_pages_window + qw - 1) / qw);
    const long long n8 = units * p8->n_splits;
    if (n8 + nw > slots && 4 * (n8 + nw) <= 5 * slots) {
        // A grid a little over one round would leave a few int8 work-groups
        // to run after all the others: widen the int8 work-groups until it
        // fits.  If one window page per work-group takes at most an eighth of
        // the slots, use that: those work-groups end early and the int8
        // work-groups keep the rest (measured at 128K, 4 KV heads: 845 us
        // per 16-layer step against 857 with four window pages per
        // work-group).  int8 splits share a request's pages near-equally, so
        // any count works.
        if (8 * units * max_pages_window <= slots) {
            qw = 1;
            nw = units * max_pages_window;
        }
        if (slots - nw >= units) {
            const int splits = (int)std::min<long long>((slots - nw) / units, max_pages_int8);
            const int q8 = (max_pages_int8 + splits - 1) / splits;
            // no more work-groups than that many pages each needs: a few slots
            // stay free, which streams slightly better than a completely full chip
            if ((q8 + 3) / 4 <= kMaxPagesPerWave) *p8 = SplitPlan{q8, (max_pages_int8 + q8 - 1) / q8};
        }
    } else if (4 * (n8 + nw) > 5 * slots) {
        // Several rounds of work-groups (many requests): at most five int8
        // pages per wave and four window pages per work-group, so the slots
        // that requests of different lengths free are handed new work-groups
        // and the rounds even out (measured on 32 requests of 4K-16K tokens:
        // 2.27 ms per step against 2.32 with one wide round per request).
        const int q8 = std::min(p8->pages_per_split, 20);
        *p8 = SplitPlan{q8, (max_pages_int8 + q8 - 1) / q8};
        qw = std::min(qw, 4);
    }
    if (g_shape.hybrid_int8_pages > 0) {
        const int q8 = std::min(std::min(g_shape.hybrid_int8_pages, 4 * kMaxPagesPerWave), max_pages_int8);
        *p8 = SplitPlan{q8, (max_pages_int8 + q8 - 1) / q8};
    }
    if (g_shape.hybrid_window_pages > 0) qw = g_shape.hybrid_window_pages;
    qw = std::min(qw, max_pages_window);
    *pw = SplitPlan{qw, (max_pages_window + qw - 1) / qw};
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

extern "C" akv_status akv_set_launch_shape(const akv_launch_shape* shape) {
    akv::clear_error();
    if (!shape) {
        akv::g_shape = akv_launch_shape{0, 0, 0, 0, 0, 0};
        return AKV_OK;
    }
    if (shape->pages_per_split < 0 || shape->pages_per_wave < 0 || shape->hybrid_int8_pages < 0 ||
        shape->hybrid_window_pages < 0)
        return akv::fail(AKV_ERR_ARG, "launch shape fields must be >= 0 (0 = planned)");
    if (shape->pv_fp16 != 0 && shape->pv_fp16 != 1) return akv::fail(AKV_ERR_ARG, "pv_fp16 must be 0 or 1");
    if (shape->issue_priority < 0 || shape->issue_priority > 2)
        return akv::fail(AKV_ERR_ARG, "issue_priority must be 0, 1 or 2");
    if (shape->pages_per_wave > akv::kMaxPagesPerWave || shape->hybrid_int8_pages > 4 * akv::kMaxPagesPerWave)
        return akv::fail(AKV_ERR_ARG, "launch shape beyond %d pages per wave (%d per int8 work-group)",
                         akv::kMaxPagesPerWave, 4 * akv::kMaxPagesPerWave);
    akv::g_shape = *shape;
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
    akv::SplitPlan p8, pw;
    akv::plan_hybrid(dims, batch, max_pages_int8, max_pages_window, &p8, &pw);
    return akv::partial_bytes(dims, batch, p8.n_splits + pw.n_splits);
}
