// ring.cpp -- host-staged mode: layer-at-a-time staging of pinned host history
// into a ring of caller-owned device slots ("ActiveKV" page, "The idea" and
// "What I built").  The pinned host copy is the authoritative history and the
// device holds only a budgeted working set; copies are asynchronous, and
// events order every reuse of a slot after both the copy into it and the
// kernels reading it have finished; a request too large for a slot is
// refused up front instead of stalling.
//
// Lifecycle of slot s = layer % n_slots:
//   free --stage--> staged --release--> free
// stage:   copy_stream waits slot_free[s] (if it was ever released), copies,
//          records copy_done[s]; compute_stream waits copy_done[s].
// release: compute_stream records slot_free[s] after the kernels that read it.
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "akv_host.h"

struct akv_ring {
    std::vector<void*> slots;
    size_t slot_bytes = 0;
    std::vector<hipEvent_t> slot_free;
    std::vector<hipEvent_t> copy_done;
    std::vector<int> staged;          // 1 between stage and release
    std::vector<int> free_recorded;   // slot_free[s] has been recorded at least once
};

using akv::fail;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

extern "C" akv_status akv_ring_create(void* const* slots, size_t slot_bytes, int32_t n_slots, akv_ring** out) {
    akv::clear_error();
    if (!slots || !out) return fail(AKV_ERR_ARG, "NULL pointer");
    if (n_slots < 2) return fail(AKV_ERR_ARG, "ring needs at least 2 slots (got %d)", n_slots);
    if (slot_bytes == 0) return fail(AKV_ERR_ARG, "slot_bytes is 0");
    for (int i = 0; i < n_slots; ++i) {
        if (!slots[i]) return fail(AKV_ERR_ARG, "slot %d is NULL", i);
        if (!akv::aligned16(slots[i])) return fail(AKV_ERR_ALIGN, "slot %d not 16-byte aligned", i);
    }
    akv_ring* r = new (std::nothrow) akv_ring();
    if (!r) return fail(AKV_ERR_ARG, "out of host memory");
    r->slots.assign(slots, slots + n_slots);
    r->slot_bytes = slot_bytes;
    r->slot_free.resize(n_slots, nullptr);
    r->copy_done.resize(n_slots, nullptr);
    r->staged.assign(n_slots, 0);
    r->free_recorded.assign(n_slots, 0);
    for (int i = 0; i < n_slots; ++i) {
        if (hipEventCreateWithFlags(&r->slot_free[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&r->copy_done[i], hipEventDisableTiming) != hipSuccess) {
            for (auto e : r->slot_free)
                if (e) (void)hipEventDestroy(e);
            for (auto e : r->copy_done)
                if (e) (void)hipEventDestroy(e);
            delete r;
            return fail(AKV_ERR_HIP, "hipEventCreateWithFlags failed");
        }
    }
    *out = r;
    return AKV_OK;
}

extern "C" akv_status akv_ring_stage(akv_ring* r, int32_t layer, const void* const* host_srcs, const size_t* bytes,
                                     int32_t n_srcs, void* copy_stream, void* compute_stream, void** slot_out,
                                     size_t* offsets) {
    akv::clear_error();
    if (!r || !host_srcs || !bytes || !slot_out) return fail(AKV_ERR_ARG, "NULL pointer");
    if (layer < 0 || n_srcs < 0) return fail(AKV_ERR_ARG, "negative layer or n_srcs");
    const int n = (int)r->slots.size();
    const int s = layer % n;
    if (r->staged[s]) return fail(AKV_ERR_STATE, "slot %d staged again before release", s);
    size_t total = 0;
    for (int k = 0; k < n_srcs; ++k) {
        if (!host_srcs[k] && bytes[k]) return fail(AKV_ERR_ARG, "host source %d is NULL", k);
        total += align256(bytes[k]);
    }
    if (total > r->slot_bytes)
        return fail(AKV_ERR_BUDGET, "layer %d needs %zu bytes, slot holds %zu", layer, total, r->slot_bytes);
    hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)compute_stream;
    if (r->free_recorded[s] && hipStreamWaitEvent(cs, r->slot_free[s], 0) != hipSuccess)
        return fail(AKV_ERR_HIP, "hipStreamWaitEvent(slot_free)");
    char* base = static_cast<char*>(r->slots[s]);
    size_t off = 0;
    for (int k = 0; k < n_srcs; ++k) {
        if (bytes[k] && hipMemcpyAsync(base + off, host_srcs[k], bytes[k], hipMemcpyHostToDevice, cs) != hipSuccess)
            return fail(AKV_ERR_HIP, "hipMemcpyAsync (source %d)", k);
        if (offsets) offsets[k] = off;
        off += align256(bytes[k]);
    }
    if (hipEventRecord(r->copy_done[s], cs) != hipSuccess) return fail(AKV_ERR_HIP, "hipEventRecord(copy_done)");
    if (hipStreamWaitEvent(ks, r->copy_done[s], 0) != hipSuccess)
        return fail(AKV_ERR_HIP, "hipStreamWaitEvent(copy_done)");
    r->staged[s] = 1;
    *slot_out = base;
    return AKV_OK;
}

extern "C" akv_status akv_ring_release(akv_ring* r, int32_t layer, void* compute_stream) {
    akv::clear_error();
    if (!r) return fail(AKV_ERR_ARG, "NULL ring");
    if (layer < 0) return fail(AKV_ERR_ARG, "negative layer");
    const int s = layer % (int)r->slots.size();
    if (!r->staged[s]) return fail(AKV_ERR_STATE, "slot %d released while not staged", s);
    if (hipEventRecord(r->slot_free[s], (hipStream_t)compute_stream) != hipSuccess)
        return fail(AKV_ERR_HIP, "hipEventRecord(slot_free)");
    r->free_recorded[s] = 1;
    r->staged[s] = 0;
    return AKV_OK;
}

extern "C" akv_status akv_ring_destroy(akv_ring* r) {
    akv::clear_error();
    if (!r) return AKV_OK;
    akv_status st = AKV_OK;
    for (size_t i = 0; i < r->slots.size(); ++i) {
        if (r->free_recorded[i] && hipEventSynchronize(r->slot_free[i]) != hipSuccess) st = AKV_ERR_HIP;
        if (hipEventSynchronize(r->copy_done[i]) != hipSuccess) st = AKV_ERR_HIP;
        (void)hipEventDestroy(r->slot_free[i]);
        (void)hipEventDestroy(r->copy_done[i]);
    }
    delete r;
    return st == AKV_OK ? AKV_OK : fail(st, "event synchronize failed during destroy");
}
