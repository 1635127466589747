// akv_host.h -- host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/akv.h"

namespace akv {

// Record a thread-local message for akv_last_error() and return `s`.
akv_status fail(akv_status s, const char* fmt, ...);
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Instrumentation: the event pair the calling thread set with
// akv_set_profile_events (both NULL when unset).  The decode entry points
// launch their split-K kernel with hipExtLaunchKernelGGL when it is set, so
// the events bracket that kernel's dispatch and execution.
hipEvent_t prof_start_event();
hipEvent_t prof_stop_event();
// the calling thread's launch shape asks for the FP16 PV operand of the int8 tier
bool pv_fp16();
// the calling thread's wave issue-priority probe (0 = off, 1 = by pages left, 2 = by wave)
int issue_priority();

// Shape checks common to every attention/quantize call.
akv_status check_dims(const akv_dims* d);

// Split-K plan for the paged decode kernels: pages per work-group and the
// number of splits for page tables of `max_pages` columns.
struct SplitPlan {
    int pages_per_split;
    int n_splits;
};
SplitPlan plan_splits(const akv_dims* d, int batch, int max_pages);

// Plan of the int8 tier: n_splits work-groups per (request, KV head) share
// the request's pages near-equally (at most pages_per_split each) and split
// them near-equally over their four waves, each of which stages at most
// kMaxPagesPerWave page slots.
constexpr int kMaxPagesPerWave = 64;
SplitPlan plan_int8_splits(const akv_dims* d, int batch, int max_pages, int min_ppw = 2);

// Workspace bytes for `batch` requests with `n_splits` splits each.
size_t partial_bytes(const akv_dims* d, int batch, int n_splits);

// Split plan for the recent window of the hybrid call: few pages per split so
// the window's work-groups spread across the chip next to the int8 ones.
SplitPlan plan_window_splits(const akv_dims* d, int batch, int max_pages);

// Both tiers of akv_decode_hybrid: window work-groups stream about as many
// bytes as int8 ones, and when the grid would spill just past one round of
// resident work-groups (two per compute unit) the int8 work-groups widen so
// that it fits.  The thread's launch shape (akv_set_launch_shape) overrides
// the pages per work-group of each tier.
void plan_hybrid(const akv_dims* d, int batch, int max_pages_int8, int max_pages_window, SplitPlan* p8,
                 SplitPlan* pw);

// Compute units of the current device (256 if it cannot be queried).
int device_cu_count();

inline akv_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(AKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return AKV_OK;
}

// Second pass of split-K: fold the n_splits partials of each of `rows` rows
// (part_o [rows][n_splits][D], part_lse [rows][n_splits]) into out_o/out_lse.
akv_status launch_combine(int rows, int D, const float* part_o, const float* part_lse, int n_splits, float* out_o,
                          float* out_lse, hipStream_t stream);

}  // namespace akv
