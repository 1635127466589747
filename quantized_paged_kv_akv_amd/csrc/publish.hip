// publish.hip -- streaming page publication ("Model quantization" page, "An
// 8-bit page format shaped for its kernel": conversion happens in the
// background and only for pages complete in every layer; an unpublished page
// stays with the exact tier, so decode never waits for a conversion).
//
// akv_publish_pages converts full BF16 pages on a side stream once that
// stream has seen the caller's "pages complete" event, and records a "done"
// event; the caller polls that event (hipEventQuery) between decode steps and,
// once it has completed, publishes with akv_tables_advance on the compute
// stream: the new int8 slots are appended to the int8 table and the same
// number of pages leave the front of the window table.  Neither call blocks
// the host or the compute stream.
#include "akv_device.h"
#include "akv_host.h"

namespace akv {

// One thread per request.  Rows whose update would not fit are left as they
// are and flagged in status[b] (-1); others get 0.
__global__ void tables_advance_kernel(int batch, const int32_t* __restrict__ count,
                                      const int32_t* __restrict__ new_int8, int max_new,
                                      int32_t* __restrict__ int8_table, int32_t* __restrict__ n8, int max_int8,
                                      int32_t* __restrict__ window_table, int32_t* __restrict__ window_len,
                                      int max_window, int32_t* __restrict__ status) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int c = count[b];
    const int have = n8[b];
    const int wlen = window_len[b];
    const int wpages = (wlen + kP - 1) / kP;
    const bool ok = c >= 0 && c <= max_new && have + c <= max_int8 && c * kP <= wlen && wpages <= max_window;
    if (status) status[b] = ok ? 0 : -1;
    if (!ok || c == 0) return;
    int32_t* it = int8_table + (size_t)b * max_int8;
    const int32_t* nw = new_int8 + (size_t)b * max_new;
    for (int i = 0; i < c; ++i) it[have + i] = nw[i];
    int32_t* wt = window_table + (size_t)b * max_window;
    // the whole row moves, so slots the caller reserved past the window's
    // current pages (pages still to be appended) stay in order behind it;
    // ascending order: each entry is read before it is overwritten
    for (int i = 0; i + c < max_window; ++i) wt[i] = wt[i + c];
    n8[b] = have + c;
    window_len[b] = wlen - c * kP;
}

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_publish_pages(const akv_dims* dims, int32_t n, const uint16_t* k_bf16,
                                        const uint16_t* v_bf16, const int32_t* src_slot, const int32_t* dst_slot,
                                        int8_t* k_codes, int8_t* v_codes, float* k_chan, float* k_tok,
                                        float* v_chan, void* ready_event, void* side_stream, void* done_event) {
    clear_error();
    akv_status st = check_dims(dims);
    if (st != AKV_OK) return st;
    hipStream_t s = (hipStream_t)side_stream;
    if (ready_event && hipStreamWaitEvent(s, (hipEvent_t)ready_event, 0) != hipSuccess)
        return fail(AKV_ERR_HIP, "hipStreamWaitEvent(ready_event)");
    if ((st = akv_quantize_pages(dims, n, k_bf16, v_bf16, src_slot, dst_slot, k_codes, v_codes, k_chan, k_tok,
                                 v_chan, side_stream)) != AKV_OK)
        return st;
    if (done_event && hipEventRecord((hipEvent_t)done_event, s) != hipSuccess)
        return fail(AKV_ERR_HIP, "hipEventRecord(done_event)");
    return AKV_OK;
}

extern "C" akv_status akv_tables_advance(int32_t batch, const int32_t* count, const int32_t* new_int8,
                                         int32_t max_new, int32_t* int8_table, int32_t* n_pages_int8,
                                         int32_t max_pages_int8, int32_t* window_table, int32_t* window_len,
                                         int32_t max_pages_window, int32_t* status, void* stream) {
    clear_error();
    if (batch < 0 || max_new < 0 || max_pages_int8 < 0 || max_pages_window < 0)
        return fail(AKV_ERR_ARG, "negative size");
    if (batch == 0) return AKV_OK;
    const void* tabs[] = {count, new_int8, int8_table, n_pages_int8, window_table, window_len};
    for (const void* p : tabs) {
        if (!p) return fail(AKV_ERR_ARG, "NULL pointer");
        if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return fail(AKV_ERR_ALIGN, "table not 4-byte aligned");
    }
    if (status && (reinterpret_cast<uintptr_t>(status) & 3u) != 0)
        return fail(AKV_ERR_ALIGN, "status not 4-byte aligned");
    const int threads = 64;
    tables_advance_kernel<<<(batch + threads - 1) / threads, threads, 0, (hipStream_t)stream>>>(
        batch, count, new_int8, max_new, int8_table, n_pages_int8, max_pages_int8, window_table, window_len,
        max_pages_window, status);
    return launch_status("tables_advance_kernel");
}
