// calib.hip -- instrumentation: a plain streaming read of a device buffer, the
// ceiling the decode kernels' HBM rate is compared against.  Each work-group
// streams a contiguous chunk with sixteen 16-byte loads per lane in flight,
// issued with the non-temporal hint (each byte is read once; on this part the
// hint lifts a plain streaming read from about 6.3 to about 7.1 TB/s), and
// folds what it read into one word (written only on an impossible value, so
// the loads cannot be removed and nothing but the sink is ever stored).
#include "akv_device.h"
#include "akv_host.h"

namespace akv {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16_per_wg,
                                                          uint32_t* __restrict__ sink) {
    const u32x4* p = src + (size_t)blockIdx.x * n16_per_wg;
    uint32_t acc = 0;
    for (size_t i = threadIdx.x; i < n16_per_wg; i += (size_t)256 * 16) {
        u32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const size_t k = i + (size_t)u * 256;
            v[u] = k < n16_per_wg ? __builtin_nontemporal_load(p + k) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    clear_error();
    if (!buf || !sink) return fail(AKV_ERR_ARG, "NULL pointer");
    if (!aligned16(buf) || (bytes & 15) != 0) return fail(AKV_ERR_ALIGN, "buffer or size not 16-byte aligned");
    const int wgs = 2048;
    const size_t n16 = bytes / 16 / wgs;
    if (n16 == 0) return fail(AKV_ERR_ARG, "buffer of %zu bytes too small (at least %d x 16 bytes)", bytes, wgs);
    stream_read_kernel<<<wgs, 256, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(buf), n16, sink);
    return launch_status("stream_read_kernel");
}
