// merge.hip -- exact log-sum-exp merges ("SYCL" page, "A merge that joins
// the tiers": partials fold into one FP32 accumulator, an LSE of -inf is a
// valid empty partial).
//
// akv_merge_lse: one work-group per row (a request's query head), one thread
// per channel.  The split-K second pass (launch_combine: one of four kernels
// by the number of split columns) uses the same rule over all of a row's
// split partials.
#include <math.h>

#include "akv_device.h"
#include "akv_host.h"

namespace akv {

__global__ void fill_empty_kernel(int rows, int D, float* __restrict__ o, float* __restrict__ lse) {
    const size_t total = (size_t)rows * D;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x)
        o[i] = 0.0f;
    for (size_t r = (size_t)blockIdx.x * blockDim.x + threadIdx.x; r < (size_t)rows;
         r += (size_t)gridDim.x * blockDim.x)
        lse[r] = -INFINITY;
}

// acc <- acc (+) part, exactly, per row.
__global__ void merge_lse_kernel(int D, float* __restrict__ acc_o, float* __restrict__ acc_lse,
                                 const float* __restrict__ part_o, const float* __restrict__ part_lse) {
    const int r = blockIdx.x;
    const float a = acc_lse[r], p = part_lse[r];
    const float m = fmaxf(a, p);
    float wa = 0.0f, wp = 0.0f, L = -INFINITY;
    if (m != -INFINITY) {
        const float ea = (a == -INFINITY) ? 0.0f : expf(a - m);
        const float ep = (p == -INFINITY) ? 0.0f : expf(p - m);
        const float s = ea + ep;
        L = m + logf(s);
        wa = ea / s;
        wp = ep / s;
    }
    __syncthreads();  // every thread has read acc_lse[r] before it is rewritten
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        const size_t i = (size_t)r * D + d;
        // an empty side contributes nothing, whatever its O holds
        float v = 0.0f;
        if (wa != 0.0f) v += wa * acc_o[i];
        if (wp != 0.0f) v += wp * part_o[i];
        acc_o[i] = v;
    }
    if (threadIdx.x == 0) acc_lse[r] = L;
}

// Split-K second pass.  Row r = b*Hq + j holds n_splits partials
// part_o[r][s][D], part_lse[r][s]; every split slot is written by the split
// pass on every call (an empty split writes LSE = -inf), so no counts are
// needed here.  Block (r, c) owns channels [32c, 32c + 32): 8 split lanes x
// 32 channels, the LSE statistics are block-reduced once.
__device__ __forceinline__ float block_reduce_max(float v, float* red) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return v;
}

constexpr int kCombineMaxSplits = 2048;  // weights staged in LDS; larger counts loop in chunks

__global__ __launch_bounds__(256) void combine_kernel(int D, int n_splits, const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, float* __restrict__ out_o,
                                                      float* __restrict__ out_lse) {
    const int r = blockIdx.x, chunk = blockIdx.y;
    const int tid = threadIdx.x, sl = tid >> 5, c = tid & 31;
    __shared__ float red[4];
    __shared__ float wgt[kCombineMaxSplits];
    __shared__ float acc_s[8][32];
    const float* lse = part_lse + (size_t)r * n_splits;
    float m = -INFINITY;
    for (int s = tid; s < n_splits; s += 256) m = fmaxf(m, lse[s]);
    m = block_reduce_max(m, red);
    const int d = chunk * 32 + c;
    if (m == -INFINITY) {
        if (sl == 0) out_o[(size_t)r * D + d] = 0.0f;
        if (chunk == 0 && tid == 0) out_lse[r] = -INFINITY;
        return;
    }
    float sum = 0.0f;
    float acc = 0.0f;
    const float* po = part_o + (size_t)r * n_splits * D + d;
    for (int base = 0; base < n_splits; base += kCombineMaxSplits) {
        const int cnt = min(kCombineMaxSplits, n_splits - base);
        for (int s = tid; s < cnt; s += 256) {
            const float l = lse[base + s];
            const float e = (l == -INFINITY) ? 0.0f : expf(l - m);
            wgt[s] = e;
            sum += e;
        }
        __syncthreads();
        // 8 split lanes x 32 channels; independent loads, a zero weight skips nothing
        // (an empty split's O slot may hold anything, so it is masked, not multiplied)
        int s = sl;
        for (; s + 24 < cnt; s += 32) {
            const float w0 = wgt[s], w1 = wgt[s + 8], w2 = wgt[s + 16], w3 = wgt[s + 24];
            const float o0 = po[(size_t)(base + s) * D], o1 = po[(size_t)(base + s + 8) * D];
            const float o2 = po[(size_t)(base + s + 16) * D], o3 = po[(size_t)(base + s + 24) * D];
            acc += (w0 != 0.0f ? w0 * o0 : 0.0f) + (w1 != 0.0f ? w1 * o1 : 0.0f) +
                   (w2 != 0.0f ? w2 * o2 : 0.0f) + (w3 != 0.0f ? w3 * o3 : 0.0f);
        }
        for (; s < cnt; s += 8) {
            const float w0 = wgt[s];
            if (w0 != 0.0f) acc += w0 * po[(size_t)(base + s) * D];
        }
        __syncthreads();
    }
    sum = block_reduce_sum(sum, red);
    acc_s[sl][c] = acc;
    __syncthreads();
    if (sl == 0) {
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t += acc_s[k][c];
        out_o[(size_t)r * D + d] = t / sum;
    }
    if (chunk == 0 && tid == 0) out_lse[r] = m + logf(sum);
}

// The same pass for up to 8*K splits with every load issued up front: each
// thread holds the LSE and one channel's O of its K splits in registers, so
// the whole pass waits on memory once (the loop above waits once per group
// of four splits, which dominates at the usual hundred-odd splits).
template <int K>
__global__ __launch_bounds__(256) void combine_reg_kernel(int D, int n_splits, const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          float* __restrict__ out_o, float* __restrict__ out_lse) {
    const int r = blockIdx.x, chunk = blockIdx.y;
    const int tid = threadIdx.x, sl = tid >> 5, c = tid & 31;
    const int d = chunk * 32 + c;
    __shared__ float red_m[8], red_w[8], acc_s[8][32];
    const float* lse = part_lse + (size_t)r * n_splits;
    const float* po = part_o + (size_t)r * n_splits * D + d;
    float l[K], o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int sp = sl + 8 * k;
        l[k] = sp < n_splits ? lse[sp] : -INFINITY;
        o[k] = sp < n_splits ? po[(size_t)sp * D] : 0.0f;
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) m = fmaxf(m, l[k]);
    if (c == 0) red_m[sl] = m;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, red_m[k]);
    if (m == -INFINITY) {  // every split empty
        if (sl == 0) out_o[(size_t)r * D + d] = 0.0f;
        if (chunk == 0 && tid == 0) out_lse[r] = -INFINITY;
        return;
    }
    float w = 0.0f, acc = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float e = (l[k] == -INFINITY) ? 0.0f : expf(l[k] - m);
        w += e;
        if (e != 0.0f) acc += e * o[k];  // an empty split's O slot may hold anything
    }
    acc_s[sl][c] = acc;
    if (c == 0) red_w[sl] = w;
    __syncthreads();
    if (sl == 0) {
        float t = 0.0f, W = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            t += acc_s[k][c];
            W += red_w[k];
        }
        out_o[(size_t)r * D + d] = t / W;
        if (chunk == 0 && c == 0) out_lse[r] = m + logf(W);
    }
}

// Reductions over the 16 split lanes of a wave (the lanes that share
// lane % 4): two rotations inside each row of 16 lanes (DPP row_ror 4, then
// 8), then gfx950's row swaps (v_permlane16_swap pairs rows 0-1 and 2-3,
// v_permlane32_swap the two halves).  All in VALU: no LDS, no barrier.
// Every lane ends with the whole group's value; the association order
// differs between lanes, so one fixed lane writes the result.
__device__ __forceinline__ float rotate_in_row(float x, int by8) {
    const int v = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, by8 ? __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false)
                                         : __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
}

__device__ __forceinline__ float split_lanes_max(float x) {
    x = fmaxf(x, rotate_in_row(x, 0));
    x = fmaxf(x, rotate_in_row(x, 1));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float split_lanes_sum(float x) {
    x = x + rotate_in_row(x, 0);
    x = x + rotate_in_row(x, 1);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The pass for one request's many splits (17-128 columns: a long context
// split over the whole chip), where it is a chain of latencies rather than
// of bytes: block (row, 64 channels), each wave 16 of the channels as 16
// split lanes x 4 threads x 4 channels, up to 16*K splits in registers, the
// reductions over split lanes inside the wave (about 0.4 us less per layer
// than reducing over 16 split lanes x 16 threads through LDS with two
// barriers).
template <int K>
__global__ __launch_bounds__(256) void combine_wave_kernel(int D, int n_splits, const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           float* __restrict__ out_o, float* __restrict__ out_lse) {
    const int r = blockIdx.x, chunk = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int sl = lane >> 2;
    const int d = chunk * 64 + 16 * (tid >> 6) + 4 * (lane & 3);
    const float* lse = part_lse + (size_t)r * n_splits;
    const float* po = part_o + (size_t)r * n_splits * D + d;
    float l[K];
    f32x4 o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int sp = sl + 16 * k;
        l[k] = sp < n_splits ? lse[sp] : -INFINITY;
        o[k] = sp < n_splits ? *reinterpret_cast<const f32x4*>(po + (size_t)sp * D) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) m = fmaxf(m, l[k]);
    m = split_lanes_max(m);
    if (m == -INFINITY) {  // every split empty
        if (sl == 0) *reinterpret_cast<f32x4*>(out_o + (size_t)r * D + d) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (chunk == 0 && tid == 0) out_lse[r] = -INFINITY;
        return;
    }
    float w = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float e = (l[k] == -INFINITY) ? 0.0f : expf(l[k] - m);
        w += e;
        if (e != 0.0f) acc += e * o[k];  // an empty split's O slot may hold anything
    }
    w = split_lanes_sum(w);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = split_lanes_sum(acc[c]);
    if (sl == 0) {
        *reinterpret_cast<f32x4*>(out_o + (size_t)r * D + d) = acc / w;
        if (chunk == 0 && tid == 0) out_lse[r] = m + logf(w);
    }
}

// Few split columns (up to S): a thread owns 4 channels of one row and folds
// every column itself, so no reduction crosses threads; a block is 4 rows x
// 64 threads.  This is the many-requests case (the 32-request step: 768
// rows of 4 columns), where a block per (row, channel chunk) made 3,072
// short work-groups: 2.20 against 2.26 ms per 16-layer batched step.
template <int S>
__global__ __launch_bounds__(256) void combine_thread_kernel(int rows, int D, int n_splits,
                                                             const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             float* __restrict__ out_o, float* __restrict__ out_lse) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int d = 4 * (threadIdx.x & 63);
    const float* lse = part_lse + (size_t)r * n_splits;
    const float* po = part_o + (size_t)r * n_splits * D + d;
    float l[S];
    f32x4 o[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
        l[k] = k < n_splits ? lse[k] : -INFINITY;
        o[k] = k < n_splits ? *reinterpret_cast<const f32x4*>(po + (size_t)k * D) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < S; ++k) m = fmaxf(m, l[k]);
    if (m == -INFINITY) {  // every split empty
        *reinterpret_cast<f32x4*>(out_o + (size_t)r * D + d) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (d == 0) out_lse[r] = -INFINITY;
        return;
    }
    float w = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < S; ++k) {
        const float e = (l[k] == -INFINITY) ? 0.0f : expf(l[k] - m);
        w += e;
        if (e != 0.0f) acc += e * o[k];  // an empty split's O slot may hold anything
    }
    *reinterpret_cast<f32x4*>(out_o + (size_t)r * D + d) = acc / w;
    if (d == 0) out_lse[r] = m + logf(w);
}

akv_status launch_combine(int rows, int D, const float* part_o, const float* part_lse, int n_splits, float* out_o,
                          float* out_lse, hipStream_t stream) {
    if (rows == 0) return AKV_OK;
    dim3 grid((unsigned)rows, (unsigned)(D / 32));
    if (n_splits <= 4 && D == 256)  // the 32-request step: 4 columns, 3-4 us less per step than S = 8
        combine_thread_kernel<4><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, stream>>>(
            rows, D, n_splits, part_o, part_lse, out_o, out_lse);
    else if (n_splits <= 8 && D == 256)
        combine_thread_kernel<8><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, stream>>>(
            rows, D, n_splits, part_o, part_lse, out_o, out_lse);
    else if (n_splits <= 16 && D == 256)
        combine_thread_kernel<16><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, stream>>>(
            rows, D, n_splits, part_o, part_lse, out_o, out_lse);
    else if (n_splits <= 16 * 4)  // 32K: 50 columns, 2-3 us less per step than with K = 8
        combine_wave_kernel<4><<<dim3((unsigned)rows, (unsigned)(D / 64)), 256, 0, stream>>>(
            D, n_splits, part_o, part_lse, out_o, out_lse);
    else if (n_splits <= 16 * 8)
        combine_wave_kernel<8><<<dim3((unsigned)rows, (unsigned)(D / 64)), 256, 0, stream>>>(
            D, n_splits, part_o, part_lse, out_o, out_lse);
    else if (n_splits <= 8 * 32)
        combine_reg_kernel<32><<<grid, 256, 0, stream>>>(D, n_splits, part_o, part_lse, out_o, out_lse);
    else
        combine_kernel<<<grid, 256, 0, stream>>>(D, n_splits, part_o, part_lse, out_o, out_lse);
    return launch_status("combine_kernel");
}

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_fill_empty(int32_t rows, int32_t head_dim, float* o, float* lse, void* stream) {
    clear_error();
    if (rows < 0 || head_dim < 0) return fail(AKV_ERR_ARG, "negative size");
    if (rows == 0) return AKV_OK;
    if (!o || !lse) return fail(AKV_ERR_ARG, "NULL pointer");
    if (!aligned16(o) || !aligned16(lse)) return fail(AKV_ERR_ALIGN, "o/lse not 16-byte aligned");
    const size_t total = (size_t)rows * head_dim;
    int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    if (blocks < 1) blocks = 1;
    fill_empty_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(rows, head_dim, o, lse);
    return launch_status("fill_empty_kernel");
}

extern "C" akv_status akv_merge_lse(int32_t rows, int32_t head_dim, float* acc_o, float* acc_lse,
                                    const float* part_o, const float* part_lse, void* stream) {
    clear_error();
    if (rows < 0 || head_dim < 0) return fail(AKV_ERR_ARG, "negative size");
    if (rows == 0) return AKV_OK;
    if (!acc_o || !acc_lse || !part_o || !part_lse) return fail(AKV_ERR_ARG, "NULL pointer");
    if (!aligned16(acc_o) || !aligned16(acc_lse) || !aligned16(part_o) || !aligned16(part_lse))
        return fail(AKV_ERR_ALIGN, "tensor not 16-byte aligned");
    merge_lse_kernel<<<rows, 256, 0, (hipStream_t)stream>>>(head_dim, acc_o, acc_lse, part_o, part_lse);
    return launch_status("merge_lse_kernel");
}
