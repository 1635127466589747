// quantize.hip -- BF16 pages -> the 8-bit page format ("Model quantization"
// page, "An 8-bit page format shaped for its kernel").
//
// Per (page, KV head), one work-group of 256 threads (thread d owns channel d):
//   ms_d   = mean over the 64 tokens of K[t][d]^2            (float64)
//   u_d    = ms_d^(1/4)                                       (sqrt of the RMS)
//   g      = exp(mean of ln u_d over channels with ms_d > 0)
//   c_d    = clamp(u_d / g, 2^-14, 2^14), or 1 for a zero channel -> FP32
//   s_t    = max_d(|K[t][d]| / c_d) / 127                     -> FP32
//   vs_d   = max_t |V[t][d]| / 127                            -> FP32
//   codes  = clamp(rint(x / scale), -127, 127) with the quotient an IEEE
//            float64 divide by the exact product of the FP32 scales (taken
//            only near rounding boundaries; elsewhere a reciprocal product
//            gives the same integer).
// The factor normalisation happens before the clamp (the order the format
// states).  Codes are written in the pool layouts: K in tile order, V
// channel-major.  The kernel reads 64 KB and writes 35,072 B per page-head;
// it is off the decode path.
#include <math.h>

#include "akv_device.h"
#include "akv_host.h"

namespace akv {

// Code of x at scale = a * b (a, b FP32, so the product is exact in float64):
// round half to even of the float64 quotient x / scale, clamped to +-127.  The
// quotient is first estimated as x * inv_ab with inv_ab a product of rounded
// reciprocals (a few ulp off, under 2^-40 absolute for |q| <= 128); only when
// that estimate lies within 2^-30 of a half-integer (the boundaries of
// rounding to an integer) is the correctly rounded divide taken, so the
// result is always that of the IEEE float64 divide.
__device__ __forceinline__ int code_of(double x, double a, double b, double inv_ab) {
    if (a * b == 0.0) return 0;
    const double q = x * inv_ab;
    const double fl = floor(q);
    const double fr = q - fl;
    double r;
    if (fabs(fr - 0.5) < 0x1p-30)
        r = rint(x / (a * b));  // near a boundary: the exact quotient decides
    else
        r = fr < 0.5 ? fl : fl + 1.0;
    r = fmin(fmax(r, -127.0), 127.0);
    return (int)r;
}

// code_of for a nonzero scale, with fewer operations: the nearest integer
// of the estimate is the answer unless the estimate lies within 2^-30 of a
// half-integer, where the correctly rounded quotient decides -- the same
// decisions as code_of.  (Callers give a zero scale code 0 themselves.)
__device__ __forceinline__ int code_rint(double x, double a, double b, double inv_ab) {
    const double q = x * inv_ab;
    double r = rint(q);
    if (fabs(fabs(q - r) - 0.5) < 0x1p-30) r = rint(x / (a * b));
    r = fmin(fmax(r, -127.0), 127.0);
    return (int)r;
}

__global__ __launch_bounds__(256) void quantize_kernel(
    int Hkv, const uint16_t* __restrict__ kbf, const uint16_t* __restrict__ vbf,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int8_t* __restrict__ kcodes,
    int8_t* __restrict__ vcodes, float* __restrict__ kchan, float* __restrict__ ktok,
    float* __restrict__ vchan) {
    const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const size_t sp = (size_t)src[i] * Hkv + h;
    const size_t dp = (size_t)dst[i] * Hkv + h;
    const uint16_t* K = kbf + sp * (kP * kD);
    const uint16_t* V = vbf + sp * (kP * kD);

    __shared__ uint16_t Ks[kP][kD];
    __shared__ float c32s[kD];
    __shared__ double invc[kD];
    __shared__ float s32s[kP];
    __shared__ double invs[kP];
    __shared__ double red_sum[4];
    __shared__ int red_cnt[4];

    // value rows first (thread d owns channel row d: 64 contiguous tokens), so
    // their latency overlaps the key staging
    uint32_t vw[32];
    {
        const u32x4* row = reinterpret_cast<const u32x4*>(V + (size_t)tid * kP);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const u32x4 x = row[k];
            vw[4 * k + 0] = x.x;
            vw[4 * k + 1] = x.y;
            vw[4 * k + 2] = x.z;
            vw[4 * k + 3] = x.w;
        }
    }
    // stage the key page (32 KB) in LDS with coalesced 16-byte loads
    {
        const u32x4* src4 = reinterpret_cast<const u32x4*>(K);
        u32x4* dst4 = reinterpret_cast<u32x4*>(&Ks[0][0]);
#pragma unroll
        for (int k = 0; k < (kP * kD * 2) / (16 * 256); ++k) dst4[tid + 256 * k] = src4[tid + 256 * k];
    }
    __syncthreads();

    // channel factor
    const int d = tid;
    double ms = 0.0;
    for (int t = 0; t < kP; ++t) {
        const double k = (double)bf16_to_f32(Ks[t][d]);
        ms += k * k;
    }
    ms = ms / (double)kP;
    const bool nz = ms > 0.0;
    const double u = sqrt(sqrt(ms));
    double lg = nz ? log(u) : 0.0;
    int cnt = nz ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) {
        lg += __shfl_xor(lg, off, 64);
        cnt += __shfl_xor(cnt, off, 64);
    }
    if ((tid & 63) == 0) {
        red_sum[tid >> 6] = lg;
        red_cnt[tid >> 6] = cnt;
    }
    __syncthreads();
    const double lsum = red_sum[0] + red_sum[1] + red_sum[2] + red_sum[3];
    const int ncnt = red_cnt[0] + red_cnt[1] + red_cnt[2] + red_cnt[3];
    const double gmean = ncnt > 0 ? exp(lsum / (double)ncnt) : 1.0;
    double c = 1.0;
    if (nz) c = fmin(fmax(u / gmean, 1.0 / 16384.0), 16384.0);
    const float c32 = (float)c;
    c32s[d] = c32;
    invc[d] = 1.0 / (double)c32;
    kchan[dp * kD + d] = c32;
    __syncthreads();

    // token factor: 4 threads per token, 64 channels each (visited from a
    // per-token offset so the four-byte LDS words spread over the banks);
    // the max of |K| / c is taken on |K| * (1/c), which moves s_t by at most
    // a few float64 ulp before its FP32 rounding
    {
        const int t = tid >> 2, part = tid & 3;
        double m = 0.0;
        for (int e = 0; e < 64; ++e) {
            const int dd = part * 64 + ((e + 2 * t) & 63);
            m = fmax(m, fabs((double)bf16_to_f32(Ks[t][dd])) * invc[dd]);
        }
        m = fmax(m, __shfl_xor(m, 1, 64));
        m = fmax(m, __shfl_xor(m, 2, 64));
        const float s32 = (float)(m / 127.0);
        if (part == 0) {
            s32s[t] = s32;
            invs[t] = s32 != 0.0f ? 1.0 / (double)s32 : 0.0;
            ktok[dp * kP + t] = s32;
        }
    }
    __syncthreads();

    // key codes in tile order (kcode_offset): thread d writes channel d of
    // every token; 16 neighbouring channels land in one 16-byte run
    {
        int8_t* out = kcodes + dp * (kP * kD);
        const double cd = (double)c32s[d], icd = invc[d];
        int8_t* od = out + kcode_offset(0, d);  // kcode_offset(t, d) - kcode_offset(0, d) depends on t only
#pragma unroll
        for (int t = 0; t < kP; ++t) {
            const double x = (double)bf16_to_f32(Ks[t][d]);
            // c_d is never zero; a zero token factor (the same for every lane) gives code 0
            const int keep = __builtin_amdgcn_readfirstlane(__float_as_int(s32s[t])) == 0 ? 0 : -1;
            od[kcode_offset(t, 0)] = (int8_t)(code_rint(x, cd, (double)s32s[t], icd * invs[t]) & keep);
        }
    }

    // value scale and codes: channel-major rows of 64 tokens, 16-byte stores
    {
        double m = 0.0;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            m = fmax(m, fabs((double)bf16_to_f32((uint16_t)(vw[k] & 0xFFFFu))));
            m = fmax(m, fabs((double)bf16_to_f32((uint16_t)(vw[k] >> 16))));
        }
        const float vs32 = (float)(m / 127.0);
        const int vkeep = vs32 == 0.0f ? 0 : -1;  // a zero value scale gives code 0
        vchan[dp * kD + d] = vs32;
        const double vs = (double)vs32, ivs = vs != 0.0 ? 1.0 / vs : 0.0;
        u32x4* out = reinterpret_cast<u32x4*>(vcodes + dp * (kP * kD) + (size_t)d * kP);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t wds[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * k + 4 * j + e;
                    const uint16_t b = (tok & 1) ? (uint16_t)(vw[tok >> 1] >> 16) : (uint16_t)(vw[tok >> 1] & 0xFFFFu);
                    const int cv = code_rint((double)bf16_to_f32(b), vs, 1.0, ivs) & vkeep;
                    packed |= ((uint32_t)(cv & 0xFF)) << (8 * e);
                }
                wds[j] = packed;
            }
            out[k] = u32x4{wds[0], wds[1], wds[2], wds[3]};
        }
    }
}

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_quantize_pages(const akv_dims* dims, int32_t n, const uint16_t* k_bf16,
                                         const uint16_t* v_bf16, const int32_t* src_slot,
                                         const int32_t* dst_slot, int8_t* k_codes, int8_t* v_codes,
                                         float* k_chan, float* k_tok, float* v_chan, void* stream) {
    clear_error();
    akv_status st = check_dims(dims);
    if (st != AKV_OK) return st;
    if (n < 0) return fail(AKV_ERR_ARG, "n = %d < 0", n);
    if (n == 0) return AKV_OK;
    if (!k_bf16 || !v_bf16 || !src_slot || !dst_slot || !k_codes || !v_codes || !k_chan || !k_tok ||
        !v_chan)
        return fail(AKV_ERR_ARG, "NULL pointer");
    const void* ptrs[] = {k_bf16, v_bf16, src_slot, dst_slot, k_codes, v_codes, k_chan, k_tok, v_chan};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(AKV_ERR_ALIGN, "tensor not 16-byte aligned");
    dim3 grid((unsigned)n, (unsigned)dims->num_kv_heads);
    quantize_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(dims->num_kv_heads, k_bf16, v_bf16, src_slot,
                                                           dst_slot, k_codes, v_codes, k_chan, k_tok,
                                                           v_chan);
    return launch_status("quantize_kernel");
}
