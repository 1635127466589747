// quantize.hip -- BF16 pages -> the 8-bit page format ("Model quantization"
// page, "An 8-bit page format shaped for its kernel").
//
// Per (page, KV head), one work-group of 256 threads:
//   ms_d   = mean over the 64 tokens of K[t][d]^2            (float64)
//   u_d    = ms_d^(1/4)                                       (sqrt of the RMS)
//   g      = exp(mean of ln u_d over channels with ms_d > 0)
//   c_d    = clamp(u_d / g, 2^-14, 2^14), or 1 for a zero channel -> FP32
//   s_t    = max_d(|K[t][d]| / c_d) / 127                     -> FP32
//   vs_d   = max_t |V[t][d]| / 127                            -> FP32
//   codes  = clamp(rint(x / scale), -127, 127), the quotient being the IEEE
//            float64 divide by the exact product of the FP32 scales.
// The factor normalisation happens before the clamp (the order the format
// states).  Codes are written in the pool layouts: K in tile order, V
// channel-major.  The kernel reads 64 KB and writes 35,072 B per page-head;
// it is off the decode path.
//
// Codes are decided from an FP32 estimate of the quotient, x * (1/c) * (1/s)
// with both reciprocals correctly rounded: for scales in [2^-100, 2^100] the
// estimate is within 127.5 * 4 * 2^-24 < 2^-15 of the exact quotient, so
// whenever it lies more than 2^-13 from a half-integer it rounds to the same
// integer as the float64 quotient.  Estimates closer than that (about one
// value in 4,000) take the float64 divide, as does every value of a token or
// channel whose scale is outside that range (zero scales give code 0 on the
// fast path).  The clamp never binds on the fast path: every |x| / scale is at
// most 127 (1 + 2^-22) by the construction of the scales.
//
// Thread roles: thread d owns value channel d (its 64 tokens arrive as one
// 128-byte row) and channel d of the key page for the channel factor; for the
// key codes, thread (wave w, lane l) owns token 16 ((l >> 2) & 3) + 4 w + (l & 3)
// and channels 64 j + 16 (l >> 4) + [0, 16) for j = 0..3, which makes each of
// its four 16-byte code runs land in the lane slot of tile 4 j + w that the
// decode kernel reads, so one wave stores whole 1 KB tiles, and the four lanes
// sharing a token finish its maximum with two lane exchanges.
#include <math.h>

#include "akv_device.h"
#include "akv_host.h"

namespace akv {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kNearHalf = 0.5f - 0x1p-13f;  // |estimate - rint| beyond this: exact divide
constexpr float kScaleLo = 0x1p-100f, kScaleHi = 0x1p100f;

// scales whose codes the FP32 estimate decides (zero included)
__device__ __forceinline__ bool fast_scale(float s) {
    return s == 0.0f || (s >= kScaleLo && s <= kScaleHi);
}

// round half to even of the float64 quotient x / scale, clamped to +-127; a
// zero scale gives code 0
__device__ __forceinline__ int code_exact(double x, double scale) {
    if (scale == 0.0) return 0;
    return (int)fmin(fmax(rint(x / scale), -127.0), 127.0);
}

// low bytes of four ints, byte e from c_e
__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
    return __builtin_amdgcn_perm((uint32_t)c1, (uint32_t)c0, 0x0c0c0400u) |
           __builtin_amdgcn_perm((uint32_t)c3, (uint32_t)c2, 0x04000c0cu);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The key page sits in LDS as 16-byte chunks, chunk c of token row t stored
// at c ^ ksw(t): the eight lanes that read one chunk column together in the
// code pass then hit eight different bank groups, while a wave reading one
// token row across 64 channels still covers 128 contiguous bytes.
__device__ __forceinline__ int ksw(int t) { return (t & 3) | ((t >> 2) & 4); }

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

    __shared__ u32x4 Ks4[kP * kD / 8];
    __shared__ float c32s[kD];
    __shared__ float ic32s[kD];
    __shared__ double red_sum[4];
    __shared__ int red_cnt[4];
    const uint16_t* Ks16 = reinterpret_cast<const uint16_t*>(Ks4);

    // Both pages are read as whole lines (each load instruction covers 1 KB
    // contiguous), non-temporal: the value page goes through LDS to give
    // thread d its channel row d (64 tokens, 128 bytes; piece k of row d at
    // d * 8 + (k ^ (d & 7)), so eight neighbouring rows spread over eight
    // bank groups), then the key page takes the same LDS.
    u32x4 kin[(kP * kD * 2) / (16 * 256)];
    uint32_t vw[32];
    {
        const u32x4* v4 = reinterpret_cast<const u32x4*>(V);
        const u32x4* k4 = reinterpret_cast<const u32x4*>(K);
        u32x4 vin[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) vin[k] = __builtin_nontemporal_load(v4 + tid + 256 * k);
#pragma unroll
        for (int k = 0; k < 8; ++k) kin[k] = __builtin_nontemporal_load(k4 + tid + 256 * k);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = tid + 256 * k, row = c >> 3;
            Ks4[row * 8 + ((c & 7) ^ (row & 7))] = vin[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const u32x4 x = Ks4[tid * 8 + (k ^ (tid & 7))];
            vw[4 * k + 0] = x.x;
            vw[4 * k + 1] = x.y;
            vw[4 * k + 2] = x.z;
            vw[4 * k + 3] = x.w;
        }
        __syncthreads();
        // the key page, token rows of 32 chunks, chunk c of row t at c ^ ksw(t)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = tid + 256 * k, row = c >> 5;
            Ks4[row * 32 + ((c & 31) ^ ksw(row))] = kin[k];
        }
    }

    // value scale and codes (thread d = channel d)
    {
        const int d = tid;
        // max |V| on the bit patterns: for non-negative floats the integer
        // order is the float order; a pattern above 0x7F80 is a NaN
        u16x2 mx = {0, 0};
#pragma unroll
        for (int k = 0; k < 32; ++k)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, vw[k] & 0x7FFF7FFFu));
        const uint32_t mb = mx.x > mx.y ? mx.x : mx.y;
        float vs32 = (float)((double)__uint_as_float(mb << 16) / 127.0);
        const bool fast = mb <= 0x7F80u && fast_scale(vs32);
        if (!fast) {  // NaNs take no part in the maximum
            double m = 0.0;
            for (int k = 0; k < 32; ++k) {
                m = fmax(m, fabs((double)bf16_lo(vw[k])));
                m = fmax(m, fabs((double)bf16_hi(vw[k])));
            }
            vs32 = (float)(m / 127.0);
        }
        vchan[dp * kD + d] = vs32;
        const float ivs = fast && vs32 != 0.0f ? (float)(1.0 / (double)vs32) : 0.0f;
        u32x4* out = reinterpret_cast<u32x4*>(vcodes + dp * (kP * kD) + (size_t)d * kP);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t wds[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int c[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * k + 4 * j + e;
                    const float x = (tok & 1) ? bf16_hi(vw[tok >> 1]) : bf16_lo(vw[tok >> 1]);
                    const float q = x * ivs;
                    const float r = __builtin_rintf(q);
                    c[e] = (int)r;
                    if (!fast || fabsf(q - r) > kNearHalf) c[e] = code_exact((double)x, (double)vs32);
                }
                wds[j] = pack4(c[0], c[1], c[2], c[3]);
            }
            out[k] = u32x4{wds[0], wds[1], wds[2], wds[3]};
        }
    }
    __syncthreads();

    // channel factor (thread d = channel d, reading down the LDS column)
    {
        const int d = tid;
        int col[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) col[f] = (((d >> 3) ^ f) << 3) | (d & 7);
        double ms = 0.0;
#pragma unroll
        for (int t = 0; t < kP; ++t) {
            const double k = (double)bf16_to_f32(Ks16[t * kD + col[ksw(t)]]);
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
        ic32s[d] = (float)(1.0 / (double)c32);
        kchan[dp * kD + d] = c32;
    }
    __syncthreads();

    // token factor and key codes: one token, 64 channels per thread
    {
        const int lane = tid & 63, w = tid >> 6, q4 = lane >> 4;
        const int t = 16 * ((lane >> 2) & 3) + 4 * w + (lane & 3);
        const int f = ksw(t);
        float y[64];  // x / c as x * (1/c), channel 64 j + 16 q4 + e at y[16 j + e]
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 xa = Ks4[t * 32 + ((8 * j + 2 * q4) ^ f)];
            const u32x4 xb = Ks4[t * 32 + ((8 * j + 2 * q4 + 1) ^ f)];
            const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const float4* ic4 = reinterpret_cast<const float4*>(&ic32s[64 * j + 16 * q4]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 ic = ic4[v];
                const float icv[4] = {ic.x, ic.y, ic.z, ic.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 4 * v + e;
                    const float x = (n & 1) ? bf16_hi(xw[n >> 1]) : bf16_lo(xw[n >> 1]);
                    y[16 * j + n] = x * icv[e];
                    m = fmaxf(m, fabsf(y[16 * j + n]));
                }
            }
        }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        float s32 = (float)((double)m / 127.0);
        const bool fast = fast_scale(s32);
        if (!fast) {  // the four lanes of this token take this branch together
            double md = 0.0;
            for (int n = 0; n < 64; ++n) {
                const int dd = 64 * (n >> 4) + 16 * q4 + (n & 15);
                const double x = (double)bf16_to_f32(Ks16[t * kD + ((((dd >> 3) ^ f) << 3) | (dd & 7))]);
                md = fmax(md, fabs(x) / (double)c32s[dd]);
            }
            md = fmax(md, __shfl_xor(md, 16, 64));
            md = fmax(md, __shfl_xor(md, 32, 64));
            s32 = (float)(md / 127.0);
        }
        if (q4 == 0) ktok[dp * kP + t] = s32;
        const float is = fast && s32 != 0.0f ? (float)(1.0 / (double)s32) : 0.0f;
        int8_t* out = kcodes + dp * (kP * kD);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t wds[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int c[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 4 * v + e;
                    const float q = y[16 * j + n] * is;
                    const float r = __builtin_rintf(q);
                    c[e] = (int)r;
                    if (!fast || fabsf(q - r) > kNearHalf) {
                        const int dd = 64 * j + 16 * q4 + n;
                        const double x = (double)bf16_to_f32(Ks16[t * kD + ((((dd >> 3) ^ f) << 3) | (dd & 7))]);
                        c[e] = code_exact(x, (double)c32s[dd] * (double)s32);
                    }
                }
                wds[v] = pack4(c[0], c[1], c[2], c[3]);
            }
            *reinterpret_cast<u32x4*>(out + kcode_offset(t, 64 * j + 16 * q4)) = u32x4{wds[0], wds[1], wds[2], wds[3]};
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
