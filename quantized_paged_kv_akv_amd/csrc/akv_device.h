// akv_device.h -- device-side building blocks for the gfx950 kernels.
//
// Wave64 lane naming used by every kernel: l = lane (0..63), n = l & 15,
// g = l >> 4.  For the 16x16x32 MFMAs (f16 and bf16) the operands are laid out
// as on CDNA3/4: lane (n, g) holds row n of A and column n of B, each with the
// 8 contraction elements of group g; the 16x16 FP32 result gives lane (n, g)
// the four rows 4g..4g+3 of column n.  Only that result layout is relied on:
// which contraction index a group's elements stand for is chosen by the
// kernels, identically for A and B.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace akv {

constexpr int kD = 256;  // head dimension
constexpr int kP = 64;   // tokens per page
constexpr int kMaxGroup = 8;
constexpr int kThreads = 256;  // 4 waves; wave w owns channels [64w, 64w + 64)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load through the vector memory path (no scalar cache).
template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte load with the non-temporal (streaming) hint, for data read once
// in whole 64-byte runs (code tiles, per-page scales): on this part it moves
// the int8 pages 6-9% faster than the default policy.  Not for partial-line
// reads, whose other half the default policy keeps cached for the next
// instruction (there the hint costs as much as it gains elsewhere).
template <typename T>
__device__ __forceinline__ u32x4 ld16_stream(const T* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Byte offset of key code K[t][d] inside a page-head's 16 KB of codes in
// tile order: tile 4 (d / 64) + (t / 4) % 4 holds, for lane 16 g + n, the 16
// codes of token 16 (n / 4) + 4 ((t / 4) % 4) + n % 4 at channels
// 64 (d / 64) + 16 g .. + 16 -- exactly what that lane loads for QK.
__host__ __device__ __forceinline__ int kcode_offset(int t, int d) {
    const int tile = 4 * (d >> 6) + ((t >> 2) & 3);
    const int lane = 16 * ((d >> 4) & 3) + 4 * (t >> 4) + (t & 3);
    return (tile * 64 + lane) * 16 + (d & 15);
}

// Signed int8 codes -> exact FP16.  Each byte b is biased to b + 128 (xor
// 0x80), placed under the exponent byte 0x64 (FP16 0x64XX = 1024 + XX) with a
// byte permute, and the packed result minus 1152 is b exactly.
__device__ __forceinline__ half8 i8x8_to_f16(uint32_t w0, uint32_t w1) {
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    // v_perm_b32: bytes 0..3 come from the second operand, 4..7 from the first
    u32x4 r;
    r.x = __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u);
    r.y = __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u);
    r.z = __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u);
    r.w = __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u);
    half8 h = __builtin_bit_cast(half8, r);
    const half8 bias = {1152, 1152, 1152, 1152, 1152, 1152, 1152, 1152};
    return h - bias;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, ((uint32_t)b) << 16);
}

// Butterfly over the four lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}
__device__ __forceinline__ float group_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// The value held by the neighbouring lane of the pair (lanes 2i and 2i+1
// exchange; a DPP quad permutation [1,0,3,2]).
__device__ __forceinline__ float swap_pair(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}

// x = a*b rounded to FP32, split as hi + lo with hi = fp16(x) and
// lo = fp16(x - hi).  Contraction is off: fusing a*b into the conversions
// would round hi two different ways and break hi + lo ~ x.
__device__ __forceinline__ void split_prod_f16(float a, float b, _Float16& hi, _Float16& lo) {
#pragma clang fp contract(off)
    float x = a * b;
    asm volatile("" : "+v"(x));  // x is a rounded FP32 value: no mixed-precision fusion through it
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}
// Two at a time with the packed conversions (v_cvt_pk_f16_f32).
__device__ __forceinline__ void split_prod_f16x2(float a0, float b0, float a1, float b1, half2& hi, half2& lo) {
#pragma clang fp contract(off)
    float x0 = a0 * b0, x1 = a1 * b1;
    asm volatile("" : "+v"(x0), "+v"(x1));
    hi = half2{(_Float16)x0, (_Float16)x1};
    lo = half2{(_Float16)(x0 - (float)hi[0]), (_Float16)(x1 - (float)hi[1])};
}
__device__ __forceinline__ void split_f16x2(float x0, float x1, half2& hi, half2& lo) {
#pragma clang fp contract(off)
    hi = half2{(_Float16)x0, (_Float16)x1};
    lo = half2{(_Float16)(x0 - (float)hi[0]), (_Float16)(x1 - (float)hi[1])};
}
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
#pragma clang fp contract(off)
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
#pragma clang fp contract(off)
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace akv
