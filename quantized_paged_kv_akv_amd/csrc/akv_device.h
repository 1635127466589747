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
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_f16(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x64 int8 MFMA: 16 signed bytes of A and of B per lane, exact int32 sums.
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0,
                                                 0, 0);
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

// Eight signed int8 codes (w0 bytes 0..3, then w1) -> exact FP16, in order:
// one sub-dword conversion per code that sign-extends its byte (every int8
// value is an FP16 integer) and writes one half of a result register; one
// instruction per code against 1.25 for a byte permute under an FP16 exponent
// byte and a packed bias subtraction (4 us less per 16-layer 32K step,
// bit-identical results).  On gfx950 an instruction that writes part of a
// register must not be followed at once by one that reads that register, and
// the compiler cannot space instructions inside an asm block: so the four low
// halves are written first, the four high halves (which keep the low ones)
// after them, and a closing s_nop keeps the last write one instruction away
// from its first reader.  (Written as pairs, each high-half write right after
// its low half, the outputs went wrong as soon as the waves' issue priorities
// were changed.)
__device__ __forceinline__ half8 i8x8_to_f16(uint32_t w0, uint32_t w1) {
    uint32_t r0, r1, r2, r3;
    asm("v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
        "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
        "s_nop 0"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(w0), "v"(w1));
    const u32x4 r = {r0, r1, r2, r3};
    return __builtin_bit_cast(half8, r);
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

// An FP32 operand x enters a half-precision MFMA as hi + lo with
// hi = fp16(x) and lo = fp16(x - hi), the two parts in neighbouring columns.
// A lane takes the hi part when m = 0 and the lo part when m = 1: x - m * hi
// is exact either way (hi keeps the leading bits of x), so no select is needed.
__device__ __forceinline__ half2 split_sel_f16x2(float x0, float x1, float m) {
#pragma clang fp contract(off)
    const half2 hi = half2{(_Float16)x0, (_Float16)x1};
    return half2{(_Float16)__builtin_fmaf(-m, (float)hi[0], x0), (_Float16)__builtin_fmaf(-m, (float)hi[1], x1)};
}
// The same for x = a*b rounded to FP32.  Contraction is off and the product
// is pinned: fusing a*b into the conversions would round hi two different
// ways and break hi + lo ~ x.
__device__ __forceinline__ half2 split_prod_sel_f16x2(float a0, float b0, float a1, float b1, float m) {
#pragma clang fp contract(off)
    float x0 = a0 * b0, x1 = a1 * b1;
    asm volatile("" : "+v"(x0), "+v"(x1));  // rounded FP32 values: no mixed-precision fusion through them
    return split_sel_f16x2(x0, x1, m);
}
// BF16 parts: bf16(x) for m = 0, bf16(x - bf16(x)) for m = 1.
__device__ __forceinline__ __bf16 split_sel_bf16(float x, float m) {
#pragma clang fp contract(off)
    const __bf16 hi = (__bf16)x;
    return (__bf16)__builtin_fmaf(-m, (float)hi, x);
}

// Exact-tier page order: QK tile t, A-operand row i is token
// 16 (i / 4) + 4 t + i % 4 of the page.
__host__ __device__ __forceinline__ int qk_row_token(int t, int i) { return 16 * (i >> 2) + 4 * t + (i & 3); }

// Lane-slot order of a BF16 page-head (the exact body's MFMA operands, and
// the order in which 13-bit planes are stored): register 2t + s of lane
// (w, n, g) holds key token qk_row_token(t, n) at channels 64w + 16g + 8s .. + 8;
// register 2j + s holds value channel 64w + 16j + n at tokens 16g + 8s .. + 8.
// These stores write a lane's registers to a BF16 page-head in that order.
__device__ __forceinline__ void bf16_keys_store(uint16_t* kp, int w, int n, int g, const u32x4 (&K)[8]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            *reinterpret_cast<u32x4*>(kp + qk_row_token(t, n) * kD + 64 * w + 16 * g + 8 * s) = K[2 * t + s];
}
__device__ __forceinline__ void bf16_values_store(uint16_t* vp, int w, int n, int g, const u32x4 (&V)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            *reinterpret_cast<u32x4*>(vp + (64 * w + 16 * j + n) * kP + 16 * g + 8 * s) = V[2 * j + s];
}

// ---------------------------------------------------------------- 13-bit planes
// Lossless 13-bit plane ("Model quantization" page, "A lossless tier first"):
// each BF16 value is the 5-bit position of its high byte (sign and upper
// seven exponent bits) in the plane's 32-entry table, plus its low byte.
// Storage follows the lane that consumes the value: lane slot (w, l, v) --
// wave w, lane l, value v < 64 of that lane -- is, for a key plane, token
// 16 (n / 4) + 4 (v / 16) + n % 4 at channel 64 w + 16 g + 8 ((v / 8) % 2)
// + v % 8, and for a value plane channel 64 w + 16 ((v / 16) % 4) + n at
// token 16 g + 8 ((v / 8) % 2) + v % 8 (n = l % 16, g = l / 16): the 8
// values of operand register r = v / 8 are exactly what the BF16 pool's
// 16-byte load r gives that lane in the exact tier's body.
// A coded plane is 26,624 bytes: 16 KB of low bytes, 8 KB of index nibbles,
// 2 KB of index bit 4.
constexpr int kL13PlaneBytes = 26624;
constexpr int kL13RawBytes = kP * kD * 2;
constexpr int kL13NibbleBase = 16384;
constexpr int kL13HighBase = 24576;

// Byte offsets of lane (w, l)'s chunks: low bytes chunk q < 4 (values
// 16q .. 16q + 15), nibble chunk h < 2 (values 32h .. 32h + 31; u32 word k
// holds values 32h + 8k + b in the low nibble of byte b and 32h + 8k + 4 + b
// in the high nibble), index bit 4 (u32 word k < 2 covers values 32k ..
// 32k + 31: value 32k + i sits at bit 8 (i % 4) + i / 4).
__host__ __device__ __forceinline__ int l13_low_offset(int w, int l, int q) { return ((4 * w + q) * 64 + l) * 16; }
__host__ __device__ __forceinline__ int l13_nibble_offset(int w, int l, int h) {
    return kL13NibbleBase + ((2 * w + h) * 64 + l) * 16;
}
__host__ __device__ __forceinline__ int l13_high_offset(int w, int l) { return kL13HighBase + (w * 64 + l) * 8; }

// Byte offset of the 16 bytes lane (w, l) loads into register r of a coded
// plane: low-byte chunks (r < 4), nibble chunks (r = 4, 5), and for r >= 6
// the aligned 16 bytes holding the index-bit-4 words of lanes l & ~1 and
// l | 1 (the lane's own 8 bytes are the first half for even l, the second
// for odd l).  Every load stays inside the plane's 26,624 bytes.
__host__ __device__ __forceinline__ int l13_chunk_offset(int w, int l, int r) {
    return r < 4 ? l13_low_offset(w, l, r) : r < 6 ? l13_nibble_offset(w, l, r - 4) : l13_high_offset(w, l & ~1);
}

// A lane's coded values: c[0..3] low-byte chunks, c[4..5] nibble chunks,
// c[6] index bit 4 of values 0..31 / 32..63 in .x / .y (even lanes) or
// .z / .w (odd lanes); c[7] is not used.
__device__ __forceinline__ void l13_load(const uint8_t* plane, int w, int l, u32x4 (&c)[8]) {
#pragma unroll
    for (int r = 0; r < 7; ++r) c[r] = ld16_stream(plane + l13_chunk_offset(w, l, r));
    c[7] = c[6];
}

// Table entry per byte: byte b of the result is T[idx_b] (idx_b < 32), with
// the table as 8 little-endian words.  Three levels of byte permutes: the
// low three index bits pick within 8-entry groups, bits 3 and 4 pick groups.
__device__ __forceinline__ uint32_t l13_lookup(const uint32_t (&T)[8], uint32_t idx) {
    const uint32_t sel = idx & 0x07070707u;
    const uint32_t p0 = __builtin_amdgcn_perm(T[1], T[0], sel);
    const uint32_t p1 = __builtin_amdgcn_perm(T[3], T[2], sel);
    const uint32_t p2 = __builtin_amdgcn_perm(T[5], T[4], sel);
    const uint32_t p3 = __builtin_amdgcn_perm(T[7], T[6], sel);
    const uint32_t s3 = ((idx >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t q0 = __builtin_amdgcn_perm(p1, p0, s3);
    const uint32_t q1 = __builtin_amdgcn_perm(p3, p2, s3);
    const uint32_t s4 = ((idx >> 2) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(q1, q0, s4);
}

// Bit j (0..7) of each byte of H moved to bit 4.
__device__ __forceinline__ uint32_t l13_bit4(uint32_t H, int j) {
    return (j <= 4 ? H << (4 - j) : H >> (j - 4)) & 0x10101010u;
}

// BF16 operand register r (values 8r .. 8r + 7 of the lane) of a coded
// plane; odd = lane index is odd.
__device__ __forceinline__ u32x4 l13_operand(const u32x4 (&c)[8], const uint32_t (&T)[8], int r, bool odd) {
    const u32x4 lo = c[r >> 1];
    const uint32_t L0 = (r & 1) ? lo.z : lo.x;
    const uint32_t L1 = (r & 1) ? lo.w : lo.y;
    const u32x4 nb = c[4 + (r >> 2)];
    const int k = r & 3;
    const uint32_t N = k == 0 ? nb.x : k == 1 ? nb.y : k == 2 ? nb.z : nb.w;
    const uint32_t H = (r >> 2) ? (odd ? c[6].w : c[6].y) : (odd ? c[6].z : c[6].x);
    const uint32_t i0 = (N & 0x0F0F0F0Fu) | l13_bit4(H, 2 * k);
    const uint32_t i1 = ((N >> 4) & 0x0F0F0F0Fu) | l13_bit4(H, 2 * k + 1);
    const uint32_t E0 = l13_lookup(T, i0), E1 = l13_lookup(T, i1);
    // value pairs: low byte from L, high byte from E
    return u32x4{__builtin_amdgcn_perm(E0, L0, 0x05010400u), __builtin_amdgcn_perm(E0, L0, 0x07030602u),
                 __builtin_amdgcn_perm(E1, L1, 0x05010400u), __builtin_amdgcn_perm(E1, L1, 0x07030602u)};
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace akv
