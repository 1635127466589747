// lossless.hip -- the lossless 13-bit page tier ("Model quantization" page,
// "A lossless tier first"): BF16 pages to 13-bit planes and back.  Attention
// that reads the planes directly is decode_l13_kernel in decode.hip.
//
// A plane is one page of one KV head, keys or values (16,384 BF16 values).
// Its table lists the distinct high bytes (sign and upper seven exponent
// bits) in ascending order; each value keeps its low byte and the 5-bit
// position of its high byte.  More than 32 distinct high bytes: the plane is
// stored raw.  Planes are packed back to back in a byte arena in call order,
// so encoding takes three launches: tables and raw flags, offsets (one
// work-group scanning the plane sizes), then the planes themselves.
#include "akv_device.h"
#include "akv_host.h"

namespace akv {

constexpr int kL13Units = kL13PlaneBytes / 256;  // 104 arena units of 256 bytes
constexpr int kL13RawUnits = kL13RawBytes / 256;  // 128

// BF16 value v (0..63) of a lane's eight 16-byte registers in lane-slot
// order (register v / 8).
__device__ __forceinline__ uint16_t value_bits(const u32x4 (&x)[8], int v) {
    const u32x4 r = x[v >> 3];
    const int c = (v >> 1) & 3;
    const uint32_t wd = c == 0 ? r.x : c == 1 ? r.y : c == 2 ? r.z : r.w;
    return (uint16_t)((v & 1) ? wd >> 16 : wd & 0xFFFFu);
}

// Copy a whole 32 KB plane (raw records), 256 threads x 8 x 16 bytes.
__device__ __forceinline__ void copy_plane(uint8_t* out, const uint8_t* in, int tid) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int off = (k * 256 + tid) * 16;
        *reinterpret_cast<u32x4*>(out + off) = ld16(in + off);
    }
}

// Flag slot of high byte hb in LDS: one dword each, bit 4 of the slot index
// flipped for negative values so that the high bytes of +x and -x, which
// differ only in bit 7, sit in different banks.
__device__ __forceinline__ int flag_slot(uint32_t hb) { return (int)(hb ^ ((hb >> 3) & 16u)); }

// Pass 1, one work-group per plane: the plane's table and raw flag (the flag
// goes to the descriptor, which pass 2 completes).  Every value stores 1 into
// its high byte's flag (all writers store the same value, so no atomics);
// each wave then gathers 64 flags with a ballot.
__global__ __launch_bounds__(256) void l13_table_kernel(int Hkv, const uint16_t* kb, const uint16_t* vb,
                                                        const int32_t* src, const int32_t* dst, int32_t* desc,
                                                        uint8_t* table) {
    const int i = blockIdx.x, h = blockIdx.y, kv = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    __shared__ uint32_t flag[256];
    __shared__ uint32_t present[8];
    __shared__ uint32_t tab[8];
    flag[tid] = 0u;
    if (tid < 8) tab[tid] = 0u;
    // the set of high bytes does not depend on which thread reads which value:
    // read the plane as whole lines, non-temporal
    u32x4 x[8];
    {
        const u32x4* p4 = reinterpret_cast<const u32x4*>((kv ? vb : kb) + ((size_t)src[i] * Hkv + h) * (kP * kD));
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_nontemporal_load(p4 + tid + 256 * k);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t wd[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            flag[flag_slot((wd[e] >> 8) & 0xFFu)] = 1u;
            flag[flag_slot(wd[e] >> 24)] = 1u;
        }
    }
    __syncthreads();
    // wave w gathers high bytes 64 w .. 64 w + 63
    const unsigned long long bits = __ballot(flag[flag_slot((uint32_t)tid)] != 0u);
    if (l == 0) {
        present[2 * w] = (uint32_t)bits;
        present[2 * w + 1] = (uint32_t)(bits >> 32);
    }
    __syncthreads();
    // thread tid stands for high byte tid: its table position is the number of present bytes below it
    int count = 0, below = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t pk = present[k];
        count += __popc(pk);
        if (k < (tid >> 5)) below += __popc(pk);
    }
    const uint32_t mine = present[tid >> 5];
    if ((mine >> (tid & 31)) & 1u) {
        const int pos = below + __popc(mine & ((1u << (tid & 31)) - 1u));
        if (pos < 32) atomicOr(&tab[pos >> 2], (uint32_t)tid << (8 * (pos & 3)));
    }
    __syncthreads();
    const size_t plane = ((size_t)dst[i] * Hkv + h) * 2 + kv;
    const bool raw = count > 32;
    if (tid < 8) reinterpret_cast<uint32_t*>(table + plane * 32)[tid] = raw ? 0u : tab[tid];
    if (tid == 0) desc[plane] = raw ? 1 : 0;
}

// Pass 2, one work-group: exclusive prefix sum of the plane sizes in call
// order (page i, head h, keys then values) from unit0; each descriptor
// becomes (offset / 256) << 1 | raw, and *arena_end the end in bytes.
__global__ __launch_bounds__(1024) void l13_offsets_kernel(int n_planes, int Hkv, const int32_t* dst, int32_t* desc,
                                                           long long unit0, long long* arena_end) {
    __shared__ int wsum[16];
    __shared__ int chunk_total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    long long carry = unit0;
    for (int c0 = 0; c0 < n_planes; c0 += 1024) {
        const int idx = c0 + tid;
        int32_t* dp = nullptr;
        int raw = 0, u = 0;
        if (idx < n_planes) {
            const int i = idx / (2 * Hkv), rem = idx - i * (2 * Hkv);  // rem = 2h + kv
            dp = desc + (size_t)dst[i] * Hkv * 2 + rem;
            raw = *dp & 1;
            u = raw ? kL13RawUnits : kL13Units;
        }
        int v = u;  // inclusive scan within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(v, off, 64);
            if (lane >= off) v += t;
        }
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int k = 0; k < 16; ++k) {
                const int t = wsum[k];
                wsum[k] = acc;
                acc += t;
            }
            chunk_total = acc;
        }
        __syncthreads();
        if (dp) *dp = (int32_t)(((carry + wsum[wave] + v - u) << 1) | raw);
        carry += chunk_total;
        __syncthreads();  // wsum and chunk_total are rewritten by the next chunk
    }
    if (tid == 0) *arena_end = carry * 256;
}

// Pass 3, one work-group per plane: write the plane at its offset.
__global__ __launch_bounds__(256) void l13_encode_kernel(int Hkv, const uint16_t* kb, const uint16_t* vb,
                                                         const int32_t* src, const int32_t* dst, const int32_t* desc,
                                                         const uint8_t* table, uint8_t* arena) {
    const int i = blockIdx.x, h = blockIdx.y, kv = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const size_t plane = ((size_t)dst[i] * Hkv + h) * 2 + kv;
    const int d = desc[plane];
    uint8_t* out = arena + (size_t)(d >> 1) * 256;
    const uint16_t* in = (kv ? vb : kb) + ((size_t)src[i] * Hkv + h) * (kP * kD);
    if (d & 1) {
        copy_plane(out, reinterpret_cast<const uint8_t*>(in), tid);
        return;
    }
    __shared__ uint8_t pos[256];
    if (tid < 32) {
        const uint8_t e = table[plane * 32 + tid];
        if (tid == 0 || e != 0) pos[e] = (uint8_t)tid;  // entries past the distinct count are 0
    }
    __syncthreads();
    // the lane's values in lane-slot order, loaded straight into registers (an
    // LDS copy read as whole lines ran this pass slower: 206 against 173 us
    // per 128K layer)
    u32x4 x[8];
    {
        const int n = l & 15, g = l >> 4;
        if (kv == 0) {
#pragma unroll
            for (int r = 0; r < 8; ++r) x[r] = ld16(in + qk_row_token(r >> 1, n) * kD + 64 * w + 16 * g + 8 * (r & 1));
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) x[r] = ld16(in + (64 * w + 16 * (r >> 1) + n) * kP + 16 * g + 8 * (r & 1));
        }
    }
    uint32_t lowb[16], nib[8], hib[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) lowb[k] = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) nib[k] = 0u;
#pragma unroll
    for (int v = 0; v < 64; ++v) {
        const uint32_t b = value_bits(x, v);
        const uint32_t idx = pos[b >> 8];
        lowb[v >> 2] |= (b & 0xFFu) << (8 * (v & 3));
        nib[v >> 3] |= (idx & 15u) << (8 * (v & 3) + 4 * ((v >> 2) & 1));
        hib[v >> 5] |= (idx >> 4) << (8 * (v & 3) + ((v & 31) >> 2));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(out + l13_low_offset(w, l, q)) =
            u32x4{lowb[4 * q], lowb[4 * q + 1], lowb[4 * q + 2], lowb[4 * q + 3]};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<u32x4*>(out + l13_nibble_offset(w, l, hh)) =
            u32x4{nib[4 * hh], nib[4 * hh + 1], nib[4 * hh + 2], nib[4 * hh + 3]};
    *reinterpret_cast<u32x2*>(out + l13_high_offset(w, l)) = u32x2{hib[0], hib[1]};
}

// Record slots src[i] back to BF16 pool slots dst[i], with the decode
// kernel's own register expansion.
__global__ __launch_bounds__(256) void l13_expand_kernel(int Hkv, const uint8_t* arena, const int32_t* desc,
                                                         const uint8_t* table, const int32_t* src, const int32_t* dst,
                                                         uint16_t* kb, uint16_t* vb) {
    const int i = blockIdx.x, h = blockIdx.y, kv = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const size_t plane = ((size_t)src[i] * Hkv + h) * 2 + kv;
    const int d = desc[plane];
    const uint8_t* in = arena + (size_t)(d >> 1) * 256;
    uint16_t* out = (kv ? vb : kb) + ((size_t)dst[i] * Hkv + h) * (kP * kD);
    if (d & 1) {
        copy_plane(reinterpret_cast<uint8_t*>(out), in, tid);
        return;
    }
    uint32_t T[8];
    const uint32_t* tp = reinterpret_cast<const uint32_t*>(table + plane * 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) T[k] = tp[k];
    u32x4 c[8], x[8];
    l13_load(in, w, l, c);
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = l13_operand(c, T, r, l & 1);
    if (kv == 0)
        bf16_keys_store(out, w, l & 15, l >> 4, x);
    else
        bf16_values_store(out, w, l & 15, l >> 4, x);
}

static akv_status check_l13_common(const akv_dims* dims, int32_t n) {
    akv_status st = check_dims(dims);
    if (st != AKV_OK) return st;
    if (n < 0) return fail(AKV_ERR_ARG, "n = %d < 0", n);
    if ((long long)n * dims->num_kv_heads * 2 > (1LL << 30))
        return fail(AKV_ERR_ARG, "%d pages x %d heads: too many planes for one call", n, dims->num_kv_heads);
    return AKV_OK;
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_l13_encode_pages(const akv_dims* dims, int32_t n, const uint16_t* k_bf16,
                                           const uint16_t* v_bf16, const int32_t* src_slot, const int32_t* dst_slot,
                                           uint8_t* l13_arena, int64_t arena_offset, int64_t arena_bytes,
                                           int32_t* l13_desc, uint8_t* l13_table, int64_t* arena_end,
                                           void* stream) {
    clear_error();
    akv_status st = check_l13_common(dims, n);
    if (st != AKV_OK) return st;
    if (!arena_end) return fail(AKV_ERR_ARG, "NULL arena_end");
    if (n > 0 && (!k_bf16 || !v_bf16 || !src_slot || !dst_slot || !l13_arena || !l13_desc || !l13_table))
        return fail(AKV_ERR_ARG, "NULL pointer");
    if (!aligned(arena_end, 8) ||
        (n > 0 && (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(l13_table) || !aligned(l13_arena, 256) ||
                   !aligned(l13_desc, 4) || !aligned(src_slot, 4) || !aligned(dst_slot, 4))))
        return fail(AKV_ERR_ALIGN, "pointer alignment (tensors 16, arena 256, int32 arrays 4, arena_end 8 bytes)");
    if (arena_offset < 0 || arena_offset % 256 != 0 || arena_bytes < arena_offset)
        return fail(AKV_ERR_ARG, "arena_offset %lld must be a multiple of 256 in [0, arena_bytes = %lld]",
                    (long long)arena_offset, (long long)arena_bytes);
    const long long planes = (long long)n * dims->num_kv_heads * 2;
    const long long worst_end = arena_offset + planes * kL13RawBytes;
    if (worst_end > arena_bytes)
        return fail(AKV_ERR_BUDGET, "arena of %lld bytes cannot hold %lld planes from offset %lld (%lld bytes if raw)",
                    (long long)arena_bytes, planes, (long long)arena_offset, planes * kL13RawBytes);
    if (worst_end > (1LL << 38)) return fail(AKV_ERR_ARG, "arena offsets past 256 GiB do not fit a descriptor");
    hipStream_t s = (hipStream_t)stream;
    const int Hkv = dims->num_kv_heads;
    if (n > 0) {
        l13_table_kernel<<<dim3((unsigned)n, (unsigned)Hkv, 2), 256, 0, s>>>(Hkv, k_bf16, v_bf16, src_slot,
                                                                              dst_slot, l13_desc, l13_table);
        if ((st = launch_status("l13_table_kernel")) != AKV_OK) return st;
    }
    l13_offsets_kernel<<<1, 1024, 0, s>>>((int)planes, Hkv, dst_slot, l13_desc, arena_offset / 256,
                                          reinterpret_cast<long long*>(arena_end));
    if ((st = launch_status("l13_offsets_kernel")) != AKV_OK) return st;
    if (n == 0) return AKV_OK;
    l13_encode_kernel<<<dim3((unsigned)n, (unsigned)Hkv, 2), 256, 0, s>>>(Hkv, k_bf16, v_bf16, src_slot, dst_slot,
                                                                           l13_desc, l13_table, l13_arena);
    return launch_status("l13_encode_kernel");
}

extern "C" akv_status akv_l13_decode_pages(const akv_dims* dims, int32_t n, const uint8_t* l13_arena,
                                           const int32_t* l13_desc, const uint8_t* l13_table,
                                           const int32_t* src_slot, const int32_t* dst_slot, uint16_t* k_bf16,
                                           uint16_t* v_bf16, void* stream) {
    clear_error();
    akv_status st = check_l13_common(dims, n);
    if (st != AKV_OK) return st;
    if (n == 0) return AKV_OK;
    if (!k_bf16 || !v_bf16 || !src_slot || !dst_slot || !l13_arena || !l13_desc || !l13_table)
        return fail(AKV_ERR_ARG, "NULL pointer");
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(l13_table) || !aligned(l13_arena, 256) ||
        !aligned(l13_desc, 4) || !aligned(src_slot, 4) || !aligned(dst_slot, 4))
        return fail(AKV_ERR_ALIGN, "pointer alignment (tensors 16, arena 256, int32 arrays 4 bytes)");
    const int Hkv = dims->num_kv_heads;
    l13_expand_kernel<<<dim3((unsigned)n, (unsigned)Hkv, 2), 256, 0, (hipStream_t)stream>>>(
        Hkv, l13_arena, l13_desc, l13_table, src_slot, dst_slot, k_bf16, v_bf16);
    return launch_status("l13_expand_kernel");
}
