// decode.hip -- single-query paged decode over int8 pages and over BF16
// pages, split-K across pages with a log-sum-exp second pass.
//
// int8 tier ("SYCL" page, "Attention that reads 8-bit history"): the key
// channel factor is folded into the query per page (q' = q (.) c), the
// per-token key factor multiplies the finished dot product, the softmax
// weights multiply the raw value codes, and the per-channel value scale is
// applied to the page's PV result at the page boundary.
// Exact tier ("SYCL" page, "A merge that joins the tiers"): BF16 decode that
// also returns the log-sum-exp, -inf for an empty range.  The same body
// reads the lossless 13-bit planes ("Model quantization" page, "A lossless
// tier first"), expanding each operand register to BF16 right before its
// MFMA, so its results are bit-identical to the BF16 pages'.
//
// QK is S^T (tokens x heads) = K Q^T and PV is O^T (channels x heads) =
// V^T P^T, with V stored channel-major so 16 bytes of a value row are one PV
// operand (int8 tiles are loaded straight into operand registers; BF16 pages
// are loaded in whole lines and their operands rebuilt through LDS, see
// Bf16Source).  The exact tier contracts both on 16x16x32 BF16 MFMAs.  The
// int8 tier runs QK on 16x16x32 FP16 MFMAs (int8 codes become FP16 exactly)
// and PV on 16x16x64 int8 MFMAs against the raw value codes.  The 16 MFMA
// columns carry each query head twice: an FP32 operand (q' for the int8 tier,
// the softmax weights P for the exact tier) is fed as a high and a low
// half-precision part in one MFMA and the two halves of the result are added
// afterwards; the int8 tier's weights go in as fixed-point limbs (see
// kPvI8), two in one operand's column pair and a third in a second operand.
//
// Work decomposition.  int8 tier: one wave owns whole pages (no barrier per
// page); a work-group's four waves share a range of one (request, KV head)'s
// pages and merge once at the end (details above int8_split).  Exact tier: a
// work-group owns a range of pages and wave w owns channels [64w, 64w+64);
// the four waves' partial logits meet in LDS once per page.
//
// Token order inside a page: A-operand row i of QK tile t is token
// 16*(i>>2) + 4t + (i&3).  The MFMA result then gives lane group g the tokens
// 16g .. 16g+15 across the four tiles, which is exactly the contraction slice
// group g holds for PV (tokens 16g + 8s + e), so P goes from the QK result to
// the PV operand without leaving the lane.
//
// Softmax runs in base 2 (logits scaled by log2 e); LSE is returned in
// natural log.  Each split writes a normalised partial (O, LSE) to the
// workspace; the second pass (launch_combine) folds them exactly.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "akv_device.h"
#include "akv_host.h"

#include <hip/hip_ext.h>

namespace akv {

struct Int8Args {
    const uint16_t* q;
    const int8_t* kc;
    const int8_t* vc;
    const float* kchan;
    const float* ktok;
    const float* vchan;
    const int32_t* page_table;
    const int32_t* n_pages;
    int max_pages, Hkv, G;
    int splits;        // work-groups per (request, KV head): split s reads pages [s np / splits, (s+1) np / splits)
    int col0, n_cols;  // this tier's first partial column and the partial row stride
    float scale_log2;
    float* part_o;
    float* part_lse;
};

// The int8 tier's first reads (the page count and the first page-table
// entry) and its share arithmetic need only the page table, the page counts,
// the table's row length and the split count.  The kernels take these four
// again as leading scalar arguments, ahead of the argument structs, because
// the library is built with kernel-argument preloading: leading scalar
// arguments arrive in scalar registers when the wave starts, so the first
// reads go out without waiting for a kernel-argument load (a struct argument
// is never preloaded).
__device__ __forceinline__ Int8Args with_lead(Int8Args a, const int32_t* page_table, const int32_t* n_pages,
                                              int max_pages, int splits) {
    a.page_table = page_table;
    a.n_pages = n_pages;
    a.max_pages = max_pages;
    a.splits = splits;
    return a;
}

struct ExactArgs {
    const uint16_t* q;
    const uint16_t* kb;
    const uint16_t* vb;
    const int32_t* page_table;
    const int32_t* seq_len;
    int max_pages, Hkv, G, pps;
    int col0, n_cols;
    float scale_log2;
    float* part_o;
    float* part_lse;
};

// Wave issue-priority probe of akv_set_launch_shape, a template argument of
// the decode bodies (the default instantiation, 0, carries no code for it):
// 1 sets each wave's priority from the pages it has left, 2 from its index in
// the work-group.
constexpr int kPrioOff = 0, kPrioPagesLeft = 1, kPrioWave = 2;

// The wave's issue priority (s_setprio takes only an immediate).  Used by the
// scheduling probe of akv_set_launch_shape, which perturbs how the waves of a
// compute unit interleave without changing what any wave computes.
__device__ __forceinline__ void set_issue_priority(int level) {
    switch (level) {
        case 0: __builtin_amdgcn_s_setprio(0); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        default: __builtin_amdgcn_s_setprio(3); break;
    }
}

// LDS of the exact tier's body
struct ExactSmem {
    float part[2][4][16][64];  // QK partial logits of the four waves, double-buffered
};

// LDS of the BF16 operand source: per wave, its 64-channel quarter of a page's
// K, then of its V (64 rows of eight 16-byte pieces)
struct Bf16Stage {
    u32x4 q[4][512];
};

// Sum the four waves' partial logits for this lane: tile t, row r is token
// 16g + 4t + r of the page.
__device__ __forceinline__ void gather_logits(const float (*part)[16][64], int l, float S[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) S[k] = part[0][k][l] + part[1][k][l] + part[2][k][l] + part[3][k][l];
}

// Online-softmax step on this lane's 16 base-2 logits (masked = -inf):
// returns alpha (rescale of previous state) and writes P.  The weights come
// from the hardware base-2 exponential (v_exp_f32) without the library's
// denormal range fix-up: a weight below 2^-126 may become 0, far below what
// the FP32 sums of weights around 1 can resolve.
__device__ __forceinline__ float softmax_step(const float z[16], float& M, float& lsum, float p[16]) {
    float pm = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) pm = fmaxf(pm, z[k]);
    pm = group_max(pm);
    const float Mn = fmaxf(M, pm);
    const float alpha = __builtin_amdgcn_exp2f(M - Mn);
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        p[k] = __builtin_amdgcn_exp2f(z[k] - Mn);
        ps += p[k];
    }
    lsum = lsum * alpha + ps;
    M = Mn;
    return alpha;
}

// As softmax_step, with the running reference rounded up to an integer
// (base 2): every rescale factor is an exact power of two, and it is exactly
// 1 whenever the page does not lift the reference past the next integer.
// ("SYCL" page, "Exact tricks and a two-owner decoder".)
__device__ __forceinline__ float softmax_step_int(const float z[16], float& M, float& lsum, float p[16]) {
    float pm = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) pm = fmaxf(pm, z[k]);
    pm = group_max(pm);
    const float Mn = fmaxf(M, ceilf(pm));
    const float alpha = __builtin_amdgcn_exp2f(M - Mn);
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        p[k] = __builtin_amdgcn_exp2f(z[k] - Mn);
        ps += p[k];
    }
    lsum = lsum * alpha + ps;
    M = Mn;
    return alpha;
}

// P^T operand element (s, e) is token 16g + 8s + e = QK tile 2s + (e>>2), row e&3.
__device__ __forceinline__ float p_elem(const float p[16], int s, int e) {
    return p[(2 * s + (e >> 2)) * 4 + (e & 3)];
}

// Normalise, add the hi/lo halves and write this split's partial.
__device__ __forceinline__ void write_partial(f32x4 O[4], float M, float lsum, bool valid, bool hi_lane,
                                              int w, int g, size_t row, int n_cols, int col,
                                              float* __restrict__ part_o, float* __restrict__ part_lse) {
    const float L = group_sum(lsum);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[j][r] += __shfl_xor(O[j][r], 8, 64);
    if (valid && hi_lane) {
        const float inv = 1.0f / L;
        float* dst = part_o + (row * n_cols + col) * kD + 64 * w + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j) = O[j] * inv;
        if (w == 0 && g == 0) part_lse[row * n_cols + col] = (M + log2f(L)) * kLn2;
    }
}

// A split with no pages still owns its partial slot: mark it empty.
__device__ __forceinline__ void write_empty(int G, int Hkv, int kvh, int b, int n_cols, int col,
                                            float* __restrict__ part_lse) {
    const int t = threadIdx.x;
    if (t < G) part_lse[((size_t)b * Hkv * G + (size_t)kvh * G + t) * n_cols + col] = -INFINITY;
}

// ---------------------------------------------------------------- int8 tier
// One wave owns whole pages, so a page needs no barrier and its softmax is
// computed once.  Per page, lane (n, g) of the wave:
//   QK   tile t (16 tokens) x channel block s2 (64 channels): the lane's
//        16-byte load K[16(n>>2) + 4t + (n&3)][64 s2 + 16g .. +16] (bytes
//        [1024 (4 s2 + t) + 16 lane, +16) of the tile-ordered page, so a
//        load instruction reads 1 KB contiguous) is the A operand of two
//        k-steps; the B operand is q' = q (.) c of head n>>1
//        over the same channels, its FP16 hi part in even columns and its lo
//        part in odd ones; a pair of adjacent lanes adds the two results.
//        32 MFMAs.
//   softmax over the lane's 16 logits (tokens 16g .. 16g+15) and the group.
//   PV   channel tile j: the lane's 16-byte load V^T[16j + n][16g .. +16] is
//        the A operand of one int8 k-step over the page's 64 tokens, P^T the
//        B operand as limbs of head n>>1 (two int8 MFMAs: limbs 0 and 1, then
//        limb 2).  32 MFMAs.
// Code tiles stream with the non-temporal hint (each is read once, in whole
// lines).  The query's FP32 rows sit in LDS; each query row is pre-scaled by a power
// of two so max|q| < 1, which with max_d c_d >= 1 (the factors multiply to
// one) keeps every q' inside FP16's range.  The next page's codes are loaded
// into the registers the current page frees as it consumes them; its scales
// go to the other half of a per-wave LDS double buffer.  A work-group owns a
// near-equal share of one (request, KV head)'s pages; its four waves take
// every fourth page of it and merge once at the end.
struct alignas(16) Int8Smem {  // 16-byte aligned: its f32x4 rows move as 16-byte LDS accesses
    float q[kMaxGroup][kD + 4];    // query rows (scaled by 2^-e per row), FP32; +4 spreads rows over banks
    float qe[kMaxGroup];           // the row's power-of-two exponent e
    float sc[4][2][2 * kD + kP];   // per wave, per slot: k_chan | v_chan | k_tok * scale_log2
    int slot[4][kMaxPagesPerWave]; // pool slots of each wave's pages
    float mo[4][kMaxGroup][kD + 4];  // end merge: each wave's unnormalised O (padded like q)
    float mm[4][kMaxGroup];        // ... its running max (base 2)
    float ml[4][kMaxGroup];        // ... its sum of weights
};

// The PV operand of the int8 tier comes in two forms ("SYCL" page, "Attention
// that reads 8-bit history": which products run on integers was decided by
// measurement):
//   kPvI8   the weights P <= 1 as Y = rint(P (2^21 - 1)), split into three
//           7-bit limbs (Y = 2^14 l0 + 2^7 l1 + l2), against the raw value
//           codes on the int8 MFMA: exact int32 sums, no code conversion;
//   kPvF16  P as FP16 hi + lo against the value codes turned into FP16.
// The int8 form is the default; the FP16 form stays selectable for A/B runs.
constexpr int kPvF16 = 0;
constexpr int kPvI8 = 3;

// InOrder: a scheduling barrier after each PV tile keeps the products in
// tile order.  The scheduler otherwise pulls a later value tile's product
// next to the first one, so that point waits for 13 of the wave's 16 loads
// in flight.  It pays when one work-group holds a CU and four waves' loads
// in flight bound the stream (32K: 294 against 298 us per step); with two
// work-groups per CU the scheduler's order runs faster (128K: 813 against
// 817 us), so the launch picks by the size of the grid.
template <int PvLimbs, int Prio, bool InOrder = false>
__device__ __forceinline__ void int8_split(const Int8Args& a, Int8Smem& sm, int split, int kvh, int b) {
    // The wave's first page-table entry if the request fills its table row
    // (the usual single-request case), read beside the page count rather than
    // after it: one dependent round trip less before the first page streams
    // (1.3 us less per 128K step).  The entry is used only if the real share
    // starts where this guess does; the read stays inside the table row.
    const int w_s = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wg0_s = (int)((uint32_t)split * (uint32_t)a.max_pages / (uint32_t)a.splits);
    int spec_slot = 0;
    if (a.max_pages > 0)
        spec_slot = a.page_table[(size_t)b * a.max_pages + min(wg0_s + w_s, a.max_pages - 1)];
    const int np = min(a.n_pages[b], a.max_pages);
    // this work-group's pages [wg0, wg0 + len): a near-equal share of the
    // request's, in 32-bit arithmetic (the host refuses plans whose
    // splits x max_pages reaches 2^32; the 64-bit divisions cost about 380
    // scalar instructions before the first page-table read, 6 us per 128K
    // step)
    const int wg0 = (int)((uint32_t)split * (uint32_t)np / (uint32_t)a.splits);
    const int len = (int)((uint32_t)(split + 1) * (uint32_t)np / (uint32_t)a.splits) - wg0;
    if (len <= 0) {
        write_empty(a.G, a.Hkv, kvh, b, a.n_cols, a.col0 + split, a.part_lse);
        return;
    }
    const int tid = threadIdx.x, l = tid & 63, n = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    if constexpr (Prio == kPrioWave) set_issue_priority(w);
    const int G = a.G, Hkv = a.Hkv, Hq = Hkv * G;
    // MFMA column n carries head n >> 1: the FP16 hi part in even columns, the
    // lo part in odd ones (adjacent lanes add them back together)
    const int hh = n >> 1;
    const bool lo_lane = (n & 1) != 0;
    const float lo_m = lo_lane ? 1.0f : 0.0f;
    // int8 PV limbs: limb 0 in even columns and limb 1 in odd columns of the
    // first operand, limb 2 in odd columns of the second (its even columns are
    // zero); an even lane accumulates 128 l0-sums, an odd lane 128 l1-sums +
    // l2-sums, and the end merge weighs the pair 128 : 1 over 2^21 - 1
    constexpr float pv_scale = 2097151.0f;
    const uint32_t pv_shift = lo_lane ? 7u : 14u;
    const uint32_t pv_mask_b = lo_lane ? 0x7Fu : 0u;
    // wave w reads the work-group's pages w, w + 4, w + 8, ...: at any moment
    // the four waves stream neighbouring pages, which the memory system serves
    // better than four distant ranges.  The loop runs p = pa .. pb - 1 over
    // the wave's own page count; page p is table entry pt_index(p - pa).
    const int cnt = len > w ? (len - w + 3) / 4 : 0;
    const int pa = wg0 + w, pb = pa + cnt;
    auto pt_index = [&](int i) { return pa + 4 * i; };
    // per-lane byte offsets inside a page; tile offsets are immediates
    const uint32_t koff = (uint32_t)(16 * l);  // K codes in tile order: tile i is bytes [1024 i, 1024 i + 1024)
    const uint32_t voff = (uint32_t)(n * kP + 16 * g);
    const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
    const size_t row0 = (size_t)b * Hq + (size_t)kvh * G;

    // Requests go out in the order they are needed: this wave's two query
    // rows, its page slots, then the first page's scales and codes; the
    // query staging below waits only for the first of them and overlaps the
    // rest.
    const int r0 = w, r1 = w + 4;  // query rows staged by this wave
    u32x2 qraw0 = {0, 0}, qraw1 = {0, 0};
    if (r0 < G) qraw0 = *reinterpret_cast<const u32x2*>(a.q + (row0 + r0) * kD + 4 * l);
    if (r1 < G) qraw1 = *reinterpret_cast<const u32x2*>(a.q + (row0 + r1) * kD + 4 * l);
    // No branch may surround a load from here to the first page: after a
    // branch that issued loads the compiler waits for every outstanding load
    // at the join, so the first page's QK would wait for all of its ring
    // (15 us per 32K step).  Every wave therefore issues the same loads, from
    // indices clamped into this work-group's pages.
    //
    // this wave's page slots (at most 64), read once; lanes past the count
    // read the work-group's last entry
    const int last = wg0 + len - 1;
    const int my_slot = pt[min(pt_index(l), last)];
    u32x4 buf[16];
    u32x4 sk0, sv0;
    float st0;
    {
        // the first page's scales, then its codes (its QK needs the scales
        // first); a wave without pages reads the work-group's last page and
        // ignores it
        const int s0 = (wg0 == wg0_s && cnt > 0) ? spec_slot : pt[min(pt_index(0), last)];
        const size_t sb = (size_t)__builtin_amdgcn_readfirstlane(s0) * Hkv + kvh;
        const int8_t* kp = a.kc + sb * (kP * kD);
        sk0 = ld16_stream(a.kchan + sb * kD + 4 * l);
        sv0 = ld16_stream(a.vchan + sb * kD + 4 * l);
        st0 = __builtin_nontemporal_load(a.ktok + sb * kP + l);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int t = 0; t < 4; ++t) buf[4 * s2 + t] = ld16_stream(kp + koff + 1024 * (4 * s2 + t));
    }
    if (l < cnt) sm.slot[w][l] = my_slot;

    // query rows of this KV head, FP32, each scaled by 2^-e (e from its max |q|);
    // rows G..7 are zero (the MFMA columns they feed are never read)
    auto stage_row = [&](int r, u32x2 raw) {
        f32x4 v = {bf16_to_f32((uint16_t)(raw.x & 0xFFFFu)), bf16_to_f32((uint16_t)(raw.x >> 16)),
                   bf16_to_f32((uint16_t)(raw.y & 0xFFFFu)), bf16_to_f32((uint16_t)(raw.y >> 16))};
        float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        int e = 0;
        (void)frexpf(mx, &e);
        *reinterpret_cast<f32x4*>(&sm.q[r][4 * l]) =
            f32x4{ldexpf(v.x, -e), ldexpf(v.y, -e), ldexpf(v.z, -e), ldexpf(v.w, -e)};
        if (l == 0) sm.qe[r] = (float)e;
    };
    stage_row(r0, qraw0);  // zero rows stay zero: frexp(0) gives e = 0
    stage_row(r1, qraw1);
    __syncthreads();
    const float qsc = ldexpf(1.0f, (int)sm.qe[hh]);  // undoes the staging scale of this lane's head

    float M = -INFINITY, lsum = 0.0f;
    f32x4 O[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) O[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if (cnt > 0) {
        // One 16-entry register buffer cycles through a page's data: K tiles of
        // the wave's page i are replaced by its V tiles as QK consumes them, and
        // V tiles by the K tiles of page i+1 as PV consumes them (half a page
        // of lead).
        auto page_base = [&](int p) -> size_t {
            return (size_t)__builtin_amdgcn_readfirstlane(sm.slot[w][p - pa]) * Hkv + kvh;
        };
        *reinterpret_cast<u32x4*>(&sm.sc[w][0][4 * l]) = sk0;
        *reinterpret_cast<u32x4*>(&sm.sc[w][0][kD + 4 * l]) = sv0;
        sm.sc[w][0][2 * kD + l] = st0 * a.scale_log2;

        auto page = [&](auto prefetch, int p) {
            constexpr bool PF = decltype(prefetch)::value;
            if constexpr (Prio == kPrioPagesLeft) set_issue_priority(min(3, pb - p - 1));
            const int slot = (p - pa) & 1;
            const float* scl = sm.sc[w][slot];
            size_t nb = 0, ns = 0;
            u32x4 skn, svn;
            float stn = 0.0f;
            const int8_t* knp = a.kc;
            const int8_t* vcp = a.vc + page_base(p) * (kP * kD);
            if (PF) {
                ns = page_base(p + 1);
                nb = ns * (kP * kD);
                knp = a.kc + nb;
                skn = ld16_stream(a.kchan + ns * kD + 4 * l);
                svn = ld16_stream(a.vchan + ns * kD + 4 * l);
                stn = __builtin_nontemporal_load(a.ktok + ns * kP + l);
            }
            // S^T over all 256 channels: q' = q (.) c, hi + lo
            f32x4 S[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) S[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const f32x4* qr = reinterpret_cast<const f32x4*>(&sm.q[hh][64 * s2 + 16 * g]);
                const f32x4* cr = reinterpret_cast<const f32x4*>(&scl[64 * s2 + 16 * g]);
                half8 qb[2];  // the hi or the lo part of q', by column
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 qq = qr[i4], cc = cr[i4];
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const half2 v = split_prod_sel_f16x2(qq[e], cc[e], qq[e + 1], cc[e + 1], lo_m);
                        const int ix = 4 * i4 + e;
                        qb[ix >> 3][ix & 7] = v[0];
                        qb[ix >> 3][(ix & 7) + 1] = v[1];
                    }
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const u32x4 kk = buf[4 * s2 + t];
                    S[t] = mfma_f16(i8x8_to_f16(kk.x, kk.y), qb[0], S[t]);
                    S[t] = mfma_f16(i8x8_to_f16(kk.z, kk.w), qb[1], S[t]);
                    buf[4 * s2 + t] = ld16_stream(vcp + voff + 16 * (4 * s2 + t) * kP);  // this page's V tile
                }
            }
            // hi + lo: both lanes of a column pair end with the same sum
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] += swap_pair(S[t][r]);
            // logits (base 2): the token factor multiplies the finished dot product
            const f32x4* tk = reinterpret_cast<const f32x4*>(&scl[2 * kD + 16 * g]);
            float z[16], pr[16];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 tt = tk[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) z[4 * t + r] = S[t][r] * (tt[r] * qsc);
            }
            const float alpha = softmax_step_int(z, M, lsum, pr);
            // every column's rescale factor is exactly 1 on most pages: skip it
            const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
            half8 pbo[2];
            u32x4 pla = {0, 0, 0, 0}, plb = {0, 0, 0, 0};
            if constexpr (PvLimbs == kPvF16) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const half2 v = split_sel_f16x2(p_elem(pr, s, e), p_elem(pr, s, e + 1), lo_m);
                        pbo[s][e] = v[0];
                        pbo[s][e + 1] = v[1];
                    }
            } else {
                // Y = rint(p (2^21 - 1)), read from the mantissa of p S + 2^23
                // (p <= 1, so the sum stays in [2^23, 2^24) where the ulp is 1).
                // Operand byte i is token 16g + i, the order of the value row.
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t wa = 0, wb = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t y = __builtin_bit_cast(uint32_t, __builtin_fmaf(pr[4 * k + e], pv_scale, 8388608.0f));
                        wa |= __builtin_amdgcn_ubfe(y, pv_shift, 7) << (8 * e);
                        wb |= (y & pv_mask_b) << (8 * e);
                    }
                    pla[k] = wa;
                    plb[k] = wb;
                }
            }
            if (rescale) {
#pragma unroll
                for (int j = 0; j < 16; ++j) O[j] = O[j] * alpha;
            }
            // PV on raw value codes; per-channel value scale at the page boundary
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const u32x4 vv = buf[j];
                f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (PvLimbs == kPvF16) {
                    const half8 a0 = i8x8_to_f16(vv.x, vv.y);
                    const half8 a1 = i8x8_to_f16(vv.z, vv.w);
                    c = mfma_f16(a0, pbo[0], c);
                    c = mfma_f16(a1, pbo[1], c);
                } else {
                    // 128 ca + cb stays below 2^31 (|ca| <= 64 * 127 * 127)
                    const i32x4 z4 = {0, 0, 0, 0};
                    const i32x4 ca = mfma_i8(vv, pla, z4);
                    const i32x4 cb = mfma_i8(vv, plb, z4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) c[r] = (float)(ca[r] * 128 + cb[r]);
                }
                const f32x4 vs = *reinterpret_cast<const f32x4*>(&scl[kD + 16 * j + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) O[j][r] = O[j][r] + vs[r] * c[r];
                if (PF) buf[j] = ld16_stream(knp + koff + 1024 * j);  // next page's K tile
                if constexpr (InOrder) __builtin_amdgcn_sched_barrier(0);
            }
            if (PF) {
                float* nsc = sm.sc[w][slot ^ 1];
                *reinterpret_cast<u32x4*>(&nsc[4 * l]) = skn;
                *reinterpret_cast<u32x4*>(&nsc[kD + 4 * l]) = svn;
                nsc[2 * kD + l] = stn * a.scale_log2;
            }
        };

        for (int p = pa; p < pb - 1; ++p) page(std::integral_constant<bool, true>(), p);
        page(std::integral_constant<bool, false>(), pb - 1);
    }

    // merge the four waves: each publishes its unnormalised O, max and weight sum
    const float L = group_sum(lsum);
    // the column pair's parts: hi + lo, or the limb sums weighed 128 : 1 over S
    const float w_self = PvLimbs == kPvF16 ? 1.0f : 128.0f / pv_scale;
    const float w_pair = PvLimbs == kPvF16 ? 1.0f : 1.0f / pv_scale;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[j][r] = O[j][r] * w_self + swap_pair(O[j][r]) * w_pair;
    if (!lo_lane) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            *reinterpret_cast<f32x4*>(&sm.mo[w][hh][16 * j + 4 * g]) = O[j];
        if (g == 0) {
            sm.mm[w][hh] = M;
            sm.ml[w][hh] = L;
        }
    }
    __syncthreads();
    // item (h, 8 channels) per thread: half a wave covers one head, so up to
    // eight heads take one pass -- the merge is the tail of every
    // work-group (two passes of 4 channels cost 4 us per 128K step and 6 per
    // 32K step); O reads and stores are 16 bytes
    for (int it = tid; it < G * (kD / 8); it += kThreads) {
        const int h = it / (kD / 8), c8 = 8 * (it % (kD / 8));
        float mk[4], Ms = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mk[k] = sm.mm[k][h];
            Ms = fmaxf(Ms, mk[k]);
        }
        float lt = 0.0f;
        f32x4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (mk[k] == -INFINITY) continue;
            const float f = exp2f(mk[k] - Ms);
            lt += f * sm.ml[k][h];
            o0 += f * *reinterpret_cast<const f32x4*>(&sm.mo[k][h][c8]);
            o1 += f * *reinterpret_cast<const f32x4*>(&sm.mo[k][h][c8 + 4]);
        }
        const size_t row = row0 + h;
        const float inv = 1.0f / lt;
        float* dst = &a.part_o[(row * a.n_cols + a.col0 + split) * kD + c8];
        *reinterpret_cast<f32x4*>(dst) = o0 * inv;
        *reinterpret_cast<f32x4*>(dst + 4) = o1 * inv;
        if (c8 == 0) a.part_lse[row * a.n_cols + a.col0 + split] = (Ms + log2f(lt)) * kLn2;
    }
}

// --------------------------------------------------------------- exact tier
// A work-group owns pages [p0, p1) of one (request, KV head); wave w owns
// channels [64w, 64w + 64).  Per page: each wave's QK partial logits (its 64
// channels) go to LDS, one barrier, every wave sums the four and runs the
// same softmax, and PV runs over the wave's own channels with P fed hi
// (columns h < 8) and lo (columns h + 8).  The query is exact in BF16 and
// stays the B operand; the next page's K and V are loaded at the start of
// the current one; the last, partial page masks logits and zeroes the value
// elements past the length so padding never reaches the MFMA.

// zero the BF16 elements of an 8-token operand whose token index >= limit
__device__ __forceinline__ u32x4 mask_tokens(u32x4 v, int first, int limit) {
    uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo_keep = (first + 2 * i < limit) ? 0x0000FFFFu : 0u;
        const uint32_t hi_keep = (first + 2 * i + 1 < limit) ? 0xFFFF0000u : 0u;
        wd[i] &= (lo_keep | hi_keep);
    }
    return u32x4{wd[0], wd[1], wd[2], wd[3]};
}

// Operand sources of the exact body.  load() fetches one page-head's
// registers for this lane (the next page's while the current one is in
// use); keys() and values() hand the eight BF16 operand registers, in
// order, to f.
// The BF16 pool.  Loads are issued in whole 128-byte lines (register i of
// lane l is piece l % 8 of row 8 i + l / 8 of the wave's quarter: K token
// rows, V channel rows), non-temporal, and the MFMA operands are rebuilt
// through the wave's LDS quarter page: the operand layout alone would give
// each load instruction half lines, which streams about 12% slower.  Piece p
// of row x is stored at 8 x + (p ^ swizzle(x)), so the operand reads of eight
// lanes fall in eight different bank groups.
struct Bf16Source {
    const uint16_t* kb;
    const uint16_t* vb;
    u32x4* stage;  // this wave's LDS quarter page (512 pieces)
    struct Page {
        u32x4 k[8], v[8];
    };
    __device__ __forceinline__ void load(int slot, int kvh, int Hkv, int w, int l, Page& R) const {
        const size_t base = ((size_t)slot * Hkv + kvh) * (kP * kD);
        const uint16_t* kp = kb + base + (l >> 3) * kD + 64 * w + 8 * (l & 7);
        const uint16_t* vp = vb + base + (64 * w + (l >> 3)) * kP + 8 * (l & 7);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            R.k[i] = ld16_stream(kp + 8 * i * kD);
            R.v[i] = ld16_stream(vp + 8 * i * kP);
        }
    }
    // Key register 2t + s of lane (n, g) is token qk_row_token(t, n),
    // channels 64 w + 16 g + 8 s .. + 8 (piece 2 g + s); key rows swizzle by
    // (T & 3) | (T >> 2 & 4), which is n & 7 for the rows a lane reads.
    // Before reading pieces that other lanes wrote, the wave waits for its LDS
    // writes to complete (lgkmcnt 0); the empty asm statements keep the
    // compiler from moving LDS accesses across those points.
    template <class F>
    __device__ __forceinline__ void keys(const Page& R, F&& f) const {
        const int l = threadIdx.x & 63, n = l & 15, g = l >> 4;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int T = 8 * i + (l >> 3);
            stage[8 * T + ((l & 7) ^ ((T & 3) | ((T >> 2) & 4)))] = R.k[i];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        u32x4 op[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int T = qk_row_token(r >> 1, n);
            op[r] = stage[8 * T + ((2 * g + (r & 1)) ^ (n & 7))];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) f(r, op[r]);
    }
    // Value register 2j + s of lane (n, g) is channel 64 w + 16 j + n, tokens
    // 16 g + 8 s .. + 8 (piece 2 g + s); value rows swizzle by c & 7.
    template <class F>
    __device__ __forceinline__ void values(const Page& R, F&& f) const {
        const int l = threadIdx.x & 63, n = l & 15, g = l >> 4;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * i + (l >> 3);
            stage[8 * c + ((l & 7) ^ (c & 7))] = R.v[i];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        u32x4 op[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int c = 16 * (r >> 1) + n;
            op[r] = stage[8 * c + ((2 * g + (r & 1)) ^ (c & 7))];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) f(r, op[r]);
    }
};

// The lossless 13-bit planes ("Model quantization" page, "A lossless tier
// first"): per plane a descriptor ((byte offset / 256) << 1 | raw) and a
// 32-entry table; a coded plane is expanded to BF16 in registers right
// before its MFMA, a raw plane is read as the BF16 pool is.
struct L13Source {
    const uint8_t* arena;
    const int32_t* desc;
    const uint8_t* table;
    struct Page {
        u32x4 k[8], v[8];
        uint32_t tk[8], tv[8];
        int raw_k, raw_v;
        bool odd;  // lane parity (selects the lane's half of the index-bit-4 load)
    };
    __device__ __forceinline__ void load(int slot, int kvh, int Hkv, int w, int l, Page& R) const {
        const size_t plane = ((size_t)slot * Hkv + kvh) * 2;
        const int dk = __builtin_amdgcn_readfirstlane(desc[plane]);
        const int dv = __builtin_amdgcn_readfirstlane(desc[plane + 1]);
        const uint32_t* tp = reinterpret_cast<const uint32_t*>(table + plane * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            R.tk[i] = __builtin_amdgcn_readfirstlane(tp[i]);
            R.tv[i] = __builtin_amdgcn_readfirstlane(tp[8 + i]);
        }
        R.raw_k = dk & 1;
        R.raw_v = dv & 1;
        R.odd = l & 1;
        const uint8_t* kp = arena + (size_t)(dk >> 1) * 256;
        const uint8_t* vp = arena + (size_t)(dv >> 1) * 256;
        const int n = l & 15, g = l >> 4;
        // one 16-byte load per register either way (the choice of address is
        // uniform): a raw plane's BF16 operand, or a coded plane's chunk
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int coded = l13_chunk_offset(w, l, r);
            const int rk = 2 * (qk_row_token(r >> 1, n) * kD + 64 * w + 16 * g + 8 * (r & 1));
            const int rv = 2 * ((64 * w + 16 * (r >> 1) + n) * kP + 16 * g + 8 * (r & 1));
            R.k[r] = ld16_stream(kp + (R.raw_k ? rk : coded));
            R.v[r] = ld16_stream(vp + (R.raw_v ? rv : coded));
        }
    }
    template <class F>
    __device__ __forceinline__ void keys(const Page& R, F&& f) const {
        if (R.raw_k) {
#pragma unroll
            for (int r = 0; r < 8; ++r) f(r, R.k[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) f(r, l13_operand(R.k, R.tk, r, R.odd));
        }
    }
    template <class F>
    __device__ __forceinline__ void values(const Page& R, F&& f) const {
        if (R.raw_v) {
#pragma unroll
            for (int r = 0; r < 8; ++r) f(r, R.v[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) f(r, l13_operand(R.v, R.tv, r, R.odd));
        }
    }
};

template <int Prio, class Src>
__device__ __forceinline__ void exact_split(const ExactArgs& a, const Src& src, ExactSmem& sm, int split, int kvh,
                                            int b) {
    const int len = a.seq_len[b];
    const int np = min((len + kP - 1) / kP, a.max_pages);
    const int p0 = split * a.pps;
    if (p0 >= np) {
        write_empty(a.G, a.Hkv, kvh, b, a.n_cols, a.col0 + split, a.part_lse);
        return;
    }
    const int p1 = min(np, p0 + a.pps);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
    if constexpr (Prio == kPrioWave) set_issue_priority(3 - __builtin_amdgcn_readfirstlane(w));
    const int hh = n & 7;
    const bool hi_lane = n < 8;
    const bool valid = hh < a.G;
    const int Hkv = a.Hkv, Hq = Hkv * a.G;
    const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
    const size_t row = (size_t)b * Hq + (size_t)kvh * a.G + hh;

    float (*s_part)[4][16][64] = sm.part;

    // the query is exact in BF16 and needs no per-page work: keep it as the B operand
    bf16x8 qb[2];
    {
        u32x4 q0 = {0, 0, 0, 0}, q1 = {0, 0, 0, 0};
        if (valid) {
            const uint16_t* qp = a.q + row * kD + 64 * w + 16 * g;
            q0 = ld16(qp);
            q1 = ld16(qp + 8);
        }
        qb[0] = as_bf16x8(q0);
        qb[1] = as_bf16x8(q1);
    }

    typename Src::Page cur;
    src.load(pt[p0], kvh, Hkv, w, l, cur);
    const float vm = valid ? 1.0f : 0.0f, lo_m = hi_lane ? 0.0f : 1.0f;

    float M = -INFINITY, lsum = 0.0f;
    f32x4 O[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) O[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // The page step; PF: load the next page first.  The last page runs
    // outside the loop so that no load in the loop sits behind a branch:
    // after such a branch the compiler waits for every outstanding load at
    // the loop head, and the next page's loads no longer overlap the
    // current page's work (all-BF16 step 1.46 against 1.50 ms at 128K, 0.47
    // against 0.49 ms at 32K).
    auto page = [&](auto prefetch, int p, int it) {
        constexpr bool PF = decltype(prefetch)::value;
        if constexpr (Prio == kPrioPagesLeft) set_issue_priority(min(3, p1 - p - 1));
        typename Src::Page nxt;
        if constexpr (PF) src.load(pt[p + 1], kvh, Hkv, w, l, nxt);

        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // key register 2t + s is tile t, contraction half s
        src.keys(cur, [&](int r, u32x4 kop) { acc[r >> 1] = mfma_bf16(as_bf16x8(kop), qb[r & 1], acc[r >> 1]); });
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_part[it & 1][w][4 * t + r][l] = acc[t][r];
        __syncthreads();

        const int in_page = len - p * kP;  // valid tokens in this page (>= 1)
        const bool partial = in_page < kP;
        float S[16], z[16], pr[16];
        gather_logits(s_part[it & 1], l, S);
        if (partial) {
#pragma unroll
            for (int k = 0; k < 16; ++k) z[k] = (16 * g + k < in_page) ? S[k] * a.scale_log2 : -INFINITY;
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) z[k] = S[k] * a.scale_log2;
        }
        const float alpha = softmax_step(z, M, lsum, pr);

        // P^T operand: the hi part in hi lanes, the lo part in lo lanes, 0 for heads past G
        bf16x8 pb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) pb[s][e2] = split_sel_bf16(p_elem(pr, s, e2) * vm, lo_m);

#pragma unroll
        for (int j = 0; j < 4; ++j) O[j] = O[j] * alpha;
        // value register 2j + s is channel tile j, contraction half s (tokens 16g + 8s ..);
        // on the last, partial page masked values must not reach the MFMA
        src.values(cur, [&](int r, u32x4 vop) {
            if (partial) vop = mask_tokens(vop, 16 * g + 8 * (r & 1), in_page);
            O[r >> 1] = mfma_bf16(as_bf16x8(vop), pb[r & 1], O[r >> 1]);
        });

        if constexpr (PF) cur = nxt;
    };
    int it = 0;
    for (int p = p0; p < p1 - 1; ++p, ++it) page(std::integral_constant<bool, true>(), p, it);
    page(std::integral_constant<bool, false>(), p1 - 1, it);


    write_partial(O, M, lsum, valid, hi_lane, w, g, row, a.n_cols, a.col0 + split, a.part_o, a.part_lse);
}

union SplitSmem {
    Int8Smem i8;
    struct {
        ExactSmem ex;
        Bf16Stage st;
    } bx;
};

template <int PvLimbs, int Prio, bool InOrder = false>
__global__ __launch_bounds__(kThreads, 2) void decode_int8_kernel(const int32_t* page_table, const int32_t* n_pages,
                                                                  int max_pages, int splits, Int8Args a) {
    __shared__ Int8Smem sm;
    int8_split<PvLimbs, Prio, InOrder>(with_lead(a, page_table, n_pages, max_pages, splits), sm, blockIdx.x,
                                       blockIdx.y, blockIdx.z);
}

template <int Prio>
__global__ __launch_bounds__(kThreads, 2) void decode_exact_kernel(ExactArgs a) {
    __shared__ ExactSmem sm;
    __shared__ Bf16Stage st;
    exact_split<Prio>(a, Bf16Source{a.kb, a.vb, st.q[threadIdx.x >> 6]}, sm, blockIdx.x, blockIdx.y, blockIdx.z);
}

// The exact body over lossless 13-bit planes: same split plan and
// arithmetic as decode_exact_kernel, so the result is bit-identical to it on
// the decoded pages.
template <int Prio>
__global__ __launch_bounds__(kThreads, 2) void decode_l13_kernel(ExactArgs a, L13Source src) {
    __shared__ ExactSmem sm;
    exact_split<Prio>(a, src, sm, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Both tiers of a layer in one launch: in each (request, KV head) row of the
// grid the first n8s work-groups are the int8 tier's and the rest read the
// BF16 window (measured against window-first: the same at 128K, 2 us faster
// per 32K step, 0.8% faster batched); all write partial columns of the same
// rows (int8 columns first, window columns after them).  The leading scalar
// arguments are the int8 tier's (see with_lead) and its column count.
template <int PvLimbs, int Prio, bool InOrder = false>
__global__ __launch_bounds__(kThreads, 2) void decode_hybrid_kernel(const int32_t* page_table, const int32_t* n_pages,
                                                                    int max_pages, int splits, int n8s, Int8Args a8,
                                                                    ExactArgs ax) {
    __shared__ SplitSmem sm;
    if ((int)blockIdx.x >= n8s)
        exact_split<Prio>(ax, Bf16Source{ax.kb, ax.vb, sm.bx.st.q[threadIdx.x >> 6]}, sm.bx.ex, blockIdx.x - n8s,
                          blockIdx.y, blockIdx.z);
    else
        int8_split<PvLimbs, Prio, InOrder>(with_lead(a8, page_table, n_pages, max_pages, splits), sm.i8, blockIdx.x,
                                           blockIdx.y, blockIdx.z);
}

// Tensors: non-NULL and 16-byte aligned.  int32 page tables and length
// arrays (read one element at a time) need only 4-byte alignment, so a
// caller can pass a slice of requests.
static akv_status check_ptrs(const void* const* ptrs, int nptrs, const void* const* tables, int ntables) {
    for (int i = 0; i < nptrs; ++i) {
        if (!ptrs[i]) return fail(AKV_ERR_ARG, "NULL pointer (tensor argument %d)", i);
        if (!aligned16(ptrs[i])) return fail(AKV_ERR_ALIGN, "tensor argument %d not 16-byte aligned", i);
    }
    for (int i = 0; i < ntables; ++i) {
        if (!tables[i]) return fail(AKV_ERR_ARG, "NULL pointer (table argument %d)", i);
        if ((reinterpret_cast<uintptr_t>(tables[i]) & 3u) != 0)
            return fail(AKV_ERR_ALIGN, "table argument %d not 4-byte aligned", i);
    }
    return AKV_OK;
}

static akv_status check_shape(const akv_dims* dims, int32_t batch, int32_t max_pages) {
    akv_status st = check_dims(dims);
    if (st != AKV_OK) return st;
    if (batch < 0 || max_pages < 0) return fail(AKV_ERR_ARG, "negative batch or max_pages");
    if (batch > 65535) return fail(AKV_ERR_UNSUPPORTED, "batch %d > 65535", batch);
    return AKV_OK;
}

static akv_status check_workspace(void* ws, size_t have, size_t need) {
    if (need == 0) return AKV_OK;
    if (!ws || have < need) return fail(AKV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
    if (!aligned16(ws)) return fail(AKV_ERR_ALIGN, "workspace not 16-byte aligned");
    return AKV_OK;
}

static void split_workspace(const akv_dims* d, int batch, int n_cols, void* ws, float** po, float** pl) {
    const size_t rows = (size_t)batch * d->num_kv_heads * d->group;
    const size_t o = ((rows * n_cols * d->head_dim * sizeof(float) + 255) / 256) * 256;
    *po = reinterpret_cast<float*>(ws);
    *pl = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + o);
}

static Int8Args int8_args(const akv_dims* dims, const uint16_t* q, const int8_t* k_codes, const int8_t* v_codes,
                          const float* k_chan, const float* k_tok, const float* v_chan, const int32_t* page_table,
                          const int32_t* n_pages, int max_pages, float scale, const SplitPlan& plan) {
    Int8Args a;
    a.q = q;
    a.kc = k_codes;
    a.vc = v_codes;
    a.kchan = k_chan;
    a.ktok = k_tok;
    a.vchan = v_chan;
    a.page_table = page_table;
    a.n_pages = n_pages;
    a.max_pages = max_pages;
    a.Hkv = dims->num_kv_heads;
    a.G = dims->group;
    a.splits = plan.n_splits;
    a.col0 = 0;
    a.n_cols = plan.n_splits;
    a.scale_log2 = scale * kLog2e;
    a.part_o = a.part_lse = nullptr;
    return a;
}

// A wave stages at most kMaxPagesPerWave page slots in LDS: a work-group's
// share, at most ceil(max_pages / n_splits) pages, must fit four waves.  The
// kernel computes the shares in 32-bit arithmetic: splits x max_pages must
// stay below 2^32 (always so below 65,536 pages per table row).
static akv_status check_int8_plan(const SplitPlan& p, int max_pages) {
    const long long per_wg = p.n_splits > 0 ? ((long long)max_pages + p.n_splits - 1) / p.n_splits : 0;
    if (p.n_splits < 1 || per_wg > 4 * kMaxPagesPerWave)
        return fail(AKV_ERR_ARG, "int8 split plan of %d splits for %d pages exceeds %d pages per work-group",
                    p.n_splits, max_pages, 4 * kMaxPagesPerWave);
    if ((long long)p.n_splits * max_pages >= (1LL << 32))
        return fail(AKV_ERR_UNSUPPORTED, "int8 split plan of %d splits for %d pages: splits x pages reaches 2^32",
                    p.n_splits, max_pages);
    return AKV_OK;
}

static ExactArgs exact_args(const akv_dims* dims, const uint16_t* q, const uint16_t* k_bf16, const uint16_t* v_bf16,
                            const int32_t* page_table, const int32_t* seq_len, int max_pages, float scale,
                            const SplitPlan& plan) {
    ExactArgs a;
    a.q = q;
    a.kb = k_bf16;
    a.vb = v_bf16;
    a.page_table = page_table;
    a.seq_len = seq_len;
    a.max_pages = max_pages;
    a.Hkv = dims->num_kv_heads;
    a.G = dims->group;
    a.pps = plan.pages_per_split;
    a.col0 = 0;
    a.n_cols = plan.n_splits;
    a.scale_log2 = scale * kLog2e;
    a.part_o = a.part_lse = nullptr;
    return a;
}

// Split partials of akv_decode_hybrid_static: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` is only
// a stand-in for the symbol; its device address (different on every GPU) is
// looked up once per device with that device current and used from then on.
constexpr size_t kStaticScratchBytes = AKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static akv_status static_scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(AKV_ERR_HIP, "no current HIP device (or device id %d beyond %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(AKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return AKV_OK;
}

// Launch the split-K kernel; with profile events set, through
// hipExtLaunchKernelGGL so the events time the kernel itself.
template <typename... A>
static void launch_split(void (*kernel)(A...), dim3 grid, hipStream_t s, A... args) {
    hipEvent_t e0 = prof_start_event(), e1 = prof_stop_event();
    if (e0 && e1)
        hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, e0, e1, 0, args...);
    else
        kernel<<<grid, kThreads, 0, s>>>(args...);
}

// A grid of at most one work-group per compute unit (see InOrder).
static bool one_per_cu(dim3 grid) {
    return (long long)grid.x * grid.y * grid.z <= device_cu_count();
}

// The int8 kernel with its leading copies of the struct's page table, page
// counts, row length and split count (see with_lead).
template <typename K>
static void launch_int8(K kernel, dim3 grid, hipStream_t s, const Int8Args& a) {
    launch_split(kernel, grid, s, a.page_table, a.n_pages, a.max_pages, a.splits, a);
}

}  // namespace akv

using namespace akv;

extern "C" akv_status akv_decode_attn_int8(const akv_dims* dims, int32_t batch, const uint16_t* q,
                                           const int8_t* k_codes, const int8_t* v_codes, const float* k_chan,
                                           const float* k_tok, const float* v_chan, const int32_t* page_table,
                                           const int32_t* n_pages, int32_t max_pages, float softmax_scale,
                                           float* out_o, float* out_lse, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    clear_error();
    akv_status st = check_shape(dims, batch, max_pages);
    if (st != AKV_OK || batch == 0) return st;
    const void* ptrs[] = {q, k_codes, v_codes, k_chan, k_tok, v_chan, out_o, out_lse};
    const void* tabs[] = {page_table, n_pages};
    if ((st = check_ptrs(ptrs, 8, tabs, 2)) != AKV_OK) return st;
    const int rows = batch * dims->num_kv_heads * dims->group;
    if (max_pages == 0) return akv_fill_empty(rows, dims->head_dim, out_o, out_lse, stream);
    const SplitPlan plan = plan_int8_splits(dims, batch, max_pages);
    if ((st = check_int8_plan(plan, max_pages)) != AKV_OK) return st;
    if ((st = check_workspace(workspace, workspace_bytes, partial_bytes(dims, batch, plan.n_splits))) != AKV_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    Int8Args a = int8_args(dims, q, k_codes, v_codes, k_chan, k_tok, v_chan, page_table, n_pages, max_pages,
                           softmax_scale, plan);
    split_workspace(dims, batch, plan.n_splits, workspace, &a.part_o, &a.part_lse);
    dim3 grid((unsigned)plan.n_splits, (unsigned)dims->num_kv_heads, (unsigned)batch);
    switch (pv_fp16() ? 3 + issue_priority() : issue_priority()) {
        case 0:
            if (one_per_cu(grid))
                launch_int8(decode_int8_kernel<kPvI8, kPrioOff, true>, grid, s, a);
            else
                launch_int8(decode_int8_kernel<kPvI8, kPrioOff>, grid, s, a);
            break;
        case 1: launch_int8(decode_int8_kernel<kPvI8, kPrioPagesLeft>, grid, s, a); break;
        case 2: launch_int8(decode_int8_kernel<kPvI8, kPrioWave>, grid, s, a); break;
        case 3: launch_int8(decode_int8_kernel<kPvF16, kPrioOff>, grid, s, a); break;
        case 4: launch_int8(decode_int8_kernel<kPvF16, kPrioPagesLeft>, grid, s, a); break;
        default: launch_int8(decode_int8_kernel<kPvF16, kPrioWave>, grid, s, a); break;
    }
    if ((st = launch_status("decode_int8_kernel")) != AKV_OK) return st;
    return launch_combine(rows, dims->head_dim, a.part_o, a.part_lse, plan.n_splits, out_o, out_lse, s);
}

extern "C" akv_status akv_decode_attn_exact(const akv_dims* dims, int32_t batch, const uint16_t* q,
                                            const uint16_t* k_bf16, const uint16_t* v_bf16,
                                            const int32_t* page_table, const int32_t* seq_len, int32_t max_pages,
                                            float softmax_scale, float* out_o, float* out_lse, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    clear_error();
    akv_status st = check_shape(dims, batch, max_pages);
    if (st != AKV_OK || batch == 0) return st;
    const void* ptrs[] = {q, k_bf16, v_bf16, out_o, out_lse};
    const void* tabs[] = {page_table, seq_len};
    if ((st = check_ptrs(ptrs, 5, tabs, 2)) != AKV_OK) return st;
    const int rows = batch * dims->num_kv_heads * dims->group;
    if (max_pages == 0) return akv_fill_empty(rows, dims->head_dim, out_o, out_lse, stream);
    const SplitPlan plan = plan_splits(dims, batch, max_pages);
    if ((st = check_workspace(workspace, workspace_bytes, partial_bytes(dims, batch, plan.n_splits))) != AKV_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    ExactArgs a = exact_args(dims, q, k_bf16, v_bf16, page_table, seq_len, max_pages, softmax_scale, plan);
    split_workspace(dims, batch, plan.n_splits, workspace, &a.part_o, &a.part_lse);
    dim3 grid((unsigned)plan.n_splits, (unsigned)dims->num_kv_heads, (unsigned)batch);
    switch (issue_priority()) {
        case 0: launch_split(decode_exact_kernel<kPrioOff>, grid, s, a); break;
        case 1: launch_split(decode_exact_kernel<kPrioPagesLeft>, grid, s, a); break;
        default: launch_split(decode_exact_kernel<kPrioWave>, grid, s, a); break;
    }
    if ((st = launch_status("decode_exact_kernel")) != AKV_OK) return st;
    return launch_combine(rows, dims->head_dim, a.part_o, a.part_lse, plan.n_splits, out_o, out_lse, s);
}

// One hybrid layer with its split partials in `workspace`.  With
// static_scratch set, the workspace is the library's per-device scratch
// array: its address is looked up (once per device) only after every host
// check has passed, and a plan that needs more than the array is refused.
static akv_status decode_hybrid_impl(const akv_dims* dims, int32_t batch, const uint16_t* q, const int8_t* k_codes,
                                     const int8_t* v_codes, const float* k_chan, const float* k_tok,
                                     const float* v_chan, const int32_t* page_table_int8,
                                     const int32_t* n_pages_int8, int32_t max_pages_int8, const uint16_t* k_bf16,
                                     const uint16_t* v_bf16, const int32_t* page_table_window,
                                     const int32_t* window_len, int32_t max_pages_window, float softmax_scale,
                                     float* out_o, float* out_lse, void* workspace, size_t workspace_bytes,
                                     bool static_scratch, void* stream) {
    akv_status st = check_shape(dims, batch, max_pages_int8);
    if (st != AKV_OK) return st;
    if (max_pages_window < 0) return fail(AKV_ERR_ARG, "negative max_pages_window");
    if (batch == 0) return AKV_OK;
    // a tier with no page-table columns is never read: its pointers may be NULL
    const void* ptrs_q[] = {q, out_o, out_lse};
    if ((st = check_ptrs(ptrs_q, 3, nullptr, 0)) != AKV_OK) return st;
    if (max_pages_int8 > 0) {
        const void* ptrs[] = {k_codes, v_codes, k_chan, k_tok, v_chan};
        const void* tabs[] = {page_table_int8, n_pages_int8};
        if ((st = check_ptrs(ptrs, 5, tabs, 2)) != AKV_OK) return st;
    }
    if (max_pages_window > 0) {
        const void* ptrs[] = {k_bf16, v_bf16};
        const void* tabs[] = {page_table_window, window_len};
        if ((st = check_ptrs(ptrs, 2, tabs, 2)) != AKV_OK) return st;
    }
    const int rows = batch * dims->num_kv_heads * dims->group;
    if (max_pages_int8 + max_pages_window == 0) return akv_fill_empty(rows, dims->head_dim, out_o, out_lse, stream);
    SplitPlan p8, pw;
    plan_hybrid(dims, batch, max_pages_int8, max_pages_window, &p8, &pw);
    if (max_pages_int8 > 0 && (st = check_int8_plan(p8, max_pages_int8)) != AKV_OK) return st;
    if (pw.n_splits < 0 || (max_pages_window > 0 && pw.n_splits < 1) || (max_pages_int8 == 0 && p8.n_splits != 0))
        return fail(AKV_ERR_ARG, "hybrid split plan of %d int8 and %d window splits is inconsistent", p8.n_splits,
                    pw.n_splits);
    const int n_cols = p8.n_splits + pw.n_splits;
    if (static_scratch) {
        const size_t need = partial_bytes(dims, batch, n_cols);
        if (need > kStaticScratchBytes)
            return fail(AKV_ERR_WORKSPACE, "split partials need %zu bytes, the static scratch holds %zu", need,
                        kStaticScratchBytes);
        if ((st = static_scratch_address(&workspace)) != AKV_OK) return st;
        workspace_bytes = kStaticScratchBytes;
    }
    if ((st = check_workspace(workspace, workspace_bytes, partial_bytes(dims, batch, n_cols))) != AKV_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Int8Args a8 = int8_args(dims, q, k_codes, v_codes, k_chan, k_tok, v_chan, page_table_int8, n_pages_int8,
                            max_pages_int8, softmax_scale, p8);
    ExactArgs ax = exact_args(dims, q, k_bf16, v_bf16, page_table_window, window_len, max_pages_window,
                              softmax_scale, pw);
    a8.n_cols = ax.n_cols = n_cols;
    ax.col0 = p8.n_splits;
    split_workspace(dims, batch, n_cols, workspace, &a8.part_o, &a8.part_lse);
    ax.part_o = a8.part_o;
    ax.part_lse = a8.part_lse;
    dim3 grid((unsigned)n_cols, (unsigned)dims->num_kv_heads, (unsigned)batch);
    switch (pv_fp16() ? 3 + issue_priority() : issue_priority()) {
        case 0:
            if (one_per_cu(grid))
                launch_split(decode_hybrid_kernel<kPvI8, kPrioOff, true>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax);
            else
                launch_split(decode_hybrid_kernel<kPvI8, kPrioOff>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax);
            break;
        case 1: launch_split(decode_hybrid_kernel<kPvI8, kPrioPagesLeft>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax); break;
        case 2: launch_split(decode_hybrid_kernel<kPvI8, kPrioWave>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax); break;
        case 3: launch_split(decode_hybrid_kernel<kPvF16, kPrioOff>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax); break;
        case 4: launch_split(decode_hybrid_kernel<kPvF16, kPrioPagesLeft>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax); break;
        default: launch_split(decode_hybrid_kernel<kPvF16, kPrioWave>, grid, s, a8.page_table, a8.n_pages, a8.max_pages, a8.splits, n_cols - pw.n_splits, a8, ax); break;
    }
    if ((st = launch_status("decode_hybrid_kernel")) != AKV_OK) return st;
    return launch_combine(rows, dims->head_dim, a8.part_o, a8.part_lse, n_cols, out_o, out_lse, s);
}

extern "C" akv_status akv_decode_hybrid(const akv_dims* dims, int32_t batch, const uint16_t* q,
                                        const int8_t* k_codes, const int8_t* v_codes, const float* k_chan,
                                        const float* k_tok, const float* v_chan, const int32_t* page_table_int8,
                                        const int32_t* n_pages_int8, int32_t max_pages_int8, const uint16_t* k_bf16,
                                        const uint16_t* v_bf16, const int32_t* page_table_window,
                                        const int32_t* window_len, int32_t max_pages_window, float softmax_scale,
                                        float* out_o, float* out_lse, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    clear_error();
    return decode_hybrid_impl(dims, batch, q, k_codes, v_codes, k_chan, k_tok, v_chan, page_table_int8,
                              n_pages_int8, max_pages_int8, k_bf16, v_bf16, page_table_window, window_len,
                              max_pages_window, softmax_scale, out_o, out_lse, workspace, workspace_bytes, false,
                              stream);
}

extern "C" akv_status akv_decode_hybrid_static(const akv_dims* dims, int32_t batch, const uint16_t* q,
                                               const int8_t* k_codes, const int8_t* v_codes, const float* k_chan,
                                               const float* k_tok, const float* v_chan,
                                               const int32_t* page_table_int8, const int32_t* n_pages_int8,
                                               int32_t max_pages_int8, const uint16_t* k_bf16,
                                               const uint16_t* v_bf16, const int32_t* page_table_window,
                                               const int32_t* window_len, int32_t max_pages_window,
                                               float softmax_scale, float* out_o, float* out_lse, void* stream) {
    clear_error();
    return decode_hybrid_impl(dims, batch, q, k_codes, v_codes, k_chan, k_tok, v_chan, page_table_int8,
                              n_pages_int8, max_pages_int8, k_bf16, v_bf16, page_table_window, window_len,
                              max_pages_window, softmax_scale, out_o, out_lse, nullptr, 0, true, stream);
}

extern "C" akv_status akv_decode_attn_l13(const akv_dims* dims, int32_t batch, const uint16_t* q,
                                          const uint8_t* l13_arena, const int32_t* l13_desc,
                                          const uint8_t* l13_table, const int32_t* page_table,
                                          const int32_t* seq_len, int32_t max_pages, float softmax_scale,
                                          float* out_o, float* out_lse, void* workspace, size_t workspace_bytes,
                                          void* stream) {
    clear_error();
    akv_status st = check_shape(dims, batch, max_pages);
    if (st != AKV_OK || batch == 0) return st;
    if ((uintptr_t)l13_arena % 256 != 0) return fail(AKV_ERR_ALIGN, "l13_arena not 256-byte aligned");
    const void* ptrs[] = {q, l13_arena, l13_table, out_o, out_lse};
    const void* tabs[] = {page_table, seq_len, l13_desc};
    if ((st = check_ptrs(ptrs, 5, tabs, 3)) != AKV_OK) return st;
    const int rows = batch * dims->num_kv_heads * dims->group;
    if (max_pages == 0) return akv_fill_empty(rows, dims->head_dim, out_o, out_lse, stream);
    const SplitPlan plan = plan_splits(dims, batch, max_pages);
    if ((st = check_workspace(workspace, workspace_bytes, partial_bytes(dims, batch, plan.n_splits))) != AKV_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    ExactArgs a = exact_args(dims, q, nullptr, nullptr, page_table, seq_len, max_pages, softmax_scale, plan);
    split_workspace(dims, batch, plan.n_splits, workspace, &a.part_o, &a.part_lse);
    const L13Source src{l13_arena, l13_desc, l13_table};
    dim3 grid((unsigned)plan.n_splits, (unsigned)dims->num_kv_heads, (unsigned)batch);
    switch (issue_priority()) {
        case 0: launch_split(decode_l13_kernel<kPrioOff>, grid, s, a, src); break;
        case 1: launch_split(decode_l13_kernel<kPrioPagesLeft>, grid, s, a, src); break;
        default: launch_split(decode_l13_kernel<kPrioWave>, grid, s, a, src); break;
    }
    if ((st = launch_status("decode_l13_kernel")) != AKV_OK) return st;
    return launch_combine(rows, dims->head_dim, a.part_o, a.part_lse, plan.n_splits, out_o, out_lse, s);
}
