/*
 * akv.h -- C ABI of libakv.so: ActiveKV hybrid-tier decode attention on
 * AMD MI355X (gfx950).
 *
 * The pages this follows (cited by page title and section):
 *   "Model quantization" page, "An 8-bit page format shaped for its kernel"
 *       -- the 8-bit page format and when pages are converted.
 *   "SYCL" page, "Attention that reads 8-bit history"
 *       -- decode that reads the int8 pages directly.
 *   "SYCL" page, "Exact tricks and a two-owner decoder"
 *       -- two requests with equal page counts served by one launch.
 *   "SYCL" page, "A merge that joins the tiers"
 *       -- log-sum-exp output starting at -inf; merge into one FP32
 *          accumulator.
 *   "Model quantization" page, "A lossless tier first"
 *       -- the 13-bit lossless tier the 8-bit format replaced.
 *   "ActiveKV" page, "The idea" and "What I built"
 *       -- exact BF16 tier, hybrid tier, host-authoritative pinned history,
 *          budgeted staging with a fence-safe lifecycle, explicit refusal.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise.  The
 *     caller owns every buffer, including workspaces and ring slots; the
 *     library allocates no device memory and never synchronizes the host.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  The return value reports host-side argument checks
 *     and launch errors only; device faults surface at the caller's sync.
 *   - Pointers to tensors must be 16-byte aligned (AKV_ERR_ALIGN otherwise);
 *     int32 page tables and length arrays need only 4-byte alignment, so a
 *     slice of requests' rows can be passed.
 *   - No C++ exception crosses this interface.  akv_last_error() gives a
 *     thread-local message for the last failing call.
 *
 * Shapes: Hkv KV heads, G query heads per KV head (Hq = Hkv*G; query head j
 * reads KV head j / G), head dimension D, page size P tokens.  Supported:
 * D = 256, P = 64, 1 <= G <= 8, Hkv >= 1 (AKV_ERR_UNSUPPORTED otherwise).
 *
 * Layouts (row-major, innermost last):
 *   q        BF16 [B][Hq][D]
 *   BF16 pool  K  [slot][Hkv][P][D]   token-major
 *              V  [slot][Hkv][D][P]   channel-major (a page of values is
 *                                     stored transposed, so each channel's
 *                                     64 tokens are contiguous)
 *   int8 pool  k_codes [slot][Hkv][16384] int8 in tile order: code
 *                      K[t][d] of a page-head sits at byte
 *                        ((4 (d / 64) + (t / 4) % 4) * 64 + 16 ((d / 16) % 4)
 *                         + 4 (t / 16) + t % 4) * 16 + d % 16,
 *                      so the page is 16 tiles of 1 KB, each holding 16
 *                      whole 64-byte channel runs of 16 tokens in the
 *                      order the decode kernel consumes them
 *              v_codes [slot][Hkv][D][P]   int8, channel-major
 *              k_chan  [slot][Hkv][D]      FP32 per-channel key factor
 *              k_tok   [slot][Hkv][P]      FP32 per-token key factor
 *              v_chan  [slot][Hkv][D]      FP32 per-channel value scale
 *   page tables int32 [B][max_pages]  (pool slot of each page, in order)
 *   outputs  O FP32 [B][Hq][D] (normalised), LSE FP32 [B][Hq]
 *
 * LSE is the natural log of sum_t exp(softmax_scale * q . k_t).  A request
 * with no tokens yields O = 0 and LSE = -inf (a valid empty partial).
 */
#ifndef AKV_H
#define AKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AKV_OK = 0,
    AKV_ERR_ARG = -1,         /* null pointer, negative size, bad shape   */
    AKV_ERR_UNSUPPORTED = -2, /* D != 256, P != 64, G outside [1, 8]      */
    AKV_ERR_ALIGN = -3,       /* tensor pointer not 16-byte aligned       */
    AKV_ERR_WORKSPACE = -4,   /* workspace smaller than the query result  */
    AKV_ERR_BUDGET = -5,      /* staging request exceeds the ring's slot  */
    AKV_ERR_HIP = -6,         /* a HIP runtime call failed                */
    AKV_ERR_STATE = -7        /* ring used out of its lifecycle order     */
} akv_status;

typedef struct {
    int32_t num_kv_heads; /* Hkv                                  */
    int32_t group;        /* G query heads per KV head            */
    int32_t head_dim;     /* D, must be 256                       */
    int32_t page_size;    /* P, must be 64                        */
} akv_dims;

/* Human-readable name of a status code (static string). */
const char *akv_status_string(akv_status s);
/* Message describing the last failure on the calling thread ("" if none). */
const char *akv_last_error(void);
/* Library version, e.g. "akv 0.1.0 gfx950". */
const char *akv_version(void);

/*
 * Instrumentation (the "ActiveKV" page, "What I built", keeps instrumented
 * runs apart from product timing): on the calling thread, the split-K kernel
 * of each subsequent decode call (int8, exact or hybrid) is launched with
 * start_event and stop_event attached to its dispatch (hipExtLaunchKernelGGL),
 * so the pair brackets that kernel and its dispatch; the events must allow
 * timing.
 * Both hipEvent_t handles are owned by the caller; pass NULL, NULL to stop.
 * Errors: AKV_ERR_ARG if exactly one of them is NULL.
 */
akv_status akv_set_profile_events(void *start_event, void *stop_event);

/*
 * Instrumentation (launch-shape sweeps and tests): on the calling thread,
 * override how the decode calls split their pages over work-groups.  Each
 * field is 0 for the library's own plan, else:
 *   pages_per_split      akv_decode_attn_exact / _l13: pages per work-group;
 *   pages_per_wave       akv_decode_attn_int8: pages per wave (a work-group is
 *                        four waves), at most 64;
 *   hybrid_int8_pages    akv_decode_hybrid: int8 pages per work-group, at
 *                        most 256;
 *   hybrid_window_pages  akv_decode_hybrid: window pages per work-group;
 *   pv_fp16              akv_decode_attn_int8 / akv_decode_hybrid: 1 runs the
 *                        int8 tier's PV product on FP16 operands (the softmax
 *                        weights as FP16 hi + lo against value codes turned
 *                        into FP16) instead of the int8 MFMA (the weights as
 *                        three 7-bit fixed-point limbs against the raw codes);
 *                        for A/B measurement ("SYCL" page, "Attention that
 *                        reads 8-bit history": which products run on integers
 *                        is decided by measurement).  Both stay within the
 *                        acceptance tolerances;
 *   issue_priority       akv_decode_attn_int8 / _exact / _l13 /
 *                        akv_decode_hybrid(_static): a scheduling probe for
 *                        tests.  0 leaves every wave at the default issue
 *                        priority; 1 sets each decode wave's priority
 *                        (s_setprio) from the pages it has left, 3 for four
 *                        or more down to 0 on its last; 2 sets it from the
 *                        wave's index in its work-group (int8 body w, exact
 *                        body 3 - w).  Outputs must be bit-identical to 0:
 *                        only the interleaving of the waves changes, which
 *                        exposes instruction hazards and races that the
 *                        default interleaving hides.
 * NULL restores the plan.  The workspace size queries follow the same
 * setting, so change it only between a query and the calls it sized.
 * Results do not depend on the shape beyond FP32 rounding order (and, for
 * pv_fp16, the weights' rounding: 22 significant bits either way).
 * Errors: AKV_ERR_ARG for a negative field, one beyond its limit, pv_fp16
 * other than 0 or 1 or issue_priority other than 0, 1 or 2 (nothing is
 * changed then).
 */
typedef struct {
    int32_t pages_per_split;
    int32_t pages_per_wave;
    int32_t hybrid_int8_pages;
    int32_t hybrid_window_pages;
    int32_t pv_fp16;
    int32_t issue_priority;
} akv_launch_shape;
akv_status akv_set_launch_shape(const akv_launch_shape *shape);

/*
 * Instrumentation: one plain streaming read of `bytes` (a multiple of 16 at
 * least 32 KiB) of device memory at `buf` (16-byte aligned) with non-temporal
 * 16-byte vector loads from 2048 work-groups, the streaming-read ceiling the decode
 * kernels' HBM rate is reported against.  Reads floor(bytes / 32 KiB) * 32 KiB
 * bytes; `sink` is a device word that is written only on an impossible value.
 * Errors: AKV_ERR_ARG, AKV_ERR_ALIGN.
 */
akv_status akv_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * akv_quantize_pages -- convert n full BF16 pages into the 8-bit page format.
 * ("Model quantization" page, "An 8-bit page format shaped for its kernel".)
 *
 * For each i < n and each KV head h, reads BF16 page src_slot[i] of
 * (k_bf16, v_bf16) and writes int8 page dst_slot[i] of the int8 pool:
 *   key channel factor  c_d = clamp(sqrt(RMS_d) / g, 2^-14, 2^14), where
 *       RMS_d is over the page's 64 tokens and g is the geometric mean of
 *       sqrt(RMS) over channels with nonzero RMS (zero channels: c_d = 1);
 *   key token factor    s_t = max_d(|K[t][d]| / c_d) / 127;
 *   value scale         vs_d = max_t |V[t][d]| / 127;
 *   codes               round-half-even(K / (c_d s_t)), round-half-even(V / vs_d),
 *                       clamped to [-127, 127]; a zero scale gives code 0.
 * Scales are stored FP32 (round to nearest).  The channel factor's sums,
 * root and geometric mean are float64; the token maximum max_d |K| / c_d is
 * taken over FP32 products |K| * (1 / c_d), within one FP32 ulp of the
 * float64 maximum, and then divided by 127 in float64; the value scale's
 * maximum is exact.  Each code is exactly round-half-even of the float64
 * quotient x / (c_d s_t) (x / vs_d) for the FP32 scales the call stores.
 * Only full pages are accepted: a page still being written is served by the
 * exact tier until it is converted.
 *
 * src_slot, dst_slot: int32 [n] device arrays.  n = 0 is a no-op.
 * Errors: AKV_ERR_ARG (null pointer, n < 0), AKV_ERR_UNSUPPORTED, AKV_ERR_ALIGN.
 */
akv_status akv_quantize_pages(const akv_dims *dims, int32_t n,
                              const uint16_t *k_bf16, const uint16_t *v_bf16,
                              const int32_t *src_slot, const int32_t *dst_slot,
                              int8_t *k_codes, int8_t *v_codes,
                              float *k_chan, float *k_tok, float *v_chan,
                              void *stream);

/*
 * Workspace (bytes, device memory) that akv_decode_attn_int8 and
 * akv_decode_attn_exact need for `batch` requests with page tables of
 * `max_pages` columns: split-K partial outputs.  Deterministic in its
 * arguments; 0 for empty problems.
 */
size_t akv_decode_workspace_bytes(const akv_dims *dims, int32_t batch, int32_t max_pages);

/*
 * akv_decode_attn_int8 -- single-query paged decode that reads int8 pages
 * without expanding them.  ("SYCL" page, "Attention that reads 8-bit
 * history"; "Exact tricks and a two-owner decoder".)
 *
 * For request b and query head j, attends q[b][j] over the n_pages[b] int8
 * pages page_table[b][0 .. n_pages[b]) of KV head j / G:
 *   z_t = softmax_scale * s_t * sum_d (q_d c_d) code_td   (channel factor
 *         folded into the query, token factor after the dot);
 *   online softmax over pages; P times the raw value codes per page, scaled
 *   by the page's per-channel value scale at the page boundary.
 * Writes the normalised out_o[b][j][:] and out_lse[b][j] (natural log).
 * n_pages[b] = 0 gives O = 0, LSE = -inf.  Any batch size works; batch = 2
 * with equal page counts is the two-owner launch (each request has its own
 * page-table row and its own output rows).
 *
 * n_pages: int32 [batch] device array, each in [0, max_pages].
 * workspace: at least akv_decode_workspace_bytes(dims, batch, max_pages).
 * Errors: AKV_ERR_ARG, AKV_ERR_UNSUPPORTED (also when the split plan's
 * work-groups per request times max_pages reach 2^32, never below 65,536
 * pages), AKV_ERR_ALIGN, AKV_ERR_WORKSPACE.
 */
akv_status akv_decode_attn_int8(const akv_dims *dims, int32_t batch, const uint16_t *q,
                                const int8_t *k_codes, const int8_t *v_codes,
                                const float *k_chan, const float *k_tok, const float *v_chan,
                                const int32_t *page_table, const int32_t *n_pages,
                                int32_t max_pages, float softmax_scale,
                                float *out_o, float *out_lse,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * akv_decode_attn_exact -- exact BF16 paged decode that also returns the
 * log-sum-exp statistic.  ("SYCL" page, "A merge that joins the tiers":
 * the paged decode gains an LSE output initialised to -inf.)
 *
 * For request b, attends over the first seq_len[b] tokens of the BF16 pages
 * page_table[b][0 .. ceil(seq_len[b] / P)); the last page may be partial
 * (tokens past seq_len are masked).  seq_len[b] = 0 gives O = 0, LSE = -inf.
 * seq_len: int32 [batch] device array, each in [0, max_pages * P].
 * Errors as akv_decode_attn_int8.
 */
akv_status akv_decode_attn_exact(const akv_dims *dims, int32_t batch, const uint16_t *q,
                                 const uint16_t *k_bf16, const uint16_t *v_bf16,
                                 const int32_t *page_table, const int32_t *seq_len,
                                 int32_t max_pages, float softmax_scale,
                                 float *out_o, float *out_lse,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * akv_decode_hybrid -- one layer of the hybrid tier in two launches: the
 * int8 pages (as akv_decode_attn_int8) and the BF16 recent window (as
 * akv_decode_attn_exact) are decoded by one split-K launch whose partials
 * all fold, exactly, in one second pass.  ("ActiveKV" page, "The idea":
 * recent context exact, older history 8-bit, combined with exact attention
 * arithmetic; "SYCL" page, "A merge that joins the tiers".)
 *
 * The result equals akv_merge_lse of the two separate calls' outputs up to
 * FP32 rounding order.  Either tier may be empty (max_pages_* = 0 or zero
 * counts); both empty gives O = 0, LSE = -inf.
 * workspace: at least akv_decode_hybrid_workspace_bytes(dims, batch,
 * max_pages_int8, max_pages_window).
 * Errors: AKV_ERR_ARG, AKV_ERR_UNSUPPORTED (as akv_decode_attn_int8 for the
 * int8 tier's split plan), AKV_ERR_ALIGN, AKV_ERR_WORKSPACE.
 */
size_t akv_decode_hybrid_workspace_bytes(const akv_dims *dims, int32_t batch, int32_t max_pages_int8,
                                         int32_t max_pages_window);
akv_status akv_decode_hybrid(const akv_dims *dims, int32_t batch, const uint16_t *q,
                             const int8_t *k_codes, const int8_t *v_codes,
                             const float *k_chan, const float *k_tok, const float *v_chan,
                             const int32_t *page_table_int8, const int32_t *n_pages_int8,
                             int32_t max_pages_int8,
                             const uint16_t *k_bf16, const uint16_t *v_bf16,
                             const int32_t *page_table_window, const int32_t *window_len,
                             int32_t max_pages_window, float softmax_scale,
                             float *out_o, float *out_lse,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * akv_decode_hybrid_static -- akv_decode_hybrid without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It calls no
 * allocating routine.  The split partials live in a library-owned device
 * array of AKV_STATIC_SCRATCH_BYTES on each GPU the library runs on (held
 * until the process ends); its address is looked up once per device, on the
 * first call made with that device current.  Same arguments, kernels and
 * results as akv_decode_hybrid.
 *
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there: two calls that overlap on one GPU (different streams, or threads
 * without ordering between their streams) race and give wrong results.
 * Nothing in the array has to start at zero; each call writes every partial
 * slot it reads.
 * Errors: as akv_decode_hybrid; AKV_ERR_WORKSPACE (nothing enqueued) when
 * akv_decode_hybrid_workspace_bytes(dims, batch, max_pages_int8,
 * max_pages_window) exceeds AKV_STATIC_SCRATCH_BYTES (16 MiB; with the
 * library's plan at Hkv = 4, G = 6 that holds, e.g., 256 requests of 16K
 * tokens or one request of 1M tokens);
 * AKV_ERR_HIP if the array's address cannot be found.
 */
#define AKV_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
akv_status akv_decode_hybrid_static(const akv_dims *dims, int32_t batch, const uint16_t *q,
                                    const int8_t *k_codes, const int8_t *v_codes,
                                    const float *k_chan, const float *k_tok, const float *v_chan,
                                    const int32_t *page_table_int8, const int32_t *n_pages_int8,
                                    int32_t max_pages_int8,
                                    const uint16_t *k_bf16, const uint16_t *v_bf16,
                                    const int32_t *page_table_window, const int32_t *window_len,
                                    int32_t max_pages_window, float softmax_scale,
                                    float *out_o, float *out_lse, void *stream);

/*
 * akv_merge_lse -- fold one partial into an FP32 accumulator, exactly.
 * ("SYCL" page, "A merge that joins the tiers".)
 *
 * For each of `rows` rows:  L = log(exp(acc_lse) + exp(part_lse));
 *   acc_o = exp(acc_lse - L) acc_o + exp(part_lse - L) part_o;  acc_lse = L.
 * A -inf LSE is an empty partial: merging it leaves the other side as is;
 * two empties give O = 0, LSE = -inf.  acc_o/acc_lse are read and written
 * in place (start them with akv_fill_empty).  acc_o, part_o: [rows][head_dim].
 * Errors: AKV_ERR_ARG, AKV_ERR_ALIGN.
 */
akv_status akv_merge_lse(int32_t rows, int32_t head_dim, float *acc_o, float *acc_lse,
                         const float *part_o, const float *part_lse, void *stream);

/* Set rows to the empty partial: O = 0, LSE = -inf (a kernel, graph-safe). */
akv_status akv_fill_empty(int32_t rows, int32_t head_dim, float *o, float *lse, void *stream);

/*
 * Streaming page publication ("Model quantization" page, "An 8-bit page
 * format shaped for its kernel": pages are converted in the background, and
 * only once they are full in every layer; a page not yet published is read
 * by the exact tier, so decode never waits for a conversion).
 *
 * akv_publish_pages: on side_stream, waits for ready_event (if not NULL;
 *   recorded by the caller on its compute stream once the pages are full),
 *   converts the n pages exactly as akv_quantize_pages does (same arguments
 *   and layouts), then records done_event (if not NULL).  Call it once per
 *   layer (each layer has its own pools); pass done_event on the last call.
 *   Returns at once.  Errors as akv_quantize_pages, plus AKV_ERR_HIP.
 * akv_tables_advance: one small kernel on `stream`, to be enqueued after the
 *   caller has seen done_event complete (hipEventQuery; the host never waits
 *   for it).  For each request b (device int32 arrays, 4-byte aligned):
 *   count[b] pages are published -- new_int8[b][0 .. count[b]) (row stride
 *   max_new) are appended at int8_table[b][n_pages_int8[b] ..] and
 *   n_pages_int8[b] grows by count[b]; the first count[b] entries of
 *   window_table[b] are dropped and its other max_pages_window - count[b]
 *   entries move to the front (slots reserved past the window's current
 *   pages move with them; the last count[b] entries keep their values), and
 *   window_len[b] shrinks by 64 * count[b].  A row whose update would not fit
 *   (count < 0 or > max_new, int8 table full, or fewer than 64 * count
 *   window tokens) is left unchanged and, if `status` (device int32 [batch])
 *   is not NULL, flagged -1 there (0 otherwise).  The caller owns all arrays.
 *   Errors: AKV_ERR_ARG, AKV_ERR_ALIGN, AKV_ERR_HIP.
 */
akv_status akv_publish_pages(const akv_dims *dims, int32_t n, const uint16_t *k_bf16, const uint16_t *v_bf16,
                             const int32_t *src_slot, const int32_t *dst_slot, int8_t *k_codes, int8_t *v_codes,
                             float *k_chan, float *k_tok, float *v_chan, void *ready_event, void *side_stream,
                             void *done_event);
akv_status akv_tables_advance(int32_t batch, const int32_t *count, const int32_t *new_int8, int32_t max_new,
                              int32_t *int8_table, int32_t *n_pages_int8, int32_t max_pages_int8,
                              int32_t *window_table, int32_t *window_len, int32_t max_pages_window,
                              int32_t *status, void *stream);

/*
 * Lossless 13-bit tier ("Model quantization" page, "A lossless tier first":
 * 13 bits per value, a 32-entry table per plane, a raw fallback for a plane
 * that needs more).  A plane is one page of one KV head, keys or values
 * (16,384 BF16 values).  Its table lists the plane's distinct BF16 high
 * bytes (sign and the upper seven exponent bits) in ascending order, unused
 * entries 0; each value is stored as the 5-bit position of its high byte in
 * the table plus its low byte, 13 bits, so a coded plane takes 26,624 bytes.
 * A plane with more than 32 distinct high bytes is stored raw: its 32,768
 * bytes exactly as in the BF16 pool.  Decoding is exact for every bit
 * pattern (NaN payloads, signed zeros, subnormals).
 *
 * Record storage (caller-owned device memory; record slots play the role
 * of pool slots in page tables):
 *   l13_desc   int32 [slot][Hkv][2]       (keys 0, values 1):
 *              (byte offset of the plane in the arena / 256) << 1 | raw
 *   l13_table  uint8 [slot][Hkv][2][32]
 *   l13_arena  bytes, 256-byte aligned; planes at 256-byte aligned offsets.
 * Inside a coded plane, lane slot (w, l, v) (w < 4, l < 64, v < 64; n = l % 16,
 * g = l / 16) stands for
 *   keys:    token 16 (n / 4) + 4 (v / 16) + n % 4, channel 64 w + 16 g + 8 ((v / 8) % 2) + v % 8
 *   values:  channel 64 w + 16 ((v / 16) % 4) + n, token 16 g + 8 ((v / 8) % 2) + v % 8
 * and its low byte is at byte ((4 w + v / 16) * 64 + l) * 16 + v % 16; bits
 * 0-3 of its table position at byte 16384 + ((2 w + v / 32) * 64 + l) * 16
 * + 4 ((v / 8) % 4) + v % 4 (low nibble when (v / 4) % 2 = 0, else high);
 * bit 4 at byte 24576 + (w * 64 + l) * 8 + 4 (v / 32) + v % 4, bit (v / 4) % 8.
 * (This is the order in which the decode kernel's lanes consume values.)
 *
 * akv_l13_encode_pages: encodes both planes of every KV head of BF16 pool
 *   pages src_slot[i] into record slots dst_slot[i] (i < n; dst slots
 *   distinct).  Planes are packed back to back from byte arena_offset
 *   (a multiple of 256) in the order (i, head, keys then values); coded
 *   planes take 26,624 bytes, raw ones 32,768.  The call is refused with
 *   AKV_ERR_BUDGET, nothing enqueued, unless arena_offset + n * Hkv * 2 *
 *   32,768 <= arena_bytes (room even if every plane is raw); offsets must
 *   stay below 256 GiB.  *arena_end (device int64, 8-byte aligned) receives
 *   the byte offset just past the last plane (arena_offset when n = 0; then
 *   only arena_end is used and the other pointers may be NULL): the
 *   arena_offset of a following call, and the byte count to stage.  Three
 *   kernels on `stream`; src_slot and dst_slot are device int32 arrays.
 *   Errors: AKV_ERR_ARG, AKV_ERR_UNSUPPORTED, AKV_ERR_ALIGN, AKV_ERR_BUDGET.
 * akv_l13_decode_pages: writes record slots src_slot[i] back into BF16 pool
 *   slots dst_slot[i] (both planes, every head), bit-exactly.
 *   Errors: AKV_ERR_ARG, AKV_ERR_UNSUPPORTED, AKV_ERR_ALIGN.
 * akv_decode_attn_l13: akv_decode_attn_exact over 13-bit records, reading
 *   them directly (coded planes are expanded to BF16 in registers, raw
 *   planes read as BF16); page_table holds record slots.  Same split plan and
 *   arithmetic as akv_decode_attn_exact, so the result is bit-identical to it
 *   on the decoded pages.  Descriptors must come from akv_l13_encode_pages.
 *   workspace: at least akv_decode_workspace_bytes(dims, batch, max_pages).
 *   Errors as akv_decode_attn_exact (the arena must be 256-byte aligned).
 */
akv_status akv_l13_encode_pages(const akv_dims *dims, int32_t n, const uint16_t *k_bf16, const uint16_t *v_bf16,
                                const int32_t *src_slot, const int32_t *dst_slot,
                                uint8_t *l13_arena, int64_t arena_offset, int64_t arena_bytes,
                                int32_t *l13_desc, uint8_t *l13_table, int64_t *arena_end, void *stream);
akv_status akv_l13_decode_pages(const akv_dims *dims, int32_t n, const uint8_t *l13_arena,
                                const int32_t *l13_desc, const uint8_t *l13_table,
                                const int32_t *src_slot, const int32_t *dst_slot,
                                uint16_t *k_bf16, uint16_t *v_bf16, void *stream);
akv_status akv_decode_attn_l13(const akv_dims *dims, int32_t batch, const uint16_t *q,
                               const uint8_t *l13_arena, const int32_t *l13_desc, const uint8_t *l13_table,
                               const int32_t *page_table, const int32_t *seq_len, int32_t max_pages,
                               float softmax_scale, float *out_o, float *out_lse,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Host-staged mode ("ActiveKV" page, "The idea" and "What I built"): the
 * authoritative history sits in pinned host memory and each step stages one
 * layer at a time into a ring of device slots, with events so a slot is
 * never overwritten while a copy or kernel still uses it.
 *
 * akv_ring_create: slots[i] are caller-owned device buffers of slot_bytes
 *   each (n_slots >= 2).  The ring owns only its HIP events.
 * akv_ring_stage: for `layer`, waits (on copy_stream) until the slot
 *   layer % n_slots was released by its previous user, enqueues n_srcs
 *   host-to-device copies (host_srcs[k] must be pinned host memory) packed
 *   back to back at 256-byte aligned offsets into that slot, records
 *   copy-done, and makes compute_stream wait for it.  *slot_out receives
 *   the slot's device address and offsets[k] (if not NULL) each source's
 *   offset.  A request larger than slot_bytes returns AKV_ERR_BUDGET before
 *   anything is enqueued.  Staging a layer whose slot has not been released
 *   since it was last staged returns AKV_ERR_STATE.
 * akv_ring_release: records on compute_stream that `layer`'s slot may be
 *   reused (call after the kernels that read it are enqueued).
 * akv_ring_destroy: releases the events (synchronizes them first).
 */
typedef struct akv_ring akv_ring;
akv_status akv_ring_create(void *const *slots, size_t slot_bytes, int32_t n_slots, akv_ring **out);
akv_status akv_ring_stage(akv_ring *ring, int32_t layer, const void *const *host_srcs,
                          const size_t *bytes, int32_t n_srcs, void *copy_stream,
                          void *compute_stream, void **slot_out, size_t *offsets);
akv_status akv_ring_release(akv_ring *ring, int32_t layer, void *compute_stream);
akv_status akv_ring_destroy(akv_ring *ring);

#ifdef __cplusplus
}
#endif
#endif /* AKV_H */
