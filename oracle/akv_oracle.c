/*
 * akv_oracle.c -- plain, slow, float64 CPU oracle for ActiveKV hybrid-tier
 * decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no source,
 * header, table or helper with the HIP library under
 * quantized_paged_kv_akv_amd/csrc; neither includes nor links the other.
 *
 * Sources (the four web pages on ActiveKV; cited by page title + section):
 *   [FMT]   "Model quantization" technology page, section "An 8-bit page
 *           format shaped for its kernel": keys get a separable scale, the
 *           per-channel factor is the square root of the channel RMS over the
 *           page, normalised so the channel factors multiply to one, clamped
 *           to 2^+-14; a per-token-per-head factor covers the rest; codes are
 *           symmetric in [-127, 127]; values get one scale per channel per
 *           page.  Only fully written pages are converted.
 *   [INT8]  "SYCL" technology page, section "Attention that reads 8-bit
 *           history": the channel factor leaves the inner loop, the per-token
 *           factor is applied after the dot product, PV accumulates on raw
 *           value codes and is rescaled at each page boundary.
 *   [MERGE] "SYCL" technology page, section "A merge that joins the tiers":
 *           partials from each tier fold into one FP32 accumulator; the
 *           log-sum-exp row starts at -infinity so an unwritten row is a valid
 *           empty partial.  "ActiveKV" systems page, section "The idea": the
 *           two tiers combine with exact attention arithmetic.
 *
 * Readings where the pages are silent:
 *   - "RMS over the page" = sqrt(mean over the page's tokens of K^2), per
 *     (page, KV head, channel).  The factor is sqrt(RMS) = ms^(1/4).
 *   - Normalisation divides by the geometric mean of the factors of the
 *     channels with nonzero RMS, THEN clamps (sentence order).  A channel with
 *     zero RMS gets factor 1 and is left out of the geometric mean.
 *   - Per-token factor s_t = max_d(|K[t,d]| / c32_d) / 127, from the FP32
 *     channel factors as stored; value scale vs_d = max_t |V[t,d]| / 127.
 *   - Scales are computed in float64 and stored as FP32 (round to nearest).
 *   - Code = clamp(round_half_even(K / (c32 * s32)), -127, 127) with the
 *     quotient taken in float64 (the product of two FP32 numbers is exact in
 *     float64, the division is correctly rounded).  A zero scale gives code 0.
 *   - LSE is the natural log of sum_t exp(sigma * q . k_t).  Empty -> -inf.
 *
 * Pool layouts read here (the boundary's, stated in include/akv.h; this file
 * indexes them with its own code):
 *   BF16 K  [slot][Hkv][P][D]   token-major
 *   BF16 V  [slot][Hkv][D][P]   channel-major
 *   int8 K  [slot][Hkv][P][D],  int8 V [slot][Hkv][D][P]
 *   k_chan  [slot][Hkv][D], k_tok [slot][Hkv][P], v_chan [slot][Hkv][D]  (f32)
 *   q       [B][Hkv*G][D] BF16; query head j reads KV head j / G.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define AKVO_CODE_MAX 127.0
#define AKVO_CLAMP_LO (1.0 / 16384.0) /* 2^-14 */
#define AKVO_CLAMP_HI 16384.0         /* 2^14 */

double akvo_bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------- */
/* Quantizer, stage 1: the scales of one (page, KV head).  [FMT]              */
/* K and V are float64, token-major [P][D].                                  */
/* ------------------------------------------------------------------------- */
int akvo_page_scales(int P, int D, const double *K, const double *V,
                     double *c64, float *c32, float *s32, float *vs32)
{
    if (P <= 0 || D <= 0) return -1;
    double *ms = (double *)malloc(sizeof(double) * (size_t)D);
    if (!ms) return -2;

    /* mean square of each channel over the page's tokens */
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = 0; t < P; ++t) {
            double k = K[(size_t)t * D + d];
            acc += k * k;
        }
        ms[d] = acc / (double)P;
    }

    /* factor u_d = sqrt(RMS_d) = ms_d^(1/4); geometric mean over channels
       whose RMS is nonzero */
    double log_sum = 0.0;
    int n_nonzero = 0;
    for (int d = 0; d < D; ++d) {
        if (ms[d] > 0.0) {
            double u = sqrt(sqrt(ms[d]));
            log_sum += log(u);
            n_nonzero += 1;
        }
    }
    double g = (n_nonzero > 0) ? exp(log_sum / (double)n_nonzero) : 1.0;

    /* normalise so the factors multiply to one, then clamp to 2^+-14 */
    for (int d = 0; d < D; ++d) {
        double c;
        if (ms[d] > 0.0) {
            c = sqrt(sqrt(ms[d])) / g;
            if (c < AKVO_CLAMP_LO) c = AKVO_CLAMP_LO;
            if (c > AKVO_CLAMP_HI) c = AKVO_CLAMP_HI;
        } else {
            c = 1.0;
        }
        c64[d] = c;
        c32[d] = (float)c;
    }

    /* per-token-per-head factor covers the rest of the range */
    for (int t = 0; t < P; ++t) {
        double m = 0.0;
        for (int d = 0; d < D; ++d) {
            double a = fabs(K[(size_t)t * D + d]) / (double)c32[d];
            if (a > m) m = a;
        }
        s32[t] = (float)(m / AKVO_CODE_MAX);
    }

    /* one value scale per channel per page */
    for (int d = 0; d < D; ++d) {
        double m = 0.0;
        for (int t = 0; t < P; ++t) {
            double a = fabs(V[(size_t)t * D + d]);
            if (a > m) m = a;
        }
        vs32[d] = (float)(m / AKVO_CODE_MAX);
    }
    free(ms);
    return 0;
}

/* one symmetric code; *tie set when the float64 quotient is exactly k+0.5 */
static int8_t akvo_code(double x, double scale, int *tie)
{
    *tie = 0;
    if (scale == 0.0) return 0;
    double q = x / scale;
    double fl = floor(q);
    if (q - fl == 0.5) *tie = 1;
    double r = nearbyint(q); /* default rounding mode: half to even */
    if (r > AKVO_CODE_MAX) r = AKVO_CODE_MAX;
    if (r < -AKVO_CODE_MAX) r = -AKVO_CODE_MAX;
    return (int8_t)r;
}

/* ------------------------------------------------------------------------- */
/* Quantizer, stage 2: codes of one (page, KV head) given FP32 scales.        */
/* K, V float64 token-major [P][D]; codes out token-major [P][D].            */
/* Returns the number of exact ties; tie masks may be NULL.                  */
/* ------------------------------------------------------------------------- */
int akvo_page_codes(int P, int D, const double *K, const double *V,
                    const float *c32, const float *s32, const float *vs32,
                    int8_t *kcode, int8_t *vcode, uint8_t *ktie, uint8_t *vtie)
{
    int ties = 0;
    for (int t = 0; t < P; ++t) {
        for (int d = 0; d < D; ++d) {
            size_t i = (size_t)t * D + d;
            int tie;
            /* c32*s32 is exact in float64 (24+24 significant bits) */
            kcode[i] = akvo_code(K[i], (double)c32[d] * (double)s32[t], &tie);
            if (ktie) ktie[i] = (uint8_t)tie;
            ties += tie;
            vcode[i] = akvo_code(V[i], (double)vs32[d], &tie);
            if (vtie) vtie[i] = (uint8_t)tie;
            ties += tie;
        }
    }
    return ties;
}

/* gather one (slot, head) BF16 page into float64 token-major K and V */
static void akvo_load_bf16_page(int Hkv, int D, int P, const uint16_t *kpool,
                                const uint16_t *vpool, int slot, int h,
                                double *K, double *V)
{
    size_t base_k = ((size_t)slot * Hkv + h) * (size_t)P * D;
    size_t base_v = base_k; /* same page-head size, channel-major inside */
    for (int t = 0; t < P; ++t)
        for (int d = 0; d < D; ++d) {
            K[(size_t)t * D + d] = akvo_bf16_to_f64(kpool[base_k + (size_t)t * D + d]);
            V[(size_t)t * D + d] = akvo_bf16_to_f64(vpool[base_v + (size_t)d * P + t]);
        }
}

/* ------------------------------------------------------------------------- */
/* Quantize n full BF16 pages from pool slots src[i] into int8 pool slots    */
/* dst[i], all KV heads.  Writes codes in the pool layouts and FP32 scales.  */
/* If use_given_scales != 0 the scales already in k_chan/k_tok/v_chan are    */
/* used for stage 2 (stage-2 agreement check) and left unchanged.            */
/* tie_count receives the number of exact ties; k_ties / v_ties (may be      */
/* NULL) receive 0/1 tie masks in the code pools' layouts.  [FMT]            */
/* ------------------------------------------------------------------------- */
int akvo_quantize_pages(int n, int Hkv, int D, int P,
                        const uint16_t *kpool, const uint16_t *vpool,
                        const int32_t *src, const int32_t *dst,
                        int8_t *kcodes, int8_t *vcodes,
                        float *k_chan, float *k_tok, float *v_chan,
                        int use_given_scales, int64_t *tie_count,
                        uint8_t *k_ties, uint8_t *v_ties)
{
    int64_t ties_total = 0;
    int err = 0;
#pragma omp parallel for schedule(dynamic) reduction(+ : ties_total) reduction(| : err)
    for (int u = 0; u < n * Hkv; ++u) {
        int i = u / Hkv, h = u % Hkv;
        size_t PD = (size_t)P * D;
        double *K = (double *)malloc(sizeof(double) * PD);
        double *V = (double *)malloc(sizeof(double) * PD);
        double *c64 = (double *)malloc(sizeof(double) * (size_t)D);
        int8_t *kc = (int8_t *)malloc(PD);
        int8_t *vc = (int8_t *)malloc(PD);
        uint8_t *kt = (uint8_t *)malloc(PD);
        uint8_t *vt = (uint8_t *)malloc(PD);
        if (!K || !V || !c64 || !kc || !vc || !kt || !vt) {
            err |= 1;
        } else {
            akvo_load_bf16_page(Hkv, D, P, kpool, vpool, src[i], h, K, V);
            size_t ph = (size_t)dst[i] * Hkv + h;
            float *c32 = k_chan + ph * D;
            float *s32 = k_tok + ph * P;
            float *vs32 = v_chan + ph * D;
            if (!use_given_scales) akvo_page_scales(P, D, K, V, c64, c32, s32, vs32);
            ties_total += akvo_page_codes(P, D, K, V, c32, s32, vs32, kc, vc, kt, vt);
            int8_t *kout = kcodes + ph * PD;
            int8_t *vout = vcodes + ph * PD;
            for (int t = 0; t < P; ++t)
                for (int d = 0; d < D; ++d) {
                    kout[(size_t)t * D + d] = kc[(size_t)t * D + d];
                    vout[(size_t)d * P + t] = vc[(size_t)t * D + d];
                    if (k_ties) k_ties[ph * PD + (size_t)t * D + d] = kt[(size_t)t * D + d];
                    if (v_ties) v_ties[ph * PD + (size_t)d * P + t] = vt[(size_t)t * D + d];
                }
        }
        free(K); free(V); free(c64); free(kc); free(vc); free(kt); free(vt);
    }
    if (tie_count) *tie_count = ties_total;
    return err ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Dense softmax attention for one query row over n tokens (the plain        */
/* definition).  K, V float64 [n][D].  Empty -> O = 0, lse = -inf.           */
/* ------------------------------------------------------------------------- */
int akvo_attend(int n, int D, const double *q, const double *K, const double *V,
                double sigma, double *O, double *lse)
{
    for (int d = 0; d < D; ++d) O[d] = 0.0;
    if (n <= 0) { *lse = -INFINITY; return 0; }
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    if (!z) return -2;
    double M = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += q[d] * K[(size_t)t * D + d];
        z[t] = sigma * acc;
        if (z[t] > M) M = z[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(z[t] - M);
        l += w;
        for (int d = 0; d < D; ++d) O[d] += w * V[(size_t)t * D + d];
    }
    for (int d = 0; d < D; ++d) O[d] /= l;
    *lse = M + log(l);
    free(z);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Merge of partials (O_i, lse_i), the exact log-sum-exp combination.        */
/* parts_O [n_parts][rows][D], parts_lse [n_parts][rows].  Partials with     */
/* lse = -inf are empty and skipped; all empty -> (0, -inf).  [MERGE]        */
/* ------------------------------------------------------------------------- */
int akvo_merge(int n_parts, int rows, int D, const double *parts_O,
               const double *parts_lse, double *O, double *lse)
{
    for (int r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int i = 0; i < n_parts; ++i) {
            double v = parts_lse[(size_t)i * rows + r];
            if (v > M) M = v;
        }
        double *o = O + (size_t)r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double l = 0.0;
        for (int i = 0; i < n_parts; ++i) {
            double v = parts_lse[(size_t)i * rows + r];
            if (v == -INFINITY) continue;
            l += exp(v - M);
        }
        double L = M + log(l);
        for (int i = 0; i < n_parts; ++i) {
            double v = parts_lse[(size_t)i * rows + r];
            if (v == -INFINITY) continue;
            double w = exp(v - L);
            const double *po = parts_O + ((size_t)i * rows + r) * D;
            for (int d = 0; d < D; ++d) o[d] += w * po[d];
        }
        lse[r] = L;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact (BF16) decode over paged history: for each request b and query head */
/* j, dense attention over the first seq_len[b] tokens of the pages listed   */
/* in page_table[b][..].  O [B][Hq][D], lse [B][Hq].                         */
/* ------------------------------------------------------------------------- */
int akvo_decode_exact(int B, int Hkv, int G, int D, int P, const uint16_t *q,
                      const uint16_t *kpool, const uint16_t *vpool,
                      const int32_t *page_table, const int32_t *seq_len,
                      int max_pages, double sigma, double *O, double *lse)
{
    int Hq = Hkv * G;
    int err = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int u = 0; u < B * Hkv; ++u) {
        int b = u / Hkv, h = u % Hkv;
        int n = seq_len[b];
        size_t PD = (size_t)P * D;
        int npg = (n + P - 1) / P;
        double *K = (double *)malloc(sizeof(double) * (size_t)(npg > 0 ? npg : 1) * PD);
        double *V = (double *)malloc(sizeof(double) * (size_t)(npg > 0 ? npg : 1) * PD);
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!K || !V || !qd) { err |= 1; free(K); free(V); free(qd); continue; }
        for (int p = 0; p < npg; ++p) {
            int slot = page_table[(size_t)b * max_pages + p];
            akvo_load_bf16_page(Hkv, D, P, kpool, vpool, slot, h, K + p * PD, V + p * PD);
        }
        for (int g = 0; g < G; ++g) {
            int j = h * G + g;
            for (int d = 0; d < D; ++d)
                qd[d] = akvo_bf16_to_f64(q[((size_t)b * Hq + j) * D + d]);
            akvo_attend(n, D, qd, K, V, sigma, O + ((size_t)b * Hq + j) * D,
                        lse + (size_t)b * Hq + j);
        }
        free(K); free(V); free(qd);
    }
    return err ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* int8-tier decode over paged codes.                                         */
/*  mode 0: dequantize every page (K^ = code*c*s, V^ = code*vs) and apply    */
/*          the plain dense definition (akvo_attend).                        */
/*  mode 1: the int8-path formula in the pages' order [INT8]: per page,      */
/*          q' = q (.) c_page; z_t = sigma * s_t * sum_d q'_d code_td;       */
/*          online softmax with a running maximum rescaled at each page;     */
/*          PV accumulated on raw value codes within the page and scaled by  */
/*          the page's per-channel value scale at the page boundary.         */
/* Both must agree to rounding; mode 1 is a check of the formula.            */
/* ------------------------------------------------------------------------- */
int akvo_decode_int8(int B, int Hkv, int G, int D, int P, const uint16_t *q,
                     const int8_t *kcodes, const int8_t *vcodes,
                     const float *k_chan, const float *k_tok, const float *v_chan,
                     const int32_t *page_table, const int32_t *n_pages,
                     int max_pages, double sigma, int mode, double *O, double *lse)
{
    int Hq = Hkv * G;
    int err = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int u = 0; u < B * Hkv; ++u) {
        int b = u / Hkv, h = u % Hkv;
        int np = n_pages[b];
        size_t PD = (size_t)P * D;
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!qd) { err |= 1; continue; }
        if (mode == 0) {
            size_t n = (size_t)(np > 0 ? np : 1) * PD;
            double *K = (double *)malloc(sizeof(double) * n);
            double *V = (double *)malloc(sizeof(double) * n);
            if (!K || !V) { err |= 1; free(K); free(V); free(qd); continue; }
            for (int p = 0; p < np; ++p) {
                size_t ph = (size_t)page_table[(size_t)b * max_pages + p] * Hkv + h;
                const int8_t *kc = kcodes + ph * PD;
                const int8_t *vc = vcodes + ph * PD;
                const float *c = k_chan + ph * D, *s = k_tok + ph * P, *vs = v_chan + ph * D;
                for (int t = 0; t < P; ++t)
                    for (int d = 0; d < D; ++d) {
                        K[p * PD + (size_t)t * D + d] =
                            (double)kc[(size_t)t * D + d] * (double)c[d] * (double)s[t];
                        V[p * PD + (size_t)t * D + d] =
                            (double)vc[(size_t)d * P + t] * (double)vs[d];
                    }
            }
            for (int g = 0; g < G; ++g) {
                int j = h * G + g;
                for (int d = 0; d < D; ++d)
                    qd[d] = akvo_bf16_to_f64(q[((size_t)b * Hq + j) * D + d]);
                akvo_attend(np * P, D, qd, K, V, sigma, O + ((size_t)b * Hq + j) * D,
                            lse + (size_t)b * Hq + j);
            }
            free(K); free(V);
        } else {
            double *qp = (double *)malloc(sizeof(double) * (size_t)D);
            double *z = (double *)malloc(sizeof(double) * (size_t)P);
            double *acc = (double *)malloc(sizeof(double) * (size_t)D);
            if (!qp || !z || !acc) { err |= 1; free(qp); free(z); free(acc); free(qd); continue; }
            for (int g = 0; g < G; ++g) {
                int j = h * G + g;
                double *o = O + ((size_t)b * Hq + j) * D;
                for (int d = 0; d < D; ++d) {
                    qd[d] = akvo_bf16_to_f64(q[((size_t)b * Hq + j) * D + d]);
                    o[d] = 0.0;
                }
                double M = -INFINITY, l = 0.0;
                for (int p = 0; p < np; ++p) {
                    size_t ph = (size_t)page_table[(size_t)b * max_pages + p] * Hkv + h;
                    const int8_t *kc = kcodes + ph * PD;
                    const int8_t *vc = vcodes + ph * PD;
                    const float *c = k_chan + ph * D, *s = k_tok + ph * P, *vs = v_chan + ph * D;
                    /* the channel factor leaves the inner loop: fold it into q */
                    for (int d = 0; d < D; ++d) qp[d] = qd[d] * (double)c[d];
                    double pm = -INFINITY;
                    for (int t = 0; t < P; ++t) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += qp[d] * (double)kc[(size_t)t * D + d];
                        z[t] = sigma * (double)s[t] * dot; /* token factor after the dot */
                        if (z[t] > pm) pm = z[t];
                    }
                    double Mn = pm > M ? pm : M;
                    double alpha = (M == -INFINITY) ? 0.0 : exp(M - Mn);
                    /* PV on raw value codes within the page */
                    for (int d = 0; d < D; ++d) acc[d] = 0.0;
                    double lp = 0.0;
                    for (int t = 0; t < P; ++t) {
                        double w = exp(z[t] - Mn);
                        lp += w;
                        for (int d = 0; d < D; ++d) acc[d] += w * (double)vc[(size_t)d * P + t];
                    }
                    /* page boundary: rescale the accumulator, apply value scale */
                    for (int d = 0; d < D; ++d) o[d] = alpha * o[d] + (double)vs[d] * acc[d];
                    l = alpha * l + lp;
                    M = Mn;
                }
                if (np <= 0) {
                    lse[(size_t)b * Hq + j] = -INFINITY;
                } else {
                    for (int d = 0; d < D; ++d) o[d] /= l;
                    lse[(size_t)b * Hq + j] = M + log(l);
                }
            }
            free(qp); free(z); free(acc);
        }
        free(qd);
    }
    return err ? -2 : 0;
}

/* number of OpenMP threads this library would use (for reporting) */
int akvo_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
