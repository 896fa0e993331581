/* Plain CPU oracle for DeepSeek-V4.1 sparse latent attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the bench's CPU-baseline leg use this file; the
 * GPU library never includes, links or calls it, and the two share no code. It is written
 * for reading, not speed: one query at a time, sums in index order, no blocking or fusion.
 * Citations name the page and the passage (see sa_oracle.h for the page list).
 */
#include "sa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int32_t orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------ */
/* bf16 <-> f32. [attn-docs] precision paragraph: tensors are bf16, arithmetic is f32.   */
/* The pages do not name a rounding mode for "returns bf16"; the reading taken is        */
/* round-to-nearest-even, which is what a torch .to(bfloat16) cast does.                 */
/* ------------------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* NaN stays a (quiet) NaN */
    uint32_t upper = u >> 16;                             /* truncated result */
    uint32_t lower = u & 0xffffu;                         /* discarded bits */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1;                                       /* nearest, ties to even */
    return (uint16_t)upper;
}

void orc_f32_to_bf16_array(const float *x, uint16_t *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(x[i]);
}

void orc_bf16_to_f32_array(const uint16_t *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16_to_f32(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* pow2_ceil. [attn-docs] pow2_ceil: 2**ceil(log2 v) for a positive normal f32, read off  */
/* the IEEE fields. With biased exponent E and mantissa M, v = 2^(E-127) * (1 + M/2^23); */
/* log2 v is an integer exactly when M == 0, otherwise its ceiling is E-127+1.           */
/* ------------------------------------------------------------------------------------ */
float orc_pow2_ceil(float v)
{
    uint32_t u = f32_bits(v);
    uint32_t e = (u >> 23) & 0xffu;
    uint32_t m = u & 0x7fffffu;
    if (m != 0) e += 1;
    return bits_f32(e << 23);
}

/* ------------------------------------------------------------------------------------ */
/* e4m3. [attn-docs] act_quant_inplace: values go to e4m3 with round-to-nearest-even,    */
/* clamped. The 448 bound of the same passage is the OCP "e4m3fn" variant: bias 7,       */
/* 3 mantissa bits, largest finite 1.75 * 2^8 = 448, subnormal step 2^-9, no infinity.   */
/* Reading: the clamp to +-448 comes before rounding, so nothing ever maps to NaN.       */
/* ------------------------------------------------------------------------------------ */

/* round a non-negative float that is exactly representable as k/2 or finer to the       */
/* nearest integer, ties to even (done by hand so that no rounding mode is assumed)      */
static float round_half_even(float v)
{
    float fl = floorf(v);
    float frac = v - fl;                  /* exact: v and fl share the exponent range */
    if (frac > 0.5f) return fl + 1.0f;
    if (frac < 0.5f) return fl;
    return (fmodf(fl, 2.0f) == 0.0f) ? fl : fl + 1.0f;
}

uint8_t orc_e4m3_encode(float x)
{
    uint8_t sign = (f32_bits(x) >> 31) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (a > 448.0f) a = 448.0f;                               /* clamp */
    if (a < 0.015625f) {                                      /* below 2^-6: subnormal grid */
        float q = round_half_even(a * 512.0f);                /* units of 2^-9, exact scaling */
        return (uint8_t)(sign | (uint8_t)q);                  /* q == 8 is the code of 2^-6 */
    }
    int e2;
    frexpf(a, &e2);                                           /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                                           /* a in [2^e, 2^(e+1)) */
    float q = round_half_even(ldexpf(a, 3 - e));              /* units of 2^(e-3): q in [8, 16] */
    if (q == 16.0f) { q = 8.0f; e += 1; }
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)((int)q - 8));
}

float orc_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    float v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------------------ */
/* Block-32 ue8m0 round trip. [attn-docs] act_quant_inplace and FP8_BLOCK (32): for each */
/* block of 32 consecutive elements of a row, scale = pow2_ceil(max(amax, 1e-4) / 448),  */
/* values to e4m3 (RNE, clamped), dequantised and stored back as bf16. The precision     */
/* paragraph of the same page states the round trip is bf16-exact.                       */
/* Reading: the whole row is quantised, rope tail included ("the KV row quantised").     */
/* The scale byte is the biased exponent of the power-of-two scale (ue8m0).              */
/* ------------------------------------------------------------------------------------ */
int orc_act_quant_rows(const uint16_t *x, int64_t rows, int32_t d, uint16_t *y,
                       uint8_t *codes, uint8_t *scale_bytes)
{
    if (!x || !y || rows < 0 || d <= 0 || d % 32 != 0) return -1;
    const int nb = d / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t *xb = x + r * d + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float v = fabsf(orc_bf16_to_f32(xb[i]));
                if (v > amax) amax = v;
            }
            if (amax < 1e-4f) amax = 1e-4f;
            float s = orc_pow2_ceil(amax / 448.0f);
            uint8_t qc[32];
            for (int i = 0; i < 32; ++i) {
                float v = orc_bf16_to_f32(xb[i]) / s;          /* exact: s is a power of two */
                qc[i] = orc_e4m3_encode(v);
            }
            uint16_t *yb = y + r * d + b * 32;
            for (int i = 0; i < 32; ++i)
                yb[i] = orc_f32_to_bf16(orc_e4m3_decode(qc[i]) * s);
            if (codes) memcpy(codes + r * d + b * 32, qc, 32);
            if (scale_bytes) scale_bytes[r * nb + b] = (uint8_t)((f32_bits(s) >> 23) & 0xffu);
        }
    }
    return 0;
}

int orc_fp8_storage_decode(const uint8_t *codes, const uint8_t *scale_bytes, int64_t rows,
                           int32_t d, uint16_t *y)
{
    if (!codes || !scale_bytes || !y || rows < 0 || d <= 0 || d % 32 != 0) return -1;
    const int nb = d / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < d; ++i) {
            float s = ldexpf(1.0f, (int)scale_bytes[r * nb + i / 32] - 127);
            y[r * d + i] = orc_f32_to_bf16(orc_e4m3_decode(codes[r * d + i]) * s);
        }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Window index lists. [attn-docs] window_topk_idxs: [queries][cols] of slot indices,    */
/* -1 for a slot holding nothing; prefill is one causal window per query into the chunk */
/* itself, decode is the whole ring, oldest first. The ring-cache paragraph fixes the    */
/* slot of token p as p mod window.                                                      */
/* Readings: prefill cols = min(seqlen, window) (the list is [queries][cols], not        */
/* [queries][window]); valid entries come first, oldest first, -1 padding at the end;    */
/* decode lets every sequence carry its own start position; start_pos > 0 with more than */
/* one query (chunked prefill) is not defined by the pages and is rejected. The mode is  */
/* the caller's, as on the pages (prefill vs decode): start_pos == NULL is a prefill     */
/* from position 0, start_pos != NULL a decode step, whose list is the whole ring        */
/* (cols = window) at any position, P = 0 included (the ring then holds token 0 only).   */
/* ------------------------------------------------------------------------------------ */
int orc_window_cols(int32_t window, int32_t seqlen, const int32_t *start_pos, int32_t nseq,
                    int32_t *cols)
{
    if (window <= 0 || seqlen <= 0 || nseq <= 0 || !cols) return -1;
    if (start_pos) {
        for (int32_t n = 0; n < nseq; ++n)
            if (start_pos[n] < 0) return -1;
        if (seqlen > 1) return -2;                       /* chunked prefill: undefined */
        *cols = window;
    } else {
        *cols = seqlen < window ? seqlen : window;
    }
    return 0;
}

int orc_window_topk_idxs(int32_t window, int32_t seqlen, const int32_t *start_pos, int32_t nseq,
                         int32_t *idx, int32_t *cols)
{
    int32_t c;
    int rc = orc_window_cols(window, seqlen, start_pos, nseq, &c);
    if (rc) return rc;
    if (!idx) return -1;
    *cols = c;
    for (int32_t n = 0; n < nseq; ++n) {
        for (int32_t t = 0; t < seqlen; ++t) {
            int32_t *row = idx + ((int64_t)n * seqlen + t) * c;
            if (!start_pos) {
                /* prefill: chunk rows lo..t, lo = max(0, t - window + 1) */
                int32_t lo = t - window + 1 > 0 ? t - window + 1 : 0;
                for (int32_t j = 0; j < c; ++j) row[j] = (lo + j <= t) ? lo + j : -1;
                continue;
            }
            int32_t P = start_pos[n];
            if (P >= window - 1) {
                /* full ring: the oldest token P-window+1 sits in slot (P+1) mod window */
                for (int32_t j = 0; j < c; ++j) row[j] = (P + 1 + j) % window;
            } else {
                /* ring holds tokens 0..P in slots 0..P */
                for (int32_t j = 0; j < c; ++j) row[j] = (j <= P) ? j : -1;
            }
        }
    }
    return 0;
}

void orc_ring_prefill(uint16_t *ring, int32_t window, int32_t row_elems,
                      const uint16_t *chunk_rows, int32_t seqlen)
{
    int32_t first = seqlen - window > 0 ? seqlen - window : 0;
    for (int32_t p = first; p < seqlen; ++p)
        memcpy(ring + (int64_t)(p % window) * row_elems, chunk_rows + (int64_t)p * row_elems,
               (size_t)row_elems * 2);
}

void orc_ring_decode(uint16_t *ring, int32_t window, int32_t row_elems, const uint16_t *row,
                     int32_t pos)
{
    memcpy(ring + (int64_t)(pos % window) * row_elems, row, (size_t)row_elems * 2);
}

/* ------------------------------------------------------------------------------------ */
/* sparse_attn. [attn-docs] sparse_attn: per query and head, a softmax over the gathered */
/* rows plus the sink, the sink entering the denominator only, all in f32, output bf16;  */
/* q [s][h][d], kv [rows][d], idx [s][topk]. [attn-fwd] Attention.forward calls it with  */
/* the per-head f32 attn_sink and softmax_scale = head_dim^-0.5; the same latent row is   */
/* key and value. For the gathered set J = {j : idx_j >= 0}:                             */
/*   s_j = scale * sum_k q[k] kv[idx_j][k]                                               */
/*   p_j = exp(s_j) / (sum_{j in J} exp(s_j) + exp(sink))                                */
/*   o   = sum_{j in J} p_j kv[idx_j]        -> bf16                                     */
/* Readings: the sink is a raw logit (not multiplied by scale); any negative index is a  */
/* skip; an empty J gives o = 0; a duplicated index counts once per occurrence. The      */
/* exponentials are taken relative to m = max(sink, max s_j), which leaves every p_j     */
/* unchanged and keeps them finite.                                                      */
/* ------------------------------------------------------------------------------------ */
static int check_problem(const orc_attn_problem *p, const int64_t *qsel, int64_t nsel)
{
    if (!p || !p->q || !p->kv || !p->sink || !p->idx) return -1;
    if (p->b <= 0 || p->s <= 0 || p->h <= 0 || p->d <= 0 || p->topk <= 0 || p->kv_rows <= 0)
        return -1;
    int64_t nq = (int64_t)p->b * p->s;
    if (qsel) {
        for (int64_t i = 0; i < nsel; ++i)
            if (qsel[i] < 0 || qsel[i] >= nq) return -1;
    } else if (nsel != nq) {
        return -1;
    }
    for (int64_t i = 0; i < nsel; ++i) {
        int64_t qi = qsel ? qsel[i] : i;
        const int32_t *row = p->idx + (qi / p->s) * p->idx_seq_stride + (qi % p->s) * p->topk;
        for (int32_t j = 0; j < p->topk; ++j)
            if (row[j] >= p->kv_rows) return -1;
    }
    return 0;
}

static void attn_one_query_f32(const orc_attn_problem *p, int64_t qi, uint16_t *out,
                               float *srow, float *acc)
{
    const int64_t seq = qi / p->s, t = qi % p->s;
    const int32_t *idx = p->idx + seq * p->idx_seq_stride + t * p->topk;
    const uint16_t *kv = p->kv + seq * p->kv_seq_stride;
    for (int32_t hh = 0; hh < p->h; ++hh) {
        const uint16_t *q = p->q + seq * p->q_seq_stride + (t * p->h + hh) * (int64_t)p->d;
        /* scores */
        float m = p->sink[hh];
        int any = 0;
        for (int32_t j = 0; j < p->topk; ++j) {
            if (idx[j] < 0) continue;
            const uint16_t *k = kv + (int64_t)idx[j] * p->d;
            float dot = 0.0f;
            for (int32_t c = 0; c < p->d; ++c)
                dot += orc_bf16_to_f32(q[c]) * orc_bf16_to_f32(k[c]);
            srow[j] = p->scale * dot;
            if (srow[j] > m) m = srow[j];
            any = 1;
        }
        uint16_t *o = out + (int64_t)hh * p->d;
        if (!any) {                                       /* no rows: only the sink */
            for (int32_t c = 0; c < p->d; ++c) o[c] = orc_f32_to_bf16(0.0f);
            continue;
        }
        /* denominator: the gathered rows plus the sink */
        float l = expf(p->sink[hh] - m);
        for (int32_t j = 0; j < p->topk; ++j)
            if (idx[j] >= 0) l += expf(srow[j] - m);
        /* weighted sum of the same rows */
        for (int32_t c = 0; c < p->d; ++c) acc[c] = 0.0f;
        for (int32_t j = 0; j < p->topk; ++j) {
            if (idx[j] < 0) continue;
            float pj = expf(srow[j] - m) / l;
            const uint16_t *v = kv + (int64_t)idx[j] * p->d;
            for (int32_t c = 0; c < p->d; ++c) acc[c] += pj * orc_bf16_to_f32(v[c]);
        }
        for (int32_t c = 0; c < p->d; ++c) o[c] = orc_f32_to_bf16(acc[c]);
    }
}

int orc_sparse_attn(const orc_attn_problem *p, const int64_t *qsel, int64_t nsel,
                    uint16_t *out, int32_t nthreads)
{
    if (!out || nsel < 0 || check_problem(p, qsel, nsel)) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        float *srow = (float *)malloc(sizeof(float) * (size_t)p->topk);
        float *acc = (float *)malloc(sizeof(float) * (size_t)p->d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < nsel; ++i)
            attn_one_query_f32(p, qsel ? qsel[i] : i, out + i * (int64_t)p->h * p->d, srow, acc);
        free(srow);
        free(acc);
    }
    (void)nthreads;
    return 0;
}

/* f64 twin of the same definition, unrounded output; tests only */
static void attn_one_query_f64(const orc_attn_problem *p, int64_t qi, double *out,
                               double *srow, double *acc)
{
    const int64_t seq = qi / p->s, t = qi % p->s;
    const int32_t *idx = p->idx + seq * p->idx_seq_stride + t * p->topk;
    const uint16_t *kv = p->kv + seq * p->kv_seq_stride;
    for (int32_t hh = 0; hh < p->h; ++hh) {
        const uint16_t *q = p->q + seq * p->q_seq_stride + (t * p->h + hh) * (int64_t)p->d;
        double m = p->sink[hh];
        int any = 0;
        for (int32_t j = 0; j < p->topk; ++j) {
            if (idx[j] < 0) continue;
            const uint16_t *k = kv + (int64_t)idx[j] * p->d;
            double dot = 0.0;
            for (int32_t c = 0; c < p->d; ++c)
                dot += (double)orc_bf16_to_f32(q[c]) * (double)orc_bf16_to_f32(k[c]);
            srow[j] = (double)p->scale * dot;
            if (srow[j] > m) m = srow[j];
            any = 1;
        }
        double *o = out + (int64_t)hh * p->d;
        for (int32_t c = 0; c < p->d; ++c) o[c] = 0.0;
        if (!any) continue;
        double l = exp((double)p->sink[hh] - m);
        for (int32_t j = 0; j < p->topk; ++j)
            if (idx[j] >= 0) l += exp(srow[j] - m);
        for (int32_t c = 0; c < p->d; ++c) acc[c] = 0.0;
        for (int32_t j = 0; j < p->topk; ++j) {
            if (idx[j] < 0) continue;
            double pj = exp(srow[j] - m) / l;
            const uint16_t *v = kv + (int64_t)idx[j] * p->d;
            for (int32_t c = 0; c < p->d; ++c) acc[c] += pj * (double)orc_bf16_to_f32(v[c]);
        }
        for (int32_t c = 0; c < p->d; ++c) o[c] = acc[c];
    }
}

int orc_sparse_attn_f64(const orc_attn_problem *p, const int64_t *qsel, int64_t nsel,
                        double *out, int32_t nthreads)
{
    if (!out || nsel < 0 || check_problem(p, qsel, nsel)) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)p->topk);
        double *acc = (double *)malloc(sizeof(double) * (size_t)p->d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < nsel; ++i)
            attn_one_query_f64(p, qsel ? qsel[i] : i, out + i * (int64_t)p->h * p->d, srow, acc);
        free(srow);
        free(acc);
    }
    (void)nthreads;
    return 0;
}

int orc_sparse_attn_weights_f64(const orc_attn_problem *p, int64_t query, int32_t head,
                                double *w, double *sink_share)
{
    if (!w || !sink_share || check_problem(p, &query, 1) || head < 0 || head >= p->h) return -1;
    const int64_t seq = query / p->s, t = query % p->s;
    const int32_t *idx = p->idx + seq * p->idx_seq_stride + t * p->topk;
    const uint16_t *kv = p->kv + seq * p->kv_seq_stride;
    const uint16_t *q = p->q + seq * p->q_seq_stride + (t * p->h + head) * (int64_t)p->d;
    double m = p->sink[head];
    for (int32_t j = 0; j < p->topk; ++j) {
        w[j] = 0.0;
        if (idx[j] < 0) continue;
        const uint16_t *k = kv + (int64_t)idx[j] * p->d;
        double dot = 0.0;
        for (int32_t c = 0; c < p->d; ++c)
            dot += (double)orc_bf16_to_f32(q[c]) * (double)orc_bf16_to_f32(k[c]);
        w[j] = (double)p->scale * dot;
        if (w[j] > m) m = w[j];
    }
    double l = exp((double)p->sink[head] - m);
    for (int32_t j = 0; j < p->topk; ++j)
        if (idx[j] >= 0) l += exp(w[j] - m);
    for (int32_t j = 0; j < p->topk; ++j)
        w[j] = idx[j] >= 0 ? exp(w[j] - m) / l : 0.0;
    *sink_share = exp((double)p->sink[head] - m) / l;
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Rotary table. [attn-fwd] precompute_freqs_cis: freq_i = 1 / base^(2i/rd) for pair i,  */
/* angle = pos * freq_i, entry = (cos, sin) of the angle, everything in f32 as the page's */
/* torch code computes it (one rounding per operation, no fused multiply-add). With      */
/* original_seq_len > 0, the YaRN correction of the same function: corrected_dim(r) is   */
/* the pair index whose wavelength fits r times into original_seq_len; pairs below       */
/* low = max(floor(corrected_dim(beta_fast)), 0) keep their frequency, pairs above        */
/* high = min(ceil(corrected_dim(beta_slow)), rd - 1) are divided by factor, and a linear */
/* ramp blends the two in between. The band limits are computed in f64 (the page uses    */
/* Python's math module for them), the rest in f32. [attn-docs] freqs_cis names the      */
/* no-YaRN form (original_seq_len = 0) for the ratio-0 layers.                            */
/* ------------------------------------------------------------------------------------ */
static double yarn_corrected_dim(int32_t rd, int32_t original_seq_len, double rotations,
                                 double base)
{
    const double pi = 3.14159265358979323846;
    return rd * log((double)original_seq_len / (rotations * 2.0 * pi)) / (2.0 * log(base));
}

int orc_freqs_cis_yarn(int32_t rd, int32_t max_pos, int32_t original_seq_len, float base,
                       float factor, float beta_fast, float beta_slow, float *cos_sin)
{
    if (rd < 2 || rd % 2 || max_pos < 1 || !cos_sin || !(base > 0.0f)) return -1;
    const int32_t half = rd / 2;
    float *freq = (float *)malloc(sizeof(float) * (size_t)half);
    if (!freq) return -1;
    for (int32_t i = 0; i < half; ++i)
        freq[i] = 1.0f / powf(base, (float)(2 * i) / (float)rd);
    if (original_seq_len > 0) {
        double lo = floor(yarn_corrected_dim(rd, original_seq_len, beta_fast, base));
        double hi = ceil(yarn_corrected_dim(rd, original_seq_len, beta_slow, base));
        int32_t low = lo > 0.0 ? (int32_t)lo : 0;
        int32_t high = hi < (double)(rd - 1) ? (int32_t)hi : rd - 1;
        float span = high - low > 0 ? (float)(high - low) : 1e-3f;   /* max(high - low, 1e-3) */
        for (int32_t i = 0; i < half; ++i) {
            float ramp = ((float)i - (float)low) / span;
            if (ramp < 0.0f) ramp = 0.0f;
            if (ramp > 1.0f) ramp = 1.0f;
            float smooth = 1.0f - ramp;
            float scaled = freq[i] / factor * (1.0f - smooth);
            float kept = freq[i] * smooth;
            freq[i] = scaled + kept;
        }
    }
    for (int32_t pos = 0; pos < max_pos; ++pos)
        for (int32_t i = 0; i < half; ++i) {
            float ang = (float)pos * freq[i];
            cos_sin[((int64_t)pos * half + i) * 2 + 0] = cosf(ang);
            cos_sin[((int64_t)pos * half + i) * 2 + 1] = sinf(ang);
        }
    free(freq);
    return 0;
}

void orc_freqs_cis(int32_t rd, int32_t max_pos, float base, float *cos_sin)
{
    orc_freqs_cis_yarn(rd, max_pos, 0, base, 1.0f, 32.0f, 1.0f, cos_sin);
}

/* ------------------------------------------------------------------------------------ */
/* Rotary. [attn-fwd] apply_rotary_emb: adjacent element pairs (x0, x1) are the complex  */
/* number x0 + i x1, multiplied in f32 by freqs_cis[pos] (its conjugate when inverse)    */
/* and written back into the bf16 tensor. [attn-fwd] Attention.forward applies the       */
/* inverse to the last rope_head_dim elements of sparse_attn's output.                   */
/*   forward: (a, b) -> (a c - b s, a s + b c);  inverse: (a, b) -> (a c + b s, b c - a s) */
/* ------------------------------------------------------------------------------------ */
int orc_apply_rotary(uint16_t *x, int64_t n, int32_t h, int32_t d, int32_t rd,
                     const float *cos_sin, int32_t max_pos, const int32_t *pos, int32_t inverse)
{
    if (!x || n < 0 || h <= 0 || d <= 0 || rd < 0 || rd > d || rd % 2) return -1;
    if (rd == 0) return 0;
    if (!cos_sin || !pos) return -1;
    const int32_t half = rd / 2;
    for (int64_t r = 0; r < n; ++r) {
        if (pos[r] < 0 || pos[r] >= max_pos) return -1;
        for (int32_t hh = 0; hh < h; ++hh) {
            uint16_t *row = x + (r * h + hh) * (int64_t)d + (d - rd);
            for (int32_t i = 0; i < half; ++i) {
                float c = cos_sin[((int64_t)pos[r] * half + i) * 2 + 0];
                float s = cos_sin[((int64_t)pos[r] * half + i) * 2 + 1];
                if (inverse) s = -s;                     /* conjugate */
                float a = orc_bf16_to_f32(row[2 * i]);
                float b = orc_bf16_to_f32(row[2 * i + 1]);
                float re = a * c - b * s;
                float im = a * s + b * c;
                row[2 * i] = orc_f32_to_bf16(re);
                row[2 * i + 1] = orc_f32_to_bf16(im);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* KV write path. [attn-docs] module notes: each token's latent KV row (after wkv and    */
/* kv_norm) gets RoPE on its last rope_dim elements, is quantised to fp8 in place (block  */
/* 32, ue8m0) and goes into the sliding-window ring cache; [attn-fwd] Attention.forward  */
/* rotates with freqs_cis[start_pos + t] (apply_rotary_emb, forward); [attn-docs] ring-   */
/* cache paragraph: the slot of token p is p mod window. The steps, in that order, on a  */
/* normalised row x: forward rotation (orc_apply_rotary), fp8 round trip                 */
/* (orc_act_quant_rows), store.                                                          */
/* Readings: rows of one call that share a slot are stored last-wins, i.e. only the last */
/* `window` rows of a sequence are stored (the prefill writes tokens S-window..S-1); with */
/* window == 0 row t goes to cache row row0[n] + t (a linear cache, e.g. the compressed  */
/* one). A position outside [0, max_pos) or a destination outside the cache stores      */
/* nothing. fp8 storage keeps the codes and scale bytes instead of the bf16 round trip.  */
/* ------------------------------------------------------------------------------------ */
int orc_kv_write(const uint16_t *x, int32_t b, int32_t s, int32_t d, int32_t rd,
                 const float *cos_sin, int32_t max_pos, const int32_t *pos, int32_t window,
                 const int32_t *row0, int32_t cache_rows, uint16_t *cache_bf16,
                 uint8_t *cache_codes, uint8_t *cache_scales, uint16_t *rows_out)
{
    if (!x || !pos || b < 1 || s < 1 || d < 32 || d % 32 || rd < 0 || rd > d || rd % 2) return -1;
    if (window < 0 || (window == 0 && !row0) || cache_rows < 1) return -1;
    if (rd > 0 && !cos_sin) return -1;
    const int nb = d / 32;
    uint16_t *row = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *rt = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint8_t *codes = (uint8_t *)malloc((size_t)d);
    uint8_t *scales = (uint8_t *)malloc((size_t)nb);
    if (!row || !rt || !codes || !scales) { free(row); free(rt); free(codes); free(scales); return -1; }
    for (int32_t n = 0; n < b; ++n)
        for (int32_t t = 0; t < s; ++t) {
            const int64_t i = (int64_t)n * s + t;
            const int32_t p = pos[i];
            if (p < 0 || p >= max_pos) continue;
            memcpy(row, x + i * d, sizeof(uint16_t) * (size_t)d);
            if (rd > 0) orc_apply_rotary(row, 1, 1, d, rd, cos_sin, max_pos, &p, 0);
            orc_act_quant_rows(row, 1, d, rt, codes, scales);
            if (rows_out) memcpy(rows_out + i * d, rt, sizeof(uint16_t) * (size_t)d);
            int64_t dst;
            if (window > 0) {
                if (t < s - window) continue;                 /* a later row takes the slot */
                dst = p % window;
            } else {
                dst = (int64_t)row0[n] + t;
            }
            if (dst < 0 || dst >= cache_rows) continue;
            const int64_t r = (int64_t)n * cache_rows + dst;
            if (cache_bf16) memcpy(cache_bf16 + r * d, rt, sizeof(uint16_t) * (size_t)d);
            if (cache_codes) memcpy(cache_codes + r * d, codes, (size_t)d);
            if (cache_scales) memcpy(cache_scales + r * nb, scales, (size_t)nb);
        }
    free(row); free(rt); free(codes); free(scales);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Indexer scores. [indexer] Indexer.forward: index_score = einsum(q, index_k) over the   */
/* index head dim, rectified, times the per-head weights (the caller's weights_proj      */
/* output already times softmax_scale * n_heads^-0.5), summed over heads; positions a   */
/* query cannot see are -inf. A query at absolute position p sees the first (p+1)/ratio  */
/* compressed positions ("a block becomes visible once the query has passed its last    */
/* token": (t+1)//ratio in prefill, end_pos//ratio in decode). With a candidate mask     */
/* (the second level of select_candidate_blocks' two-level top-k) non-candidates are -inf */
/* too.                                                                                   */
/* Reading: the scores are kept in f32 (the page's torch code rounds the einsum, the      */
/* product and the head sum to bf16); the sums run in index order.                        */
/* ------------------------------------------------------------------------------------ */
static int64_t visible_positions(int32_t pos, int32_t ratio, int32_t n_pos)
{
    if (pos < 0) return 0;
    int64_t v = ((int64_t)pos + 1) / ratio;
    return v < n_pos ? v : n_pos;
}

int orc_index_scores(const uint16_t *q, const uint16_t *k, const float *w, const int32_t *pos,
                     const uint8_t *cand, int32_t b, int32_t s, int32_t h, int32_t d,
                     int32_t n_pos, int32_t ratio, float *scores, int32_t nthreads)
{
    if (!q || !k || !w || !pos || !scores || b < 1 || s < 1 || h < 1 || d < 1 || n_pos < 1 || ratio < 1)
        return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t qi = 0; qi < (int64_t)b * s; ++qi) {
        const int64_t n = qi / s;
        const int64_t vis = visible_positions(pos[qi], ratio, n_pos);
        float *row = scores + qi * n_pos;
        for (int32_t t = 0; t < n_pos; ++t) {
            if (t >= vis || (cand && !cand[qi * n_pos + t])) { row[t] = -INFINITY; continue; }
            const uint16_t *kt = k + (n * n_pos + t) * (int64_t)d;
            float acc = 0.0f;
            for (int32_t hh = 0; hh < h; ++hh) {
                const uint16_t *qh = q + (qi * h + hh) * (int64_t)d;
                float dot = 0.0f;
                for (int32_t c = 0; c < d; ++c) dot += orc_bf16_to_f32(qh[c]) * orc_bf16_to_f32(kt[c]);
                const float r = dot > 0.0f ? dot : 0.0f;                 /* relu */
                acc += r * w[qi * h + hh];
            }
            row[t] = acc;
        }
    }
    (void)nthreads;
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Indexer top-k. [indexer] Indexer.forward, last lines: take the `topk` best positions   */
/* by score, re-sort them into position order, shift them by `offset`, and mark as -1    */
/* what the query cannot reach.                                                          */
/* Readings: the pages leave ties open; equal scores go to the lower position first.     */
/* Only positions with a finite score are ever listed (the page's where() also lists a   */
/* reachable -inf pick, which a candidate mask can leave; it never arises with the       */
/* config's 2048 candidate blocks); the list is then padded with -1.                     */
/* ------------------------------------------------------------------------------------ */
typedef struct { float v; int32_t t; } scored_pos;

static int by_score_then_position(const void *a, const void *b)
{
    const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int by_position(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int orc_index_topk(const float *scores, int32_t b, int32_t s, int32_t n_pos, int32_t topk,
                   int32_t offset, int32_t *idx)
{
    if (!scores || !idx || b < 1 || s < 1 || n_pos < 1 || topk < 1) return -1;
    scored_pos *buf = (scored_pos *)malloc(sizeof(scored_pos) * (size_t)n_pos);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)topk);
    if (!buf || !sel) { free(buf); free(sel); return -1; }
    for (int64_t qi = 0; qi < (int64_t)b * s; ++qi) {
        const float *row = scores + qi * n_pos;
        int32_t nf = 0;
        for (int32_t t = 0; t < n_pos; ++t)
            if (row[t] > -INFINITY) { buf[nf].v = row[t]; buf[nf].t = t; ++nf; }
        qsort(buf, (size_t)nf, sizeof(scored_pos), by_score_then_position);
        const int32_t m = nf < topk ? nf : topk;
        for (int32_t j = 0; j < m; ++j) sel[j] = buf[j].t;
        qsort(sel, (size_t)m, sizeof(int32_t), by_position);
        int32_t *out = idx + qi * topk;
        for (int32_t j = 0; j < topk; ++j) out[j] = j < m ? sel[j] + offset : -1;
    }
    free(buf);
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Candidate blocks. [indexer] select_candidate_blocks, level one of the two-level top-k: */
/* a block of block_size positions scores the maximum of its logits (the last block      */
/* padded with -inf); the block holding the query's newest visible position,             */
/* (compress_len - 1) // block_size with floor division, is pinned to +inf; the          */
/* min(topk_blocks, num_blocks) best blocks are taken and those whose score is above     */
/* -inf are kept; the mask repeats each block's flag over its positions.                 */
/* compress_len = (pos + 1) / ratio as in orc_index_scores.                               */
/* Reading: ties between equal block scores go to the lower block first.                 */
/* ------------------------------------------------------------------------------------ */
int orc_candidate_blocks(const float *logits, const int32_t *pos, int32_t b, int32_t s,
                         int32_t n_pos, int32_t ratio, int32_t topk_blocks, int32_t block_size,
                         uint8_t *mask)
{
    if (!logits || !pos || !mask || b < 1 || s < 1 || n_pos < 1 || ratio < 1 || topk_blocks < 1 ||
        block_size < 1)
        return -1;
    const int32_t nblk = (n_pos + block_size - 1) / block_size;
    scored_pos *blk = (scored_pos *)malloc(sizeof(scored_pos) * (size_t)nblk);
    uint8_t *keep = (uint8_t *)malloc((size_t)nblk);
    if (!blk || !keep) { free(blk); free(keep); return -1; }
    for (int64_t qi = 0; qi < (int64_t)b * s; ++qi) {
        const float *row = logits + qi * n_pos;
        const int64_t len = pos[qi] < 0 ? 0 : ((int64_t)pos[qi] + 1) / ratio;
        /* floor division: len = 0 pins block -1, i.e. none */
        const int64_t last = len > 0 ? (len - 1) / block_size : -1;
        for (int32_t j = 0; j < nblk; ++j) {
            float m = -INFINITY;
            for (int32_t u = 0; u < block_size; ++u) {
                const int64_t t = (int64_t)j * block_size + u;
                const float v = t < n_pos ? row[t] : -INFINITY;     /* -inf padding */
                if (v > m) m = v;
            }
            blk[j].v = j == last ? INFINITY : m;
            blk[j].t = j;
            keep[j] = 0;
        }
        qsort(blk, (size_t)nblk, sizeof(scored_pos), by_score_then_position);
        const int32_t m = topk_blocks < nblk ? topk_blocks : nblk;
        for (int32_t j = 0; j < m; ++j)
            if (blk[j].v > -INFINITY) keep[blk[j].t] = 1;
        for (int32_t t = 0; t < n_pos; ++t) mask[qi * n_pos + t] = keep[t / block_size];
    }
    free(blk);
    free(keep);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Grouped output projection. [attn-fwd] Attention.forward: the attention output is      */
/* viewed as [tokens][groups][heads_per_group * head_dim] and multiplied, group by group, */
/* with wo_a viewed as [groups][o_lora_rank][heads_per_group * head_dim] (einsum          */
/* "bsgd,grd->bsgr"; wo_a is block-diagonal over groups). [attn-docs] precision           */
/* paragraph: a bf16 GEMM, f32 accumulation, bf16 result (round to nearest even).        */
/* o: bf16 rows of m tokens, token stride o_stride (elements) >= g * kg; w: bf16          */
/* [g][r][kg]; out: bf16 [m][g][r].                                                       */
/* ------------------------------------------------------------------------------------ */
int orc_grouped_proj(const uint16_t *o, int64_t o_stride, const uint16_t *w, int32_t m,
                     int32_t g, int32_t r, int32_t kg, uint16_t *out, int32_t nthreads)
{
    if (!o || !w || !out || m < 1 || g < 1 || r < 1 || kg < 1 || o_stride < (int64_t)g * kg) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t t = 0; t < m; ++t)
        for (int32_t gg = 0; gg < g; ++gg) {
            const uint16_t *a = o + t * o_stride + (int64_t)gg * kg;
            for (int32_t rr = 0; rr < r; ++rr) {
                const uint16_t *wr = w + ((int64_t)gg * r + rr) * kg;
                float acc = 0.0f;
                for (int32_t k = 0; k < kg; ++k) acc += orc_bf16_to_f32(a[k]) * orc_bf16_to_f32(wr[k]);
                out[(t * g + gg) * (int64_t)r + rr] = orc_f32_to_bf16(acc);
            }
        }
    (void)nthreads;
    return 0;
}
