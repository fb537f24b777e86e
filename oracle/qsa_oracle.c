/*
 * qsa_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, obviously correct CPU reference for the QSA block-score
 * select phase.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header or table with the
 * HIP library: it decodes fp16 itself, sums in float64 in plain index order
 * and sorts with the C library's qsort.
 *
 * What it computes (Strata pull request #228, part 1 "qsa_block_scores_wmma:
 * the prompt scorer arm on tensor cores", the score formula in its first
 * paragraph; restated in Strata pull request #856):
 *
 *   score(t, b) = sum over query heads h of relu( sum over channels i of
 *                 k_b[i] * q_{t,h}[i] )
 *
 * for every query t of a KV head g and every KV block b, where the H query
 * heads of KV head g share the block key k_b.  The arithmetic contract (the
 * same page, "arithmetic contract" paragraph; PR #856 "Arithmetic contract and
 * parity") bounds each fp16/fp32 result by
 *
 *   B(t, b) = 2^-9.5 * S(t, b) + 8 * 2^-24 * |score_ref(t, b)|,
 *   S(t, b) = sum_h sum_i |k_b[i] * q_{t,h}[i]|   (float64),
 *
 * and the phase then keeps, per query, the top-k blocks ("selection/topk",
 * PR #228 part 1, the paragraph after the bench table).
 *
 * Every product of two fp16 values (22 significant bits) or of an fp32 and an
 * fp16 value (35 bits) is exact in float64, so the only rounding here is the
 * float64 summation, about D * 2^-53 * S: negligible against B.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

/* Threads an OpenMP region of the oracle uses (for reporting). */
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* Sets the threads of the following OpenMP regions (the benchmark's
 * single-thread baseline); n < 1 is ignored. */
void oracle_set_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

/* IEEE 754 binary16 -> exact double, from the format's definition:
 * sign s, 5-bit biased exponent e, 10-bit fraction m.
 *   e == 0        : (-1)^s * m * 2^-24            (zero and subnormals)
 *   0 < e < 31    : (-1)^s * (1024 + m) * 2^(e-25)
 *   e == 31       : infinity (m == 0) or NaN       */
double oracle_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* fp32 -> fp16 bits, round to nearest, ties to even, written from the
 * definition rather than bit tricks:
 *  - NaN keeps its sign and the top 10 fraction bits and is made quiet;
 *  - |x| >= 65520 (halfway between 65504 and 2^16) overflows to infinity;
 *  - below 2^-14 the fp16 grid spacing is 2^-24 (subnormals);
 *  - otherwise the spacing is 2^(E-10) with E = floor(log2 |x|).
 * The quotient |x| / spacing is exact in double, and rint() rounds it to
 * the nearest integer with ties to even (the default rounding mode). */
uint16_t oracle_f32_to_f16_one(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u)                      /* NaN */
        return (uint16_t)(sign | 0x7c00u | 0x0200u | ((mag >> 13) & 0x3ffu));
    if (mag == 0x7f800000u)                     /* infinity */
        return (uint16_t)(sign | 0x7c00u);
    double a = fabs((double)x);
    if (a < ldexp(1.0, -14)) {
        double q = rint(a / ldexp(1.0, -24));   /* 0 .. 1024 */
        return (uint16_t)(sign | (uint16_t)q);  /* 1024 encodes 2^-14 */
    }
    int E;
    frexp(a, &E);                                /* a = f * 2^E, f in [0.5,1) */
    E -= 1;                                      /* a in [2^E, 2^(E+1)) */
    double q = rint(ldexp(a, 10 - E));           /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

void oracle_convert_f32_f16(const float *src, uint16_t *dst, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_f32_to_f16_one(src[i]);
}

/* Row r of a request is (g, t) = (rows[r] / nq, rows[r] % nq); a NULL row
 * list means every row r = g*nq + t in order.
 *
 * q layout:  element (t, g, h, i) at q[t*q_tok_stride + (g*H + h)*D + i],
 *            fp16 bits if q_is_f32 == 0, else float32 values.
 * k layout:  element (g, b, i) at kblk[g*k_head_stride + b*D + i], fp16 bits.
 * outputs:   score/S/B at [r*ld_out + b] for b in [0, nb); any may be NULL.
 *
 * score_ref = sum_h relu(d_h), d_h = sum_i k[i]*q_h[i]; h and i ascending. */
int oracle_scores(const void *q, int q_is_f32, int64_t q_tok_stride,
                  const uint16_t *kblk, int64_t k_head_stride,
                  int32_t G, int32_t nq, int32_t H, int32_t D, int64_t nb,
                  const int64_t *rows, int64_t n_rows,
                  double *score, double *S, double *B, int64_t ld_out)
{
    if (G < 0 || nq < 0 || H < 1 || D < 1 || nb < 0 || ld_out < nb)
        return 1;
    if (rows == NULL)
        n_rows = (int64_t)G * nq;
    const uint16_t *q16 = (const uint16_t *)q;
    const float *q32 = (const float *)q;
    const double bound_rel = ldexp(1.0, -9) / sqrt(2.0);   /* 2^-9.5 */
    const double bound_abs = 8.0 * ldexp(1.0, -24);

#pragma omp parallel
    {
        double *qrow = (double *)malloc(sizeof(double) * (size_t)H * (size_t)D);
        double *krow = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t rid = rows ? rows[r] : r;
            int64_t g = rid / nq, t = rid % nq;
            for (int32_t h = 0; h < H; ++h)
                for (int32_t i = 0; i < D; ++i) {
                    int64_t off = t * q_tok_stride + ((int64_t)g * H + h) * D + i;
                    qrow[(size_t)h * D + i] =
                        q_is_f32 ? (double)q32[off] : oracle_f16_to_f64(q16[off]);
                }
            for (int64_t b = 0; b < nb; ++b) {
                for (int32_t i = 0; i < D; ++i)
                    krow[i] = oracle_f16_to_f64(kblk[g * k_head_stride + b * D + i]);
                double sc = 0.0, sabs = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    double d = 0.0;
                    for (int32_t i = 0; i < D; ++i) {
                        double p = krow[i] * qrow[(size_t)h * D + i];
                        d += p;
                        sabs += fabs(p);
                    }
                    sc += (d > 0.0) ? d : 0.0;
                }
                if (score) score[r * ld_out + b] = sc;
                if (S) S[r * ld_out + b] = sabs;
                if (B) B[r * ld_out + b] = bound_rel * sabs + bound_abs * fabs(sc);
            }
        }
        free(qrow);
        free(krow);
    }
    return 0;
}

/* The fixed-order single-precision model of one block's scores, used to pin
 * the separate tail-block kernel bit for bit.  The pages state that the
 * partial last block is scored by its own shared kernel whose result is
 * bitwise reproducible (PR #228 part 1, the paragraph naming the tail
 * kernel; PR #856 "What").  The order fixed here:
 *   acc_h = +0; for i ascending: acc_h = fmaf(k[i], q_h[i], acc_h)
 *   r_h   = acc_h > 0 ? acc_h : +0
 *   s     = +0; for h ascending: s = s + r_h
 * Operands are fp16 bits (for fp32 queries: the fp16 values the conversion
 * produced).  out[r] for the same row convention as oracle_scores. */
int oracle_block_model_f32(const uint16_t *q16, int64_t q_tok_stride,
                           const uint16_t *kblk, int64_t k_head_stride,
                           int32_t G, int32_t nq, int32_t H, int32_t D, int64_t b,
                           const int64_t *rows, int64_t n_rows, float *out)
{
    if (G < 0 || nq < 0 || H < 1 || D < 1 || b < 0)
        return 1;
    if (rows == NULL)
        n_rows = (int64_t)G * nq;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t rid = rows ? rows[r] : r;
        int64_t g = rid / nq, t = rid % nq;
        float s = 0.0f;
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t i = 0; i < D; ++i) {
                float kv = (float)oracle_f16_to_f64(kblk[g * k_head_stride + b * D + i]);
                float qv = (float)oracle_f16_to_f64(
                    q16[t * q_tok_stride + ((int64_t)g * H + h) * D + i]);
                acc = fmaf(kv, qv, acc);
            }
            float rh = (acc > 0.0f) ? acc : 0.0f;
            s = s + rh;
        }
        out[r] = s;
    }
    return 0;
}

/* Top-k over a score row: blocks ordered by score descending, ties by block
 * id ascending; scores compare numerically (so -0 == +0) and a NaN ranks
 * below every number.  The first min(k, nb) ids are written, then -1 up to
 * k; vals (nullable) gets the selected scores and -inf in padded slots. */
typedef struct {
    double s;
    int64_t id;
} oracle_entry;

static int oracle_cmp(const void *pa, const void *pb)
{
    const oracle_entry *a = (const oracle_entry *)pa, *b = (const oracle_entry *)pb;
    int na = isnan(a->s), nb = isnan(b->s);
    if (na != nb)
        return na ? 1 : -1;                 /* NaN after every number */
    if (!na && a->s != b->s)
        return (a->s > b->s) ? -1 : 1;      /* larger score first */
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

int oracle_topk(const double *scores, int64_t ld, int64_t rows, int64_t nb, int32_t k,
                int32_t *ids, int64_t ld_ids, double *vals)
{
    if (rows < 0 || nb < 0 || k < 0 || ld < nb || ld_ids < k)
        return 1;
#pragma omp parallel
    {
        oracle_entry *e = (oracle_entry *)malloc(sizeof(oracle_entry) * (size_t)(nb > 0 ? nb : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t b = 0; b < nb; ++b) {
                e[b].s = scores[r * ld + b];
                e[b].id = b;
            }
            qsort(e, (size_t)nb, sizeof(oracle_entry), oracle_cmp);
            for (int32_t j = 0; j < k; ++j) {
                int sel = j < nb;
                ids[r * ld_ids + j] = sel ? (int32_t)e[j].id : -1;
                if (vals) vals[r * ld_ids + j] = sel ? e[j].s : -INFINITY;
            }
        }
        free(e);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Block keys (the step before the phase).  The pages index one key vector
 * k_b per KV block (PR #228 part 1, score formula) without saying how it is
 * built from the block's token keys.  The reading taken: the mean of the
 * block's token keys, per KV head and channel, rounded once to the nearest
 * fp16 (ties to even): the partial last block averages its own tokens.
 *
 * Written from the definition with exact integer arithmetic: every fp16
 * value is an integer m times 2^-24 (|m| < 2^40), so a block's sum is an
 * exact integer N (|N| < 2^53 for up to 2^13 tokens) and its mean is the
 * rational N / len.  The fp16 result is the value of the fp16 grid nearest
 * to it, found by trying exponents from the largest down. */
static int64_t oracle_f16_units(uint16_t h)   /* value * 2^24, finite input */
{
    int e = (h >> 10) & 0x1f;
    int64_t m = h & 0x3ff;
    int64_t v = (e == 0) ? m : ((1024 + m) << (e - 1));
    return (h & 0x8000) ? -v : v;
}

/* nearest fp16 (ties to even) to num / den * 2^-24, den > 0 */
uint16_t oracle_round_ratio_f16(int64_t num, int64_t den)
{
    uint16_t sign = num < 0 ? 0x8000u : 0;
    unsigned __int128 a = (unsigned __int128)(num < 0 ? -num : num);
    if (a == 0)
        return 0;   /* an exact zero mean is +0 */
    /* the fp16 binade [2^E, 2^(E+1)) holding the value, E in [-14, 15];
     * below 2^-14 the grid is the subnormal one (spacing 2^-24) */
    int E = 15;
    while (E > -14 && a < ((unsigned __int128)den << (E + 24)))
        --E;
    int spacing_log2 = (E == -14 && a < ((unsigned __int128)den << 10)) ? 0 : E + 14;
    unsigned __int128 unit = (unsigned __int128)den << spacing_log2;
    unsigned __int128 q = a / unit, r = a % unit;
    if (2 * r > unit || (2 * r == unit && (q & 1)))
        ++q;
    if (spacing_log2 == 0 && E == -14 && q <= 1024)   /* subnormal (1024 = 2^-14) */
        return (uint16_t)(sign | (uint16_t)q);
    if (q == 2048) {   /* rounded up into the next binade */
        q = 1024;
        ++E;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024));
}

/* kblk[g*head_stride + b*D + i] = nearest fp16 to the mean of
 * k_tok[t*tok_stride + g*D + i] over the tokens t of block b
 * (t in [b*bs, min((b+1)*bs, n_kv))), for every g < G, b < nb, i < D. */
int oracle_block_keys(const uint16_t *k_tok, int64_t tok_stride, int32_t G, int32_t D,
                      int64_t n_kv, int32_t bs, uint16_t *kblk, int64_t head_stride)
{
    if (G < 0 || D < 1 || n_kv < 0 || bs < 1 || bs > 8192 || tok_stride < (int64_t)G * D ||
        head_stride < ((n_kv + bs - 1) / bs) * D)
        return 1;
    int64_t nb = (n_kv + bs - 1) / bs;
#pragma omp parallel for schedule(static)
    for (int64_t gb = 0; gb < (int64_t)G * nb; ++gb) {
        int64_t g = gb / nb, b = gb % nb;
        int64_t t0 = b * bs, t1 = t0 + bs < n_kv ? t0 + bs : n_kv;
        for (int32_t i = 0; i < D; ++i) {
            int64_t sum = 0;
            for (int64_t t = t0; t < t1; ++t)
                sum += oracle_f16_units(k_tok[t * tok_stride + g * D + i]);
            kblk[g * head_stride + b * D + i] = oracle_round_ratio_f16(sum, t1 - t0);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Attention over the selected blocks (the step after the phase).  The pages
 * stop at the selection; the reading taken for the step that consumes it is
 * plain softmax attention of every query head over the tokens of the blocks
 * its (KV head, query) row selected:
 *   s_j   = scale * sum_i q[t][g][h][i] * k[j][g][i],  scale = fp32(1/sqrt(D))
 *   out   = sum_j exp(s_j - max s) v[j][g][:] / sum_j exp(s_j - max s)
 * over every token j of every listed block (ids < 0 are empty slots; a row
 * with no token gives 0).  Computed in float64 in plain order.
 *
 * Bound of a device result computed in fp32 with fp16 inputs (per output
 * element, float64), for a device that sums each logit's D exact products
 * in one fp32 chain, scales once, takes exp in fp32, and sums P*V and P per
 * chunk of at most 64 tokens before adding the chunk into a running sum
 * rescaled when the maximum grows:
 *   delta = max_j ( scale*D*u*sum_i|q_i k_ji| + 2u*|s_j| + 4u*(1 + |s_j - max s|) )
 *   E     = 2*delta + (2*(64 + C) + 16*C + 32)*u,   C = number of 64-token chunks
 *   B     = E * (sum_j p_j |v_j| / sum_j p_j) + 2u*|out|,   u = 2^-24
 * (logit errors move each weight by at most delta relatively, in the
 * numerator and the denominator; each fp32 sum is a chain of at most
 * 64 + C additions; each rescale and exp costs a few more roundings).
 *
 * The device may also take P*V from two fp16 parts of each weight scaled by
 * 2^14 (hi = fp16(p*2^14), lo = fp16(p*2^14 - hi)), each part times v exact
 * in fp32, the two parts summed in chains of their own and added once at
 * the end.  That adds to E the split's 2^-22 = 4u (relative), the lo chain's
 * (64 + C)u on sums 2^-11 as large, and the final addition's u:
 *   E    += (5 + (64 + C) / 2048) * u
 * and where a part falls below fp16's normal range its absolute error is at
 * most 2^-25 in units of p*2^14, 2^-39 in units of p, so
 *   B    += 2^-39 * (sum_j |v_j|) / sum_j p_j. */
int oracle_attention(const uint16_t *q16, int64_t q_tok_stride, const uint16_t *k_tok,
                     const uint16_t *v_tok, int64_t kv_tok_stride, const int32_t *ids,
                     int64_t ld_ids, int32_t G, int32_t nq, int32_t H, int32_t D,
                     int64_t n_kv, int32_t bs, int32_t k, double *out, double *bound)
{
    if (G < 0 || nq < 0 || H < 1 || D < 1 || n_kv < 0 || bs < 1 || k < 0 || ld_ids < k)
        return 1;
    const float scale_f = (float)(1.0 / sqrt((double)D));
    const double scale = (double)scale_f;
    const double u = ldexp(1.0, -24);
    const int64_t nb = (n_kv + bs - 1) / bs;
#pragma omp parallel
    {
        int64_t cap = (int64_t)k * bs;
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        double *sabs = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        double *kv = (double *)malloc(sizeof(double) * (size_t)D);
        double *vabs = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < (int64_t)G * nq; ++r) {
            const int64_t g = r / nq, t = r % nq;
            /* the tokens of the listed blocks, block by block */
            int64_t L = 0, chunks = 0;
            for (int32_t slot = 0; slot < k; ++slot) {
                int32_t b = ids[r * ld_ids + slot];
                if (b < 0 || b >= nb)
                    continue;
                int64_t t0 = (int64_t)b * bs, t1 = t0 + bs < n_kv ? t0 + bs : n_kv;
                chunks += (t1 - t0 + 63) / 64;
                for (int64_t j = t0; j < t1; ++j)
                    tok[L++] = j;
            }
            for (int32_t h = 0; h < H; ++h) {
                const uint16_t *qh = q16 + t * q_tok_stride + ((int64_t)g * H + h) * D;
                double *o = out + ((t * G + g) * H + h) * (int64_t)D;
                double *bo = bound + ((t * G + g) * H + h) * (int64_t)D;
                if (L == 0) {
                    for (int32_t i = 0; i < D; ++i)
                        o[i] = bo[i] = 0.0;
                    continue;
                }
                double m = -INFINITY;
                for (int64_t a = 0; a < L; ++a) {
                    const uint16_t *kj = k_tok + tok[a] * kv_tok_stride + g * D;
                    double d = 0.0, da = 0.0;
                    for (int32_t i = 0; i < D; ++i) {
                        double p = oracle_f16_to_f64(qh[i]) * oracle_f16_to_f64(kj[i]);
                        d += p;
                        da += fabs(p);
                    }
                    s[a] = scale * d;
                    sabs[a] = scale * da;
                    if (s[a] > m)
                        m = s[a];
                }
                double den = 0.0, delta = 0.0;
                for (int64_t a = 0; a < L; ++a) {
                    /* sabs already holds scale * sum_i |q_i k_ji| */
                    double e = sabs[a] * D * u + 2.0 * u * fabs(s[a]) + 4.0 * u * (1.0 + fabs(s[a] - m));
                    if (e > delta)
                        delta = e;
                    s[a] = exp(s[a] - m);   /* weight p_a, reusing the logit slot */
                    den += s[a];
                }
                const double E = 2.0 * delta +
                                 (2.0 * (64.0 + (double)chunks) + 16.0 * (double)chunks + 32.0 +
                                  5.0 + (64.0 + (double)chunks) / 2048.0) * u;
                for (int32_t i = 0; i < D; ++i)
                    o[i] = bo[i] = vabs[i] = 0.0;
                for (int64_t a = 0; a < L; ++a) {
                    const uint16_t *vj = v_tok + tok[a] * kv_tok_stride + g * D;
                    for (int32_t i = 0; i < D; ++i)
                        kv[i] = oracle_f16_to_f64(vj[i]);
                    for (int32_t i = 0; i < D; ++i) {
                        o[i] += s[a] * kv[i];
                        bo[i] += s[a] * fabs(kv[i]);
                        vabs[i] += fabs(kv[i]);
                    }
                }
                for (int32_t i = 0; i < D; ++i) {
                    o[i] /= den;
                    bo[i] = E * (bo[i] / den) + ldexp(vabs[i], -39) / den + 2.0 * u * fabs(o[i]);
                }
            }
        }
        free(tok);
        free(s);
        free(sabs);
        free(kv);
        free(vabs);
    }
    return 0;
}
