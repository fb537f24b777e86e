/* Test driver: runs the C oracle (oracle/qsa_oracle.c, linked in) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on small inputs whose
 * results are known in closed form, and over every fp32 pattern class of the
 * conversion.  Built and run by the CPU test suite with
 *   gcc -fsanitize=address,undefined -fno-sanitize-recover=all
 * Exit status 0 means every check passed and no sanitizer fired.
 *
 * Closed forms used (score(t, b) = sum_h relu(sum_i k_b[i] q_{t,h}[i]),
 * Strata pull request #228, part 1, score formula):
 *   - one-hot queries: q_{t,h} = e_{c(t,h)} gives score = sum_h relu(k_b[c(t,h)])
 *     and S = sum_h |k_b[c(t,h)]|;
 *   - integer operands: every product and sum is exact in float64.
 * Strides and row lists are exercised with padding between tokens and
 * between KV heads, so an out-of-bounds read would be reported. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_scores(const void *q, int q_is_f32, int64_t q_tok_stride, const uint16_t *kblk,
                  int64_t k_head_stride, int32_t G, int32_t nq, int32_t H, int32_t D, int64_t nb,
                  const int64_t *rows, int64_t n_rows, double *score, double *S, double *B,
                  int64_t ld_out);
int oracle_block_model_f32(const uint16_t *q16, int64_t q_tok_stride, const uint16_t *kblk,
                           int64_t k_head_stride, int32_t G, int32_t nq, int32_t H, int32_t D,
                           int64_t b, const int64_t *rows, int64_t n_rows, float *out);
int oracle_topk(const double *scores, int64_t ld, int64_t rows, int64_t nb, int32_t k,
                int32_t *ids, int64_t ld_ids, double *vals);
uint16_t oracle_f32_to_f16_one(float x);
void oracle_convert_f32_f16(const float *src, uint16_t *dst, int64_t n);
double oracle_f16_to_f64(uint16_t h);

static int failures = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);               \
            fprintf(stderr, "\n");                      \
            ++failures;                                 \
        }                                               \
    } while (0)

/* small integers as exact fp16 bits (|v| <= 2048) */
static uint16_t int_to_f16(int v)
{
    if (v == 0) return 0;
    uint16_t sign = v < 0 ? 0x8000u : 0;
    unsigned a = (unsigned)(v < 0 ? -v : v);
    int e = 0;
    while ((a >> e) > 1) ++e;                   /* a in [2^e, 2^(e+1)) */
    unsigned frac = (a << (10 - e)) & 0x3ffu;   /* exact for a <= 2048 */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | frac);
}

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static int rnd(int lo, int hi) /* uniform in [lo, hi] */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return lo + (int)(rng_state % (uint64_t)(hi - lo + 1));
}

static void check_one_hot(void)
{
    const int G = 3, nq = 5, H = 4, D = 64, nb = 7, tok_pad = 24, head_pad = 3;
    const int64_t qts = (int64_t)G * H * D + tok_pad;
    const int64_t khs = (int64_t)(nb + head_pad) * D;
    uint16_t *q = calloc((size_t)(nq * qts), sizeof(uint16_t));
    uint16_t *k = calloc((size_t)(G * khs), sizeof(uint16_t));
    int *c = malloc(sizeof(int) * (size_t)(G * nq * H));
    int *kv = malloc(sizeof(int) * (size_t)(G * nb * D));
    for (int g = 0; g < G; ++g)
        for (int t = 0; t < nq; ++t)
            for (int h = 0; h < H; ++h) {
                int ch = rnd(0, D - 1);
                c[(g * nq + t) * H + h] = ch;
                q[t * qts + (g * H + h) * D + ch] = 0x3c00u; /* 1.0 */
            }
    for (int g = 0; g < G; ++g)
        for (int b = 0; b < nb; ++b)
            for (int i = 0; i < D; ++i) {
                int v = rnd(-1000, 1000);
                kv[(g * nb + b) * D + i] = v;
                k[g * khs + b * D + i] = int_to_f16(v);
            }
    /* every other row, in reverse order, through the row list */
    int64_t rows[8];
    int n_rows = 0;
    for (int r = G * nq - 1; r >= 0 && n_rows < 8; r -= 2) rows[n_rows++] = r;
    double *sc = malloc(sizeof(double) * (size_t)(n_rows * nb));
    double *S = malloc(sizeof(double) * (size_t)(n_rows * nb));
    double *B = malloc(sizeof(double) * (size_t)(n_rows * nb));
    CHECK(oracle_scores(q, 0, qts, k, khs, G, nq, H, D, nb, rows, n_rows, sc, S, B, nb) == 0,
          "oracle_scores refused");
    for (int j = 0; j < n_rows; ++j) {
        int g = (int)(rows[j] / nq), t = (int)(rows[j] % nq);
        for (int b = 0; b < nb; ++b) {
            double want = 0, wantS = 0;
            for (int h = 0; h < H; ++h) {
                int v = kv[(g * nb + b) * D + c[(g * nq + t) * H + h]];
                want += v > 0 ? v : 0;
                wantS += v < 0 ? -v : v;
            }
            CHECK(sc[j * nb + b] == want, "one-hot score row %d block %d: %g vs %g", j, b,
                  sc[j * nb + b], want);
            CHECK(S[j * nb + b] == wantS, "one-hot S row %d block %d", j, b);
        }
    }
    /* the fixed-order fp32 model of one block: integer results are exact */
    float *m = malloc(sizeof(float) * (size_t)(G * nq));
    CHECK(oracle_block_model_f32(q, qts, k, khs, G, nq, H, D, nb - 1, NULL, 0, m) == 0,
          "block model refused");
    for (int g = 0; g < G; ++g)
        for (int t = 0; t < nq; ++t) {
            double want = 0;
            for (int h = 0; h < H; ++h) {
                int v = kv[(g * nb + nb - 1) * D + c[(g * nq + t) * H + h]];
                want += v > 0 ? v : 0;
            }
            CHECK((double)m[g * nq + t] == want, "block model g %d t %d", g, t);
        }
    free(m);
    free(sc);
    free(S);
    free(B);
    free(kv);
    free(c);
    free(k);
    free(q);
}

static void check_topk(void)
{
    /* a row with ties, signed zeros, NaN and infinities; k beyond nb pads */
    const double row[9] = {0.5, -0.0, NAN, 3.0, 0.0, INFINITY, 3.0, -INFINITY, 0.5};
    const int want[12] = {5, 3, 6, 0, 8, 1, 4, 7, 2, -1, -1, -1};
    int32_t ids[12];
    double vals[12];
    CHECK(oracle_topk(row, 9, 1, 9, 12, ids, 12, vals) == 0, "topk refused");
    for (int j = 0; j < 12; ++j) CHECK(ids[j] == want[j], "topk slot %d: %d vs %d", j, ids[j], want[j]);
    CHECK(isinf(vals[11]) && vals[11] < 0, "pad value");
    /* empty rows */
    int32_t e[4];
    CHECK(oracle_topk(row, 0, 1, 0, 4, e, 4, NULL) == 0 && e[0] == -1 && e[3] == -1, "empty row");
}

static void check_convert(void)
{
    /* one pattern per exponent and sign with fraction bits around the
     * rounding points; the result must decode back to the nearest fp16 */
    float src[2 * 256 * 6];
    int n = 0;
    const uint32_t fr[6] = {0, 1, 0xfff, 0x1000, 0x1001, 0x7fffff};
    for (uint32_t s = 0; s < 2; ++s)
        for (uint32_t e = 0; e < 256; ++e)
            for (int j = 0; j < 6; ++j) {
                uint32_t u = (s << 31) | (e << 23) | fr[j];
                memcpy(&src[n++], &u, 4);
            }
    uint16_t dst[2 * 256 * 6];
    oracle_convert_f32_f16(src, dst, n);
    for (int i = 0; i < n; ++i) {
        CHECK(dst[i] == oracle_f32_to_f16_one(src[i]), "convert %d", i);
        double x = src[i], y = oracle_f16_to_f64(dst[i]);
        if (isnan(x)) {
            CHECK(isnan(y), "NaN kept at %d", i);
        } else if (fabs(x) >= 65520.0) {
            CHECK(isinf(y) && signbit(y) == signbit(x), "overflow at %d", i);
        } else {
            /* nearest: no fp16 neighbour is closer */
            uint16_t up = (uint16_t)(dst[i] + 1), dn = (uint16_t)(dst[i] - 1);
            double err = fabs(y - x);
            if ((up & 0x7c00u) != 0x7c00u) CHECK(fabs(oracle_f16_to_f64(up) - x) >= err, "up %d", i);
            if ((dst[i] & 0x7fffu) != 0) CHECK(fabs(oracle_f16_to_f64(dn) - x) >= err, "dn %d", i);
        }
    }
}

static void check_refusals(void)
{
    double d[4];
    int32_t ids[4];
    uint16_t h[8] = {0};
    CHECK(oracle_scores(h, 0, 8, h, 8, -1, 1, 1, 8, 1, NULL, 0, d, d, d, 1) != 0, "G < 0");
    CHECK(oracle_scores(h, 0, 8, h, 8, 1, 1, 0, 8, 1, NULL, 0, d, d, d, 1) != 0, "H < 1");
    CHECK(oracle_scores(h, 0, 8, h, 8, 1, 1, 1, 8, 2, NULL, 0, d, d, d, 1) != 0, "ld < nb");
    CHECK(oracle_topk(d, 1, 1, 2, 1, ids, 1, NULL) != 0, "ld < nb");
    CHECK(oracle_topk(d, 4, 1, 4, 2, ids, 1, NULL) != 0, "ld_ids < k");
}

int main(void)
{
    check_one_hot();
    check_topk();
    check_convert();
    check_refusals();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitized checks passed\n");
    return 0;
}
