/* Test helper: compares a scalar fp32 -> fp16 converter against the x86 F16C
 * instruction (VCVTPS2PH with round-to-nearest-even), over a range of fp32
 * bit patterns.  Built by the CPU test suite with gcc -mf16c -fopenmp. */
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

typedef uint16_t (*conv_one_fn)(float);

uint16_t f16c_one(float x) { return (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT); }

/* Returns the number of mismatching patterns in [start, start + count);
 * *first_bad gets the smallest mismatching pattern (or all ones). */
int64_t f16c_compare_range(conv_one_fn conv, uint64_t start, uint64_t count, uint64_t *first_bad)
{
    int64_t bad = 0;
    uint64_t fb = ~(uint64_t)0;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad) reduction(min : fb)
    for (uint64_t i = 0; i < count; ++i) {
        uint32_t u = (uint32_t)(start + i);
        float x;
        memcpy(&x, &u, 4);
        uint16_t want = (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
        if (conv(x) != want) {
            ++bad;
            if (start + i < fb) fb = start + i;
        }
    }
    *first_bad = fb;
    return bad;
}
