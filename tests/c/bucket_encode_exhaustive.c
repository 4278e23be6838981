/* Exhaustive host check of the bucket-table NF4 encode used by the gfx950 quantize kernel.
 *
 * The code of a normalised value x (|x| <= 1) is the number of thresholds below it, the
 * thresholds being the largest fp32 values not above the midpoints of adjacent NF4 levels
 * ("Block-wise quantization in one page" and "NF4, derived from normal quantiles" on the
 * zerotofrontier.app "sft/peft" page: nearest level, ties to the lower code).  The kernel
 * instead reads entry floor(clamp(32 x, -33, 32)) + 33 of a 66-entry table: entry 1 + b
 * holds, for bucket b = floor(32 x) + 32, the count of thresholds below the bucket and the
 * bucket's own threshold (+inf if none); entry 0 ({0, +inf}) is where a NaN quotient
 * lands (the clamp's max returns the number operand), so it takes code 0 as every
 * comparison x > m_j fails for it.  It adds one strict comparison.  This program takes the
 * 16 levels (hex floats) on the command line, builds both, and compares them for every
 * fp32 x in [-1, 1] (both zeros and the subnormals included) and for NaN.  It prints
 * "<values checked> <mismatches> <max thresholds in a bucket>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int main(int argc, char** argv) {
    if (argc != 17) { fprintf(stderr, "usage: %s level0 .. level15\n", argv[0]); return 2; }
    float lv[16], th[15];
    for (int i = 0; i < 16; ++i) lv[i] = strtof(argv[1 + i], NULL);
    for (int j = 0; j < 15; ++j) {
        const double mid = ((double)lv[j] + (double)lv[j + 1]) / 2.0;
        float t = (float)mid;
        if ((double)t > mid) t = nextafterf(t, -INFINITY);
        th[j] = t;
    }
    uint32_t below[66];
    float bth[66];
    int most = 0;
    for (int b = 0; b < 66; ++b) {
        const float lo = (float)(b - 33) * (1.0f / 32.0f), hi = lo + 1.0f / 32.0f;
        below[b] = 0;
        bth[b] = INFINITY;
        int in = 0;
        for (int j = 0; j < 15; ++j) {
            below[b] += th[j] < lo;
            if (th[j] >= lo && th[j] < hi) { bth[b] = th[j]; ++in; }
        }
        if (in > most) most = in;
        if (b == 0) { below[b] = 0; bth[b] = INFINITY; }
    }
    long bad = 0, n = 0;
    const uint32_t one = 0x3F800000u;      /* bits of 1.0f */
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (long u = 0; u <= (long)one; ++u) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            const float x = from_bits((uint32_t)u | (sgn ? 0x80000000u : 0u));
            uint32_t ref = 0;
            for (int j = 0; j < 15; ++j) ref += x > th[j];
            const int b = (int)floorf(fminf(fmaxf(x * 32.0f, -33.0f), 32.0f)) + 33;
            const uint32_t got = below[b] + (x > bth[b]);
            bad += got != ref;
            ++n;
        }
    }
    {   /* a NaN quotient: no comparison holds, code 0 */
        const float x = nanf("");
        const int b = (int)floorf(fminf(fmaxf(x * 32.0f, -33.0f), 32.0f)) + 33;
        bad += (below[b] + (x > bth[b])) != 0u;
        ++n;
    }
    printf("%ld %ld %d\n", n, bad, most);
    return 0;
}
