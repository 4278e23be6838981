/* Exhaustive host check of the second-level step used by the gfx950 kernels.
 *
 * The kernels need step = fp32(c2 / 448) correctly rounded (double quantization,
 * "Double quantization" on the zerotofrontier.app "sft/peft" page, decoded as
 * c1' = E4M3(q) * step + mean).  Instead of an IEEE division they form
 *     q0 = RN(c2 * RN(1/448)),  e = fma(-q0, 448, c2),  step = fma(e, RN(1/448), q0)
 * for 2^-100 <= |c2| <= FLT_MAX.  This program compares that sequence with the
 * IEEE quotient for every non-negative fp32 value in the range (the sequence is
 * odd in c2, so the negative half follows) and prints the number of mismatches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
    const float rcp = 1.0f / 448.0f;
    const uint32_t lo = to_bits(0x1p-100f), hi = to_bits(3.4028234663852886e38f);
    long bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (long u = lo; u <= (long)hi; ++u) {
        const float c = from_bits((uint32_t)u);
        volatile float ref = c / 448.0f;
        const float q0 = c * rcp;
        const float e = fmaf(-q0, 448.0f, c);
        const float s = fmaf(e, rcp, q0);
        bad += to_bits(s) != to_bits(ref);
        n += 1;
    }
    printf("%ld %ld\n", n, bad);
    return 0;
}
