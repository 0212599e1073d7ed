/* The division identity the quantize kernel uses in place of one IEEE division per element:
 *   r = fp32(1 / a), q0 = fp32(x r), n = fma(fma(-a, q0, x), r, q0)   equals   fp32(x / a)
 * for a in [2^-60, 2^100], |x| <= a, whenever |x / a| >= 2^-40 (below that the remainder may
 * leave the normal range and n may differ in its last bits).  Samples: random significands and
 * exponents, all-ones and all-zeros significands of a, quotients spread over [2^-60, 1] and next
 * to the NF4 decision points (0.02 .. 1.02), and x = +-a.  Prints the number of samples and of
 * differences at or above 2^-40; exit status 1 if there is any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static float from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}
static uint32_t to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

int main(int argc, char **argv) {
    const long samples = argc > 1 ? atol(argv[1]) : 20000000L;
    long differ = 0;
    for (long it = 0; it < samples; ++it) {
        const uint32_t ua = (uint32_t)next(), ux = (uint32_t)next();
        const uint32_t ea = 67 + (ua >> 8) % 161;          /* biased exponent: 2^-60 .. 2^100 */
        uint32_t ma = ua & 0x7FFFFF;
        if ((ua >> 28) == 0) ma = 0x7FFFFF;
        if ((ua >> 28) == 1) ma = 0;
        const float a = from_bits((ea << 23) | ma);
        float f = from_bits(0x3F800000u | (ux & 0x7FFFFF)) - 1.0f;
        if ((ux >> 30) == 0) f = ldexpf(f, -(int)((ux >> 23) % 60));
        if ((ux >> 30) == 1) f = 0.02f + 0.001f * (float)((ux >> 10) % 1000);
        float x = f * a;
        if ((ux >> 29) & 1) x = -x;
        if ((ux & 0xFFF) == 7) x = a;
        if ((ux & 0xFFF) == 9) x = -a;
        if (fabsf(x) > a) continue;
        const float ref = x / a;
        const float r = 1.0f / a;
        const float q0 = x * r;
        const float n = fmaf(fmaf(-a, q0, x), r, q0);
        if (to_bits(n) != to_bits(ref) && fabsf(ref) >= 0x1p-40f) {
            if (differ < 5) printf("x=%a a=%a x/a=%a got %a\n", x, a, ref, n);
            ++differ;
        }
    }
    printf("%ld samples, %ld differences\n", samples, differ);
    return differ ? 1 : 0;
}
