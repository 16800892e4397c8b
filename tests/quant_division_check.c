/*
 * Exhaustive check (CPU) that the block quantizer's division step is exact: for every
 * positive finite binary16 block maximum amax, with s = amax / 448 in float32, and every
 * binary16 x with |x| <= amax, the reciprocal-and-correction sequence
 *     r = 1 / s;  y0 = x * r;  e = fma(-y0, s, x);  y = copysign(fma(e, r, y0), x)
 * (one IEEE division per block instead of one per element; Markstein's correction step;
 * copysign keeps the sign of a zero x, which the correction would turn into +0) gives the
 * same float32, bit for bit, as the IEEE quotient x / s; and that the scale itself,
 *     s0 = amax * RN(1/448);  s = fma(fma(-s0, 448, amax), RN(1/448), s0)
 * equals the IEEE quotient amax / 448 for every amax. Prints the number of pairs checked and
 * of mismatches; exits 1 on any mismatch. Build: gcc -O2 -fopenmp -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f16_value(uint16_t h) { /* exact: binary16 -> float */
    int e = (h >> 10) & 31, f = h & 1023;
    float v = e == 0 ? ldexpf((float)f, -24) : ldexpf((float)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

static uint32_t bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }

int main(void) {
    long long pairs = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad)
    for (int am = 1; am < 0x7C00; ++am) {
        const float amax = f16_value((uint16_t)am);
        const float s = amax / 448.0f;
        {
            const float inv448 = 1.0f / 448.0f;
            const float s0 = amax * inv448;
            const float s1 = fmaf(fmaf(-s0, 448.0f, amax), inv448, s0);
            ++pairs;
            if (bits(s1) != bits(s)) {
                ++bad;
                if (bad < 5) printf("scale mismatch amax=%a: %a vs %a\n", amax, s1, s);
            }
        }
        const float r = 1.0f / s;
        for (int xh = 0; xh <= am; ++xh)
            for (int sg = 0; sg < 2; ++sg) {
                const float x = f16_value((uint16_t)(xh | (sg << 15)));
                const float ref = x / s;
                const float y0 = x * r;
                const float e = fmaf(-y0, s, x);
                const float y = copysignf(fmaf(e, r, y0), x);
                ++pairs;
                if (bits(y) != bits(ref)) {
                    ++bad;
                    if (bad < 5) printf("mismatch amax=%a x=%a: %a vs %a\n", amax, x, y, ref);
                }
            }
    }
    printf("pairs %lld mismatches %lld\n", pairs, bad);
    return bad != 0;
}
