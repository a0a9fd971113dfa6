/* Exhaustive check of the three-operation quotient the GPU quantiser uses in place of a division
 * (q = RN(x*r), e = fma(-q, s, x), q' = copysign(fma(e, r, q), x) with r = RN(1/s)), against the
 * correctly rounded fp32 quotient x / s, for every block scale the quantiser can produce
 * (s = RN(max(amax, fp32(1e-4)) / 448) with amax any finite bf16 value) and every bf16 x the
 * block can hold (|x| <= amax, or below 1e-4 for the floored scale), both signs.
 * Claim checked: where |x/s| >= 2^-11 the two agree bit for bit; below, both are at most 2^-10
 * in magnitude and carry the sign of x, so both encode to the same signed E4M3 zero.
 * Built by the test with gcc -O2 -fopenmp; IEEE fp32 with subnormals, round to nearest even. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(void) {
    long long pairs = 0, bad = 0, scales = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, scales)
    for (int32_t ab = 0; ab < 0x7F80; ++ab) {            /* amax: every finite bf16 >= 0 */
        float amax = f_of((uint32_t)ab << 16);
        if (amax < 1e-4f && ab != 0) continue;            /* one floored scale, handled at ab == 0 */
        float ac = amax < 1e-4f ? 1e-4f : amax;
        float s = ac / 448.0f;
        float r = 1.0f / s;
        uint32_t xmax = (uint32_t)ab;
        if (ab == 0) while (f_of((xmax + 1) << 16) < 1e-4f) ++xmax;
        ++scales;
        for (uint32_t xb = 0; xb <= xmax; ++xb) {
            for (int neg = 0; neg < 2; ++neg) {
                float x = f_of((xb << 16) | (neg ? 0x80000000u : 0u));
                float ref = x / s;
                float q = x * r;
                float e = fmaf(-q, s, x);
                float q1 = copysignf(fmaf(e, r, q), x);
                ++pairs;
                int ok;
                if (fabsf(ref) >= 0x1p-11f) ok = b_of(q1) == b_of(ref);
                else ok = fabsf(q1) <= 0x1p-10f && signbit(q1) == signbit(ref);
                if (!ok) {
                    ++bad;
#pragma omp critical
                    if (bad < 5) printf("mismatch s=%a x=%a ref=%a got=%a\n", s, x, ref, q1);
                }
            }
        }
    }
    printf("scales %lld pairs %lld mismatches %lld\n", scales, pairs, bad);
    return bad != 0;
}
