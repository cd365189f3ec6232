/* CPU check of the division-by-6 formula the kernels use for the map-to-6
 * block scale RN(a / 6): q0 = RN(a * r6) with r6 = RN(1/6), the exact
 * remainder r = fma(-q0, 6, a), and q = fma(r, r6, q0). Every non-negative
 * binary32 a from +0 to +inf is run through the formula in binary32 with
 * hardware fused multiply-adds and compared with IEEE RN(a / 6).
 * Prints: "<mismatches for finite a >= 2^-125> <mismatches below 2^-125>
 * <1 if +inf mismatches, else 0> <inputs checked>".
 * TEST INFRASTRUCTURE: built and run by tests/test_div6_formula.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(void) {
    const float r6 = 0x1.555556p-3f; /* RN(1/6) */
    const float six = 6.0f;
    if (to_bits(r6) != to_bits(1.0f / six)) {
        printf("r6 is not RN(1/6)\n");
        return 2;
    }
    unsigned long long above = 0, below = 0, inf = 0, checked = 0;
#pragma omp parallel for schedule(static) reduction(+ : above, below, inf, checked)
    for (int64_t i = 0; i <= 0x7F800000LL; i++) {
        const float a = from_bits((uint32_t)i);
        const float q0 = a * r6;
        const float r = fmaf(-q0, six, a);
        const float q = fmaf(r, r6, q0);
        const float want = a / six;
        if (to_bits(q) != to_bits(want)) {
            if (isinf(a)) inf++;
            else if (a >= 0x1p-125f) above++;
            else below++;
        }
        checked++;
    }
    printf("%llu %llu %llu %llu\n", above, below, inf, checked);
    return 0;
}
