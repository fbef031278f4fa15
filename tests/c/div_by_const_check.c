/* Host check of the division-free quotient used for the quantizers' scales:
 * for Q in {15, 255, 7, 127} and every finite fp32 x >= 0 (all 2^31 bit
 * patterns below +inf), q0 = x * RN(1/Q), r = fma(-q0, Q, x),
 * q = fma(r, RN(1/Q), q0) must equal the IEEE quotient x / Q.
 * The plain product q0 alone is also counted: it must differ somewhere, or
 * the check would not be telling the two apart.
 * Prints one line per divisor and exits non-zero on any failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b)
{
    float x;
    memcpy(&x, &b, sizeof x);
    return x;
}

int main(void)
{
    static const float divisors[4] = {15.0f, 255.0f, 7.0f, 127.0f};
    int failed = 0;
    for (int d = 0; d < 4; ++d) {
        const float Q = divisors[d];
        const float inv = 1.0f / Q;
        uint64_t bad = 0, plain_bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad, plain_bad)
        for (int64_t i = 0; i < 0x7F800000LL; ++i) {
            const float x = from_bits((uint32_t)i);
            const float q0 = x * inv;
            const float r = fmaf(-q0, Q, x);
            const float q = fmaf(r, inv, q0);
            const float want = x / Q;
            bad += q != want;
            plain_bad += q0 != want;
        }
        printf("Q=%g mismatches=%llu plain_product_mismatches=%llu\n", (double)Q, (unsigned long long)bad,
               (unsigned long long)plain_bad);
        failed |= bad != 0 || plain_bad == 0;
    }
    return failed;
}
