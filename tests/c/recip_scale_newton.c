/* Host check of the kernels' reciprocal of a binary16 scale: one Newton step
 * r1 = fma(r0, fma(-s, r0, 1), r0) from a first approximation r0.  For every
 * positive finite binary16 s (2^-24 .. 65504) and every r0 within two fp32
 * ulps of RN(1/s) (the hardware reciprocal is documented within one), r1
 * must equal the IEEE quotient 1/s.  As a control, the same step for full
 * 24-bit divisors s = 1 + k 2^-23 must miss RN(1/s) somewhere: the proof
 * needs the 11-bit significand of a binary16 scale, and the check can tell.
 * Prints one line and exits non-zero on any failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits(float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    return b;
}

/* binary16 pattern (positive, finite) -> its exact value as fp32 */
static float f16_value(uint32_t h)
{
    const uint32_t e = h >> 10, m = h & 0x3FFu;
    return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(1024u + m), (int)e - 25);
}

int main(void)
{
    uint64_t checked = 0, bad = 0, control_off = 0;
    for (uint32_t h = 1; h < 0x7C00u; ++h) {
        const float s = f16_value(h);
        const float want = 1.0f / s;
        float r0 = nextafterf(nextafterf(want, 0.0f), 0.0f);      /* RN(1/s) - 2 ulp */
        for (int k = -2; k <= 2; ++k, r0 = nextafterf(r0, INFINITY)) {
            const float e = fmaf(-s, r0, 1.0f);
            const float r1 = fmaf(r0, e, r0);
            ++checked;
            if (bits(r1) != bits(want)) {
                if (bad < 5) printf("mismatch: h=0x%04x r0=%a r1=%a want=%a\n", h, r0, r1, want);
                ++bad;
            }
        }
    }
    for (uint32_t k = 1; k < (1u << 23); ++k) {
        const float s = 1.0f + ldexpf((float)k, -23);
        const float want = 1.0f / s;
        float r0 = nextafterf(nextafterf(want, 0.0f), 0.0f);
        for (int j = -2; j <= 2; ++j, r0 = nextafterf(r0, INFINITY))
            if (bits(fmaf(r0, fmaf(-s, r0, 1.0f), r0)) != bits(want)) ++control_off;
    }
    printf("recip_scale_newton: checked=%llu mismatches=%llu control_off=%llu\n",
           (unsigned long long)checked, (unsigned long long)bad, (unsigned long long)control_off);
    return (bad == 0 && checked == 5ull * 0x7BFFu && control_off > 0) ? 0 : 1;
}
