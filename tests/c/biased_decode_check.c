/* Host check of the owner reduce's decode of a peer's codes for an integer
 * zero point: with b = binary16(1024 + q) and c = fma(-(1024 + z), s, 0),
 * fma(b, s, c) must equal the two-step decode (q - z) * s bit for bit, for
 * every positive finite binary16 scale s and every code q and zero point z
 * in [0, 255] (8-bit codes; 4-bit codes are a subset), and for s = 0 (an
 * all-zero group's word) where q == z.  As a control, the same fma on the
 * unbiased code, fma(q, s, -z * s) with z * s rounded first, is also exact
 * (it is the form it replaced), while a decode that rounds q * s first,
 * q * s - z * s in two roundings, must differ somewhere at full 24-bit
 * scales: the check can tell an exact form from an inexact one.
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
    uint64_t checked = 0, bad = 0, old_bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : checked, bad, old_bad)
    for (int h = 0; h < 0x7C00; ++h) {
        const float s = h == 0 ? 0.0f : f16_value((uint32_t)h);
        for (int z = 0; z < 256; ++z) {
            const float c = fmaf(-(float)(1024 + z), s, 0.0f);
            const float nzs = -((float)z * s);
            for (int q = 0; q < 256; ++q) {
                if (h == 0 && q != z) continue;
                volatile float d = (float)q - (float)z;
                const float want = d * s;
                const float got = fmaf((float)(1024 + q), s, c);
                const float old = fmaf((float)q, s, nzs);
                ++checked;
                if (bits(got) != bits(want)) ++bad;
                if (bits(old) != bits(want)) ++old_bad;
            }
        }
    }
    /* control: two roundings at full 24-bit scales miss the exact value */
    uint64_t control_off = 0;
    for (uint32_t k = 1; k < (1u << 16); ++k) {
        const float s = 1.0f + ldexpf((float)(k * 127u), -23);
        for (int q = 0; q < 256; q += 7) {
            volatile float qs = (float)q * s, zs = 131.0f * s;
            if (bits(qs - zs) != bits(((float)q - 131.0f) * s)) ++control_off;
        }
    }
    printf("biased_decode_check: checked=%llu mismatches=%llu unbiased_fma_mismatches=%llu control_off=%llu\n",
           (unsigned long long)checked, (unsigned long long)bad, (unsigned long long)old_bad,
           (unsigned long long)control_off);
    return (bad == 0 && old_bad == 0 && control_off > 0 && checked == 31743ull * 65536ull + 256ull) ? 0 : 1;
}
