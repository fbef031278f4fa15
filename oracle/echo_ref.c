/*
 * echo_ref.c — the CPU oracle for Echo's error-compensated low-bit all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU library must
 * compute; it is plain, slow, single-threaded C with no blocking or fusion.
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no source, header, table or helper with the HIP
 * library, and it includes nothing from it.
 *
 * Sources (the method is described, not listed, on these pages):
 *   [EchoCard]  "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication
 *               for LLM Training and Inference" (arXiv 2610.14277), paper card:
 *               abstract, Fig. 1, Fig. 2(a)/(b), Table 8, appendix Fig. 4.
 *   [Blog]      "Your All-Reduce Is 4x Overpriced: Echo's 4-Bit Error-Feedback
 *               Trick for Tensor-Parallel Training", sections "The cancellation
 *               rule" and "The part of your stack nobody profiles".
 *
 * Arithmetic.  The pages say only "high precision" for the owner's sum; the
 * parity bar this oracle serves fixes it as IEEE fp32, summed in rank order
 * j = 0..P-1 with no fused multiply-add.  Build with
 * -O2 -ffp-contract=off -fno-fast-math so that every float operation below is
 * one correctly rounded IEEE operation (x86-64 SSE, round to nearest even).
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes):
 *   - the quantizer ("zero-aware asymmetric", [EchoCard] Table 8; Eqn. (8) is
 *     named in Fig. 4 but not printed) is the min/max affine quantizer whose
 *     range is widened to contain 0, with an integer zero point so that 0 is
 *     a grid point; its scale and zero point are stored as IEEE binary16
 *     ([Blog] "The cancellation rule": the codes travel as 4-bit integers
 *     and each group's parameters at half precision);
 *   - codes are unsigned in [0, 2^b-1]; for b = 4 two codes share a byte,
 *     the even element in the low nibble;
 *   - segment s (P equal contiguous segments) is owned by rank s;
 *   - the owner's own term is compensated but never quantized before the sum;
 *   - the two-timescale compensator is an error debt: a fraction alpha of the
 *     newest error is returned at the next call, the rest enters a slow
 *     memory M that is released at rate beta per call.
 *
 * Parity status of each function is stated at its definition.  Parity
 * unpinned: the two-timescale compensator's constants and its exact update
 * equation (the pages name the compensator and where it runs, and print
 * neither), and the values of appendix Fig. 4 (not in the text).  Everything
 * else is pinned by the CPU tests against library conversions, exact
 * arithmetic, brute force over all codes, closed forms and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_EINVAL (-1)
#define REF_EUNSUP (-3)
#define REF_ESHAPE (-4)

#define REF_ERR_NEGATED 1   /* write -e (the next call's compensation) instead of e */
#define REF_Q_NAIVE 2       /* quantizer: naive zero point (Table 8 ablation)          */
#define REF_Q_SYMMETRIC 4   /* quantizer: symmetric grid (Table 8 ablation)            */
#define REF_Q_MSE 16        /* quantizer: zero point searched for the least squared error */

enum { Q_ZERO_AWARE = 0, Q_NAIVE = 1, Q_SYMMETRIC = 2, Q_MSE = 3 };

/* quantizer selected by the flag bits; -1 when more than one is asked for */
static int quant_of(int flags)
{
    int naive = (flags & REF_Q_NAIVE) != 0, sym = (flags & REF_Q_SYMMETRIC) != 0, mse = (flags & REF_Q_MSE) != 0;
    if (naive + sym + mse > 1) return -1;
    return naive ? Q_NAIVE : (sym ? Q_SYMMETRIC : (mse ? Q_MSE : Q_ZERO_AWARE));
}
#define REF_OUT_F32 0
#define REF_OUT_BF16 1

/* ------------------------------------------------------------------------ */
/* Number formats, from the IEEE 754 definitions.                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary32 -> binary16, round to nearest, ties to even, subnormals kept.
 * Written from the format definition: the input is an integer significand M
 * times 2^(e-23); the output grid at the input's binade has quantum
 * 2^(max(e,-14)-10); drop the bits below that quantum with a
 * round-half-even decision, and let a carry roll into the exponent field.
 * Pinned against numpy's float16 conversion on every binade boundary and
 * rounding pattern (and exhaustively in the slow suite). */
uint16_t echo_ref_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);      /* NaN  */
    if (a == 0x7F800000u) return (uint16_t)(sign | 0x7C00u);     /* inf  */
    if (a < 0x00800000u) return sign;  /* binary32 subnormal: below 2^-126, far under half of 2^-24 */
    int e = (int)(a >> 23) - 127;                  /* unbiased exponent     */
    uint32_t M = (a & 0x007FFFFFu) | 0x00800000u;  /* 24-bit significand    */
    if (e > 15) return (uint16_t)(sign | 0x7C00u); /* >= 2^16: overflow     */
    if (e < -25) return sign;                      /* < 2^-25: rounds to 0  */
    int shift = 13 + (e < -14 ? (-14 - e) : 0);    /* 13 .. 24              */
    uint32_t N = M >> shift;
    uint32_t rem = M & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (N & 1u))) N += 1u;
    if (e < -14)               /* subnormal result; N == 1024 is the smallest normal */
        return (uint16_t)(sign | N);
    /* normal result: N in [1024, 2048]; a carry to 2048 bumps the exponent,
     * and exponent field 31 is infinity */
    uint32_t h = ((uint32_t)(e + 15) << 10) + (N - 1024u);
    if (h >= 0x7C00u) h = 0x7C00u;
    return (uint16_t)(sign | h);
}

/* binary16 -> binary32 (exact). */
float echo_ref_f16_to_f32(uint16_t h)
{
    uint32_t sign = (h & 0x8000u) ? 1u : 0u;
    uint32_t E = (h >> 10) & 0x1Fu;
    uint32_t m = h & 0x3FFu;
    float mag;
    if (E == 0) mag = ldexpf((float)m, -24);
    else if (E == 31) mag = m ? NAN : INFINITY;
    else mag = ldexpf((float)(1024u + m), (int)E - 25);
    return sign ? -mag : mag;
}

void echo_ref_f32_to_f16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = echo_ref_f32_to_f16(in[i]);
}

/* bfloat16 is the upper half of a binary32. */
float echo_ref_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even (drop 16 bits). */
uint16_t echo_ref_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t up = u >> 16, rem = u & 0xFFFFu;
    if (rem > 0x8000u || (rem == 0x8000u && (up & 1u))) up += 1u;
    return (uint16_t)up;
}

void echo_ref_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = echo_ref_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* O1: the group quantizer Q_b and its dequantizer.                         */
/* [EchoCard] Table 8 (full method: zero-aware asymmetric, g = 128; the     */
/* ablations "naive zero-point" and "symmetric grid"); Fig. 4 (Eqn. (8)     */
/* with b = 4); [Blog] "The cancellation rule" (half-precision parameters). */
/* All three quantizers store a binary16 scale s and a binary16 zero point z */
/* per group and decode alike: v_hat = (q - z) * s.                          */
/* ------------------------------------------------------------------------ */

/* binary16 scale from an fp32 quotient: nearest even, a zero result becomes
 * 2^-24 and an infinite one 65504 */
static uint16_t scale_bits(float s32)
{
    uint16_t sh = echo_ref_f32_to_f16(s32);
    if (sh == 0x0000u) sh = 0x0001u;
    else if (sh == 0x7C00u) sh = 0x7BFFu;
    return sh;
}

static uint8_t clamp_code(double t, int Qm)
{
    return (uint8_t)(t < 0.0 ? 0 : (t > (double)Qm ? Qm : (int)t));
}

/* Zero-aware asymmetric (the full method).  Steps:
 *   1. lo = min(0, min v), hi = max(0, max v): the range always holds 0.
 *   2. hi == lo means an all-zero group: scale +0, zero point 0, codes 0.
 *   3. s32 = (hi - lo) / Qm, Qm = 2^b - 1 (true fp32 division).
 *   4. s = binary16(s32); a zero result becomes 2^-24, an infinite one 65504.
 *   5. inv = 1 / s in fp32 (correctly rounded).
 *   6. z = clamp(rint(-lo * inv), 0, Qm): an integer, so 0 sits on the grid.
 *   7. q_i = clamp(rint(v_i * inv) + z, 0, Qm): the integer zero point is
 *      added after rounding (rint = round half to even).
 *   8. z is stored as binary16 (exact: an integer <= 255).
 * Pinned by: brute-force argmin over all codes on tiny groups, exact-rational
 * scale choice, the grid round-trip, zero-awareness and the element bound. */
static void quant_zero_aware(const float* v, int g, int Qm, uint8_t* q, uint16_t* scale_h,
                             uint16_t* zero_h)
{
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < g; ++i) {
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
    }
    if (hi == lo) {
        for (int i = 0; i < g; ++i) q[i] = 0;
        *scale_h = 0;
        *zero_h = 0;
        return;
    }
    uint16_t sh = scale_bits((hi - lo) / (float)Qm);
    float s = echo_ref_f16_to_f32(sh);
    float inv = 1.0f / s;
    int z = clamp_code((double)rintf(-lo * inv), Qm);
    for (int i = 0; i < g; ++i) q[i] = clamp_code((double)rintf(v[i] * inv) + (double)z, Qm);
    *scale_h = sh;
    *zero_h = echo_ref_f32_to_f16((float)z);
}

/* Naive zero point (Table 8 ablation; reading: the textbook min/max affine
 * quantizer with a real-valued zero point, so 0 is generally not a grid
 * point).  Steps:
 *   1. lo = min v, hi = max v (the range is not widened to hold 0).
 *   2. hi == lo: scale +0, zero point 0, codes 0 (the group decodes to 0).
 *   3. s = binary16((hi - lo) / Qm) with the clamps of the full method.
 *   4. inv = 1 / s; z = binary16((0 - lo) * inv), an overflow clamped to
 *      +-65504.  Written 0 - lo rather than -lo so that a group whose
 *      minimum is a zero gets z = +0 whichever signed zero the minimum is.
 *   5. q_i = clamp(rint(v_i * inv + z), 0, Qm): the zero point is added
 *      before rounding (two fp32 roundings, then rint).
 * Pinned by: brute force over codes and exact-rational choice of s and z on
 * tiny groups, the grid round-trip, and the existence of groups where 0 does
 * not decode to 0. */
static void quant_naive(const float* v, int g, int Qm, uint8_t* q, uint16_t* scale_h, uint16_t* zero_h)
{
    float lo = v[0], hi = v[0];
    for (int i = 1; i < g; ++i) {
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
    }
    if (hi == lo) {
        for (int i = 0; i < g; ++i) q[i] = 0;
        *scale_h = 0;
        *zero_h = 0;
        return;
    }
    uint16_t sh = scale_bits((hi - lo) / (float)Qm);
    float s = echo_ref_f16_to_f32(sh);
    float inv = 1.0f / s;
    uint16_t zh = echo_ref_f32_to_f16((0.0f - lo) * inv);
    if ((zh & 0x7FFFu) == 0x7C00u) zh = (uint16_t)((zh & 0x8000u) | 0x7BFFu);
    float zf = echo_ref_f16_to_f32(zh);
    for (int i = 0; i < g; ++i) q[i] = clamp_code((double)rintf(v[i] * inv + zf), Qm);
    *scale_h = sh;
    *zero_h = zh;
}

/* Symmetric grid (Table 8 ablation; reading: a grid symmetric about 0 with
 * the zero point fixed at the middle code).  Steps, with Qh = 2^(b-1) - 1 and
 * mid = 2^(b-1):
 *   1. a = max |v|.
 *   2. a == 0: scale +0, zero point mid, codes mid (decode to 0).
 *   3. s = binary16(a / Qh) with the clamps of the full method; inv = 1 / s.
 *   4. q_i = clamp(rint(v_i * inv) + mid, 0, Qm), so codes use mid +- Qh.
 * Pinned by: brute force over codes and exact-rational scale choice,
 * zero-awareness and the grid round-trip. */
static void quant_symmetric(const float* v, int g, int bits, uint8_t* q, uint16_t* scale_h,
                            uint16_t* zero_h)
{
    const int Qm = (1 << bits) - 1, Qh = (1 << (bits - 1)) - 1, mid = 1 << (bits - 1);
    float a = 0.0f;
    for (int i = 0; i < g; ++i)
        if (fabsf(v[i]) > a) a = fabsf(v[i]);
    *zero_h = echo_ref_f32_to_f16((float)mid);
    if (a == 0.0f) {
        for (int i = 0; i < g; ++i) q[i] = (uint8_t)mid;
        *scale_h = 0;
        return;
    }
    uint16_t sh = scale_bits(a / (float)Qh);
    float s = echo_ref_f16_to_f32(sh);
    float inv = 1.0f / s;
    for (int i = 0; i < g; ++i) q[i] = clamp_code((double)rintf(v[i] * inv) + (double)mid, Qm);
    *scale_h = sh;
}

/* Zero point searched for the least squared error (a variant of the full
 * method: Table 8 names the zero-aware quantizer's zero point as the part
 * that matters; this variant keeps the full method's scale and replaces the
 * closed-form zero point by an exhaustive search).  Reading: the scale s,
 * 1/s and the codes' rule are those of the zero-aware quantizer; the zero
 * point is the integer z in [0, Qm] whose codes
 *   q_i(z) = clamp(rint(t_i) + z, 0, Qm),   t_i = v_i * (1/s)  (fp32 product)
 * give the least squared error of the group measured in units of s,
 *   E(z) = sum_i (q_i(z) - z - t_i)^2,
 * the smallest such z when several tie.  z only moves codes through the
 * clamp: with r_i = rint(t_i) and c_i = clamp(r_i, -z, Qm - z) = q_i(z) - z,
 *   E(z) = sum_i (r_i - t_i)^2 + D(z),   D(z) = sum_i (c_i - r_i)(c_i + r_i - 2 t_i),
 * and the first sum does not depend on z, so the search compares D(z).
 * D is evaluated exactly in double: a term is nonzero only for a clamped
 * element, whose |t_i| >= 1/2 makes t_i a multiple of 2^-24 below 2^10 in
 * magnitude, so every term is a multiple of 2^-24 below 2^19 and every
 * partial sum of at most 256 of them has fewer than 53 significant bits.
 * An all-zero group gives s = +0, z = 0, codes 0.
 * Pinned by: the exact squared error of every z computed with rationals on
 * tiny groups (smallest argmin), the scale of the full method, and never a
 * larger error than the closed-form zero point. */
static void quant_mse(const float* v, int g, int Qm, uint8_t* q, uint16_t* scale_h, uint16_t* zero_h)
{
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < g; ++i) {
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
    }
    if (hi == lo) {
        for (int i = 0; i < g; ++i) q[i] = 0;
        *scale_h = 0;
        *zero_h = 0;
        return;
    }
    uint16_t sh = scale_bits((hi - lo) / (float)Qm);
    float s = echo_ref_f16_to_f32(sh);
    float inv = 1.0f / s;
    int best_z = 0;
    double best = 0.0;
    for (int z = 0; z <= Qm; ++z) {
        double d = 0.0;
        for (int i = 0; i < g; ++i) {
            float t = v[i] * inv;
            double r = (double)rintf(t);
            double c = r < (double)-z ? (double)-z : (r > (double)(Qm - z) ? (double)(Qm - z) : r);
            d += (c - r) * (c + r - 2.0 * (double)t);
        }
        if (z == 0 || d < best) {
            best = d;
            best_z = z;
        }
    }
    for (int i = 0; i < g; ++i) q[i] = clamp_code((double)rintf(v[i] * inv) + (double)best_z, Qm);
    *scale_h = sh;
    *zero_h = echo_ref_f32_to_f16((float)best_z);
}

/* Quantize one group of g values to unsigned b-bit codes (one per byte in q)
 * with quantizer `quant` (0 zero-aware, 1 naive zero point, 2 symmetric,
 * 3 zero point searched for the least squared error). */
int echo_ref_quantize_group_q(const float* v, int g, int bits, int quant, uint8_t* q,
                              uint16_t* scale_h, uint16_t* zero_h)
{
    if (bits != 4 && bits != 8) return REF_EUNSUP;
    if (g < 1) return REF_EINVAL;
    const int Qm = (1 << bits) - 1;
    switch (quant) {
    case Q_ZERO_AWARE: quant_zero_aware(v, g, Qm, q, scale_h, zero_h); return REF_OK;
    case Q_NAIVE: quant_naive(v, g, Qm, q, scale_h, zero_h); return REF_OK;
    case Q_SYMMETRIC: quant_symmetric(v, g, bits, q, scale_h, zero_h); return REF_OK;
    case Q_MSE: quant_mse(v, g, Qm, q, scale_h, zero_h); return REF_OK;
    default: return REF_EINVAL;
    }
}

/* The full method's quantizer (zero-aware asymmetric). */
int echo_ref_quantize_group(const float* v, int g, int bits, uint8_t* q,
                            uint16_t* scale_h, uint16_t* zero_h)
{
    return echo_ref_quantize_group_q(v, g, bits, Q_ZERO_AWARE, q, scale_h, zero_h);
}

/* Dequantizer: v_hat = (q - z) * s in fp32.  q - z is exact (q <= 255 and z
 * a binary16 value); with an integer z (zero-aware, symmetric) the product
 * is exact too: |q - z| <= 255 needs 8 bits and s has an 11-bit significand. */
float echo_ref_dequant(int q, uint16_t scale_h, uint16_t zero_h)
{
    float d = (float)q - echo_ref_f16_to_f32(zero_h);
    return d * echo_ref_f16_to_f32(scale_h);
}

/* Packed code stream: b = 4 -> element i in byte i/2, low nibble when i is
 * even; b = 8 -> one byte per element. */
static int code_at(const uint8_t* codes, int64_t i, int bits)
{
    if (bits == 8) return codes[i];
    uint8_t byte = codes[i >> 1];
    return (i & 1) ? (byte >> 4) : (byte & 0x0F);
}

static void code_put(uint8_t* codes, int64_t i, int bits, int q)
{
    if (bits == 8) { codes[i] = (uint8_t)q; return; }
    uint8_t* byte = &codes[i >> 1];
    if (i & 1) *byte = (uint8_t)((*byte & 0x0F) | (q << 4));
    else       *byte = (uint8_t)((*byte & 0xF0) | q);
}

/* Per-group parameter words: params[2*k] = scale bits, params[2*k+1] = zero
 * bits, for the group starting at message element k*g. */

/* Quantize the g values u[0..g) of the group that starts at message element
 * `base` into the code stream and the parameter array; count, if not NULL,
 * is incremented for every element passed through the quantizer. */
static void quantize_into(const float* u, int64_t base, int g, int bits, int quant,
                          uint8_t* codes, uint16_t* params, uint8_t* qscratch, int* count)
{
    uint16_t sh, zh;
    echo_ref_quantize_group_q(u, g, bits, quant, qscratch, &sh, &zh);
    for (int i = 0; i < g; ++i) code_put(codes, base + i, bits, qscratch[i]);
    params[2 * (base / g)] = sh;
    params[2 * (base / g) + 1] = zh;
    if (count)
        for (int i = 0; i < g; ++i) count[base + i] += 1;
}

/* ------------------------------------------------------------------------ */
/* Argument checks shared by the call-level functions below.                */
/* ------------------------------------------------------------------------ */

static int check_shape(int64_t n, int P, int64_t tile_begin, int64_t tile_len,
                       int bits, int g)
{
    if (bits != 4 && bits != 8) return REF_EUNSUP;
    if (g < 1 || (bits == 4 && (g & 1))) return REF_EUNSUP;
    if (P < 1 || P > 64) return REF_EINVAL;
    if (n < 0 || tile_begin < 0 || tile_len < 0) return REF_ESHAPE;
    if (n % ((int64_t)P * g) != 0) return REF_ESHAPE;
    int64_t S = n / P;
    if (tile_begin % g || tile_len % g || tile_begin > S || tile_len > S - tile_begin) return REF_ESHAPE;
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* O2: entry pass + push quantize, for one rank.                             */
/* [EchoCard] Fig. 2(a) (a rank quantizes only segments other ranks own);   */
/* Fig. 4 (three quantized copies, own copy kept); [Blog] "The cancellation  */
/* rule" (compensation fused into the entry pass).                           */
/* For every segment s != rank and every group of the tile [tile_begin,      */
/* tile_begin + tile_len) inside it: u = f32(x) + comp (u = f32(x) when comp */
/* is NULL); codes and parameters of Q_b(u); err = Q_hat(u) - u.             */
/* err may alias comp: each group's compensation is read before any of its  */
/* errors is written.                                                        */
/* ------------------------------------------------------------------------ */
static int push_impl(const uint16_t* x, const float* comp, int64_t n, int P, int rank,
                     int64_t tile_begin, int64_t tile_len, int bits, int g,
                     uint8_t* codes, uint16_t* params, float* err, int flags, int* count)
{
    int rc = check_shape(n, P, tile_begin, tile_len, bits, g);
    if (rc) return rc;
    if (rank < 0 || rank >= P) return REF_EINVAL;
    if ((!x || !codes || !params) && n > 0) return REF_EINVAL;
    const int quant = quant_of(flags);
    if (quant < 0) return REF_EINVAL;
    int64_t S = n / P;
    float* u = (float*)malloc(sizeof(float) * (size_t)g);
    uint8_t* qs = (uint8_t*)malloc((size_t)g);
    for (int s = 0; s < P; ++s) {
        if (s == rank) continue;
        for (int64_t off = 0; off < tile_len; off += g) {
            int64_t base = (int64_t)s * S + tile_begin + off;
            for (int i = 0; i < g; ++i) {
                float xv = echo_ref_bf16_to_f32(x[base + i]);
                u[i] = comp ? xv + comp[base + i] : xv;
            }
            quantize_into(u, base, g, bits, quant, codes, params, qs, count);
            if (err) {
                uint16_t sh = params[2 * (base / g)], zh = params[2 * (base / g) + 1];
                for (int i = 0; i < g; ++i) {
                    float e = echo_ref_dequant(qs[i], sh, zh) - u[i];
                    err[base + i] = (flags & REF_ERR_NEGATED) ? -e : e;
                }
            }
        }
    }
    free(u); free(qs);
    return REF_OK;
}

int echo_ref_quantize_ef(const uint16_t* x, const float* comp, int64_t n, int P, int rank,
                         int64_t tile_begin, int64_t tile_len, int bits, int g,
                         uint8_t* codes, uint16_t* params, float* err, int flags)
{
    return push_impl(x, comp, n, P, rank, tile_begin, tile_len, bits, g, codes, params,
                     err, flags, NULL);
}

/* ------------------------------------------------------------------------ */
/* O3: owner reduce, for one owner.                                          */
/* [EchoCard] Fig. 2(a) (the peers' codes are decoded, the owner's copy is  */
/* added without quantization, and the total is quantized a single time     */
/* before the all-gather); Fig. 4 (four copies, three of them decoded);     */
/* abstract (the sum reveals the injected error); [Blog] "The cancellation   */
/* rule".                                                                    */
/* For every group of the owner's segment inside the tile:                   */
/*   t_j = u_owner (= f32(x) + comp) when j == owner, else Q_hat(codes_j);   */
/*   acc = t_0, then acc = acc + t_j for j = 1 .. P-1 (fp32, rank order);    */
/*   sum codes/params = Q_b(acc), written at the segment's message offset;   */
/*   own_err = Q_hat(acc) - acc (the owner's share of the injected error).   */
/* peer_codes[owner] and peer_params[owner] are not read.                    */
/* ------------------------------------------------------------------------ */
static int reduce_impl(const uint16_t* own_x, const float* own_comp,
                       const uint8_t* const* peer_codes, const uint16_t* const* peer_params,
                       int P, int owner, int64_t n, int64_t tile_begin, int64_t tile_len,
                       int bits, int g, uint8_t* sum_codes, uint16_t* sum_params,
                       float* own_err, int flags, int* count)
{
    int rc = check_shape(n, P, tile_begin, tile_len, bits, g);
    if (rc) return rc;
    if (owner < 0 || owner >= P) return REF_EINVAL;
    if ((!own_x || !sum_codes || !sum_params || !peer_codes || !peer_params) && n > 0) return REF_EINVAL;
    for (int j = 0; j < P; ++j)
        if (j != owner && n > 0 && (!peer_codes[j] || !peer_params[j])) return REF_EINVAL;
    const int quant = quant_of(flags);
    if (quant < 0) return REF_EINVAL;
    int64_t S = n / P;
    float* acc = (float*)malloc(sizeof(float) * (size_t)g);
    uint8_t* qs = (uint8_t*)malloc((size_t)g);
    for (int64_t off = 0; off < tile_len; off += g) {
        int64_t base = (int64_t)owner * S + tile_begin + off;
        int64_t grp = base / g;
        for (int i = 0; i < g; ++i) {
            float sum = 0.0f;
            for (int j = 0; j < P; ++j) {
                float t;
                if (j == owner) {
                    float xv = echo_ref_bf16_to_f32(own_x[base + i]);
                    t = own_comp ? xv + own_comp[base + i] : xv;
                } else {
                    t = echo_ref_dequant(code_at(peer_codes[j], base + i, bits),
                                         peer_params[j][2 * grp], peer_params[j][2 * grp + 1]);
                }
                sum = (j == 0) ? t : sum + t;
            }
            acc[i] = sum;
        }
        quantize_into(acc, base, g, bits, quant, sum_codes, sum_params, qs, count);
        if (own_err) {
            uint16_t sh = sum_params[2 * grp], zh = sum_params[2 * grp + 1];
            for (int i = 0; i < g; ++i) {
                float e = echo_ref_dequant(qs[i], sh, zh) - acc[i];
                own_err[base + i] = (flags & REF_ERR_NEGATED) ? -e : e;
            }
        }
    }
    free(acc); free(qs);
    return REF_OK;
}

int echo_ref_reduce_segment(const uint16_t* own_x, const float* own_comp,
                            const uint8_t* const* peer_codes, const uint16_t* const* peer_params,
                            int P, int owner, int64_t n, int64_t tile_begin, int64_t tile_len,
                            int bits, int g, uint8_t* sum_codes, uint16_t* sum_params,
                            float* own_err, int flags)
{
    return reduce_impl(own_x, own_comp, peer_codes, peer_params, P, owner, n, tile_begin,
                       tile_len, bits, g, sum_codes, sum_params, own_err, flags, NULL);
}

/* ------------------------------------------------------------------------ */
/* O4: quantized all-gather and tail decode, for one rank.                   */
/* [EchoCard] Fig. 2(a) (every rank, the owner included, decodes the same    */
/* code); Fig. 4 (after the gather all GPUs agree on the result).           */
/* For every segment and every element of the tile inside it:               */
/*   out[i] = Q_hat(sum codes)[i], as fp32 or as bfloat16 (nearest even).    */
/* ------------------------------------------------------------------------ */
int echo_ref_gather_dequant(const uint8_t* sum_codes, const uint16_t* sum_params, int64_t n,
                            int64_t tile_begin, int64_t tile_len, int P, int bits, int g,
                            void* out, int out_dtype)
{
    int rc = check_shape(n, P, tile_begin, tile_len, bits, g);
    if (rc) return rc;
    if (out_dtype != REF_OUT_F32 && out_dtype != REF_OUT_BF16) return REF_EUNSUP;
    if ((!sum_codes || !sum_params || !out) && n > 0) return REF_EINVAL;
    int64_t S = n / P;
    for (int s = 0; s < P; ++s) {
        for (int64_t off = 0; off < tile_len; ++off) {
            int64_t i = (int64_t)s * S + tile_begin + off;
            int64_t grp = i / g;
            float v = echo_ref_dequant(code_at(sum_codes, i, bits),
                                       sum_params[2 * grp], sum_params[2 * grp + 1]);
            if (out_dtype == REF_OUT_F32) ((float*)out)[i] = v;
            else ((uint16_t*)out)[i] = echo_ref_f32_to_bf16(v);
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* O5: the two-timescale compensator update.                                 */
/* [EchoCard] abstract (an error, once revealed, is returned in later        */
/* calls and cancels); [Blog] "The cancellation rule" (a two-timescale       */
/* compensator; each error is paid back in later calls).                     */
/* The pages give no equation; the reading is an error debt with a fast      */
/* fraction alpha and a slow memory M released at rate beta:                 */
/*   c' = -(alpha*e + beta*M)          (the next call's compensation)        */
/*   M' = (1-beta)*M + (1-alpha)*e                                            */
/* Each product is rounded, then the sum, then negated.  With slow == NULL   */
/* (beta == 0) the update is c' = -(alpha*e); alpha == 1 then gives classic  */
/* error feedback, c' = -e.  comp_next may alias err; slow is updated in     */
/* place.  Parity of the constants is unpinned (the pages print none); the   */
/* debt identity (accumulated error == sum of M - c) pins the form.           */
/* ------------------------------------------------------------------------ */
int echo_ref_compensate(const float* err, float* comp_next, float* slow, int64_t n,
                        float alpha, float beta)
{
    if (n < 0) return REF_ESHAPE;
    if (!(alpha > 0.0f && alpha <= 1.0f) || !(beta >= 0.0f && beta <= 1.0f)) return REF_EINVAL;
    if (alpha < 1.0f && beta == 0.0f) return REF_EINVAL;   /* the rest of the debt needs a slow memory */
    if (n == 0) return REF_OK;
    if ((slow != NULL) != (beta > 0.0f)) return REF_EINVAL; /* slow memory exactly when released */
    if (!err || !comp_next) return REF_EINVAL;
    float oma = 1.0f - alpha, omb = 1.0f - beta;
    for (int64_t i = 0; i < n; ++i) {
        float e = err[i];
        if (slow) {
            float M = slow[i];
            float a = alpha * e;
            float b = beta * M;
            comp_next[i] = -(a + b);
            float m1 = omb * M;
            float m2 = oma * e;
            slow[i] = m1 + m2;
        } else {
            float a = alpha * e;
            comp_next[i] = -a;
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* One whole all-reduce call over P ranks held in host memory: push for     */
/* every rank, reduce for every owner, decode for every rank, then the      */
/* compensator.  ef = 0: no compensation (comp/err/slow ignored).            */
/* ef = 1: u = x + comp; e goes to err (temporary arrays when err is NULL)   */
/* and echo_ref_compensate turns it into comp (and slow).  For the classic   */
/* update (alpha = 1, beta = 0) with err NULL, -e is written straight into  */
/* comp, identical to computing e and then c' = -(1*e).                     */
/* qflags selects the quantizer (0, REF_Q_NAIVE, REF_Q_SYMMETRIC, REF_Q_MSE). */
/* Instrumentation ([EchoCard] abstract and Fig. 2: at most two              */
/* quantizations per element per call), filled from counters that the push  */
/* and reduce loops above increment as they run:                             */
/*   qdepth[i] (optional, n ints): the largest number of quantizer            */
/*     applications on any path from an input element into output i, i.e.    */
/*     max_j (push count of rank j at i) + (sum-quantization count at i);     */
/*   qwork[r] (optional, P int64): elements rank r passed through the         */
/*     quantizer (its pushes plus its owner requantization).                  */
/* ------------------------------------------------------------------------ */
int echo_ref_allreduce(int P, int64_t n, int bits, int g, int ef, float alpha, float beta,
                       const uint16_t* const* x, float* const* comp, float* const* slow,
                       float* const* err, void* const* out, int out_dtype,
                       int* qdepth, int64_t* qwork, int qflags)
{
    if (quant_of(qflags) < 0 || (qflags & ~(REF_Q_NAIVE | REF_Q_SYMMETRIC | REF_Q_MSE))) return REF_EINVAL;
    int rc = check_shape(n, P, 0, 0, bits, g);
    if (rc) return rc;
    if (out_dtype != REF_OUT_F32 && out_dtype != REF_OUT_BF16) return REF_EUNSUP;
    int64_t S = n / P;
    int fused = ef && !err;
    if (ef && !comp) return REF_EINVAL;
    /* a two-timescale update requested without error buffers is defined as
     * the unfused update: errors go to temporary arrays, then the compensator */
    float** tmp_err = NULL;
    if (ef && fused && !(alpha == 1.0f && beta == 0.0f)) {
        tmp_err = (float**)calloc((size_t)P, sizeof(float*));
        for (int r = 0; r < P; ++r) tmp_err[r] = (float*)calloc((size_t)n + 1, sizeof(float));
        err = tmp_err;
        fused = 0;
    }
    int counting = qdepth || qwork;
    size_t cbytes = bits == 4 ? (size_t)(n / 2) : (size_t)n;
    size_t pwords = 2 * (size_t)(n / g);
    size_t nc = counting ? (size_t)n : 0;
    uint8_t** pc = (uint8_t**)calloc((size_t)P, sizeof(uint8_t*));
    uint16_t** pp = (uint16_t**)calloc((size_t)P, sizeof(uint16_t*));
    int** pushcnt = (int**)calloc((size_t)P, sizeof(int*));
    for (int r = 0; r < P; ++r) {
        pc[r] = (uint8_t*)calloc(cbytes + 1, 1);
        pp[r] = (uint16_t*)calloc(pwords + 1, sizeof(uint16_t));
        pushcnt[r] = counting ? (int*)calloc(nc + 1, sizeof(int)) : NULL;
    }
    uint8_t* sc = (uint8_t*)calloc(cbytes + 1, 1);
    uint16_t* sp = (uint16_t*)calloc(pwords + 1, sizeof(uint16_t));
    int* sumcnt = counting ? (int*)calloc(nc + 1, sizeof(int)) : NULL;
    int flags = (fused ? REF_ERR_NEGATED : 0) | qflags;

    for (int r = 0; r < P && !rc; ++r) {
        float* c = ef ? comp[r] : NULL;
        float* e = ef ? (fused ? comp[r] : err[r]) : NULL;
        rc = push_impl(x[r], c, n, P, r, 0, S, bits, g, pc[r], pp[r], e, flags, pushcnt[r]);
    }
    for (int o = 0; o < P && !rc; ++o) {
        float* c = ef ? comp[o] : NULL;
        float* e = ef ? (fused ? comp[o] : err[o]) : NULL;
        rc = reduce_impl(x[o], c, (const uint8_t* const*)pc, (const uint16_t* const*)pp,
                         P, o, n, 0, S, bits, g, sc, sp, e, flags, sumcnt);
    }
    for (int r = 0; r < P && !rc; ++r)
        rc = echo_ref_gather_dequant(sc, sp, n, 0, S, P, bits, g, out[r], out_dtype);
    if (ef && !fused)
        for (int r = 0; r < P && !rc; ++r)
            rc = echo_ref_compensate(err[r], comp[r], slow ? slow[r] : NULL, n, alpha, beta);
    if (!rc && qdepth) {
        for (int64_t i = 0; i < n; ++i) {
            int deepest = 0;
            for (int j = 0; j < P; ++j)
                if (pushcnt[j][i] > deepest) deepest = pushcnt[j][i];
            qdepth[i] = deepest + sumcnt[i];
        }
    }
    if (!rc && qwork) {
        for (int r = 0; r < P; ++r) {
            int64_t w = 0;
            for (int64_t i = 0; i < n; ++i) w += pushcnt[r][i];
            for (int64_t i = (int64_t)r * S; i < (int64_t)(r + 1) * S; ++i) w += sumcnt[i];
            qwork[r] = w;
        }
    }
    for (int r = 0; r < P; ++r) { free(pc[r]); free(pp[r]); free(pushcnt[r]); }
    free(pc); free(pp); free(pushcnt); free(sc); free(sp); free(sumcnt);
    if (tmp_err) {
        for (int r = 0; r < P; ++r) free(tmp_err[r]);
        free(tmp_err);
    }
    return rc;
}
