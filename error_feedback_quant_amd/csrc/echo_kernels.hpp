// echo_kernels.hpp — gfx950 (CDNA4) kernels for Echo's error-compensated
// low-bit all-reduce, one simulated rank or owner per launch.
//
// Method: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for LLM
// Training and Inference" (arXiv 2610.14277), paper card Fig. 2(a), Fig. 4,
// Table 8 and abstract; PhantomByte article on Echo, "The cancellation rule".
//
// Layout and mapping (all kernels):
//  * Addressing unit: a row of 128 consecutive elements = 16 lanes x 8
//    elements, one 16-lane DPP row of a 64-lane wavefront; each lane moves its
//    8 elements with one 16-byte load (bf16).  A wavefront covers 4 rows (512
//    elements) per pass.
//  * A quantization group is GROUP = 128 (one row) or 256 (a row pair)
//    elements.  Group min/max are reduced with four row-local DPP steps
//    (quad_perm xor-1, xor-2, row_ror 4, row_ror 8) and, for 256, one
//    ds_swizzle swap-16 between the two rows: no LDS memory, no barrier.
//    min/max are exact and order-free, so the tree cannot change results.
//  * Every lane of a group derives the group's scale and zero point itself
//    (same inputs, same IEEE operations), so nothing is broadcast; the group's
//    first lane stores the 4-byte parameter word.
//  * A 256-thread block handles 16 consecutive rows per pass and U passes;
//    blockIdx.y selects the segment.  All loads of a block's U passes are
//    issued before any arithmetic to keep enough bytes in flight for HBM.
//  * Codes are packed in registers: 8 nibbles -> one dword (4-bit) or 8
//    bytes -> two dwords (8-bit), so a wavefront writes 256 / 512 contiguous
//    bytes per pass.
//  * fp32 streams (compensation, slow memory, error) move lane-contiguously
//    through a wave-private LDS slice (see Fp32Io).
// Arithmetic is IEEE fp32 with no contraction (built with -ffp-contract=off):
// the division for the scale and 1/s are correctly rounded; rint rounds half
// to even; binary16 conversion is the hardware v_cvt_f16_f32 (round to
// nearest even, binary16 subnormals kept).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace echo {

constexpr int kRow = 128;                      // addressing unit (elements)
constexpr int kEPL = 8;                        // elements per lane
constexpr int kRowLanes = kRow / kEPL;         // 16 lanes = one DPP row
constexpr int kBlock = 256;                    // 4 wavefronts of 64
constexpr int kRowsPerBlock = kBlock / kRowLanes;  // 16 rows per pass
constexpr int kMaxP = 8;

// quantizers (Table 8): the full method, its two ablations, and the full
// method with its zero point searched for the least squared error
enum Quant { kZeroAware = 0, kNaive = 1, kSymmetric = 2, kMse = 3 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers --

// Streaming accesses: every byte of the message is touched once per kernel,
// so loads and stores of the big arrays carry the non-temporal hint (measured
// faster than plain accesses on both sides).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p)
{
    return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, const T& v)
{
    __builtin_nontemporal_store(v, p);
}

// A buffer resource over `base` (raw bytes, no range limit in practice):
// loads through it take a wave-uniform base from SGPRs and a 32-bit lane
// offset.  aux = 2 sets the non-temporal bit, as the streams above.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
}

// fp32 streams (compensation in, error out) go through a wave-private LDS
// slice so that every global fp32 access is lane-contiguous (1 KB per wave
// instruction) while the arithmetic keeps 8 consecutive elements per lane.
constexpr int kWaveChunk = 4 * kRow;   // 512 elements: the 4 rows of one wave

// orders this wave's LDS accesses across lanes (no block barrier needed: the
// slice is private to the wave and the LDS executes a wave's operations in order)
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// A value moved across lanes by DPP is an integer to the compiler; a float
// min/max of it first re-canonicalizes it (one more instruction per step).
// The group reduction therefore works on integers, and the move folds into
// the integer min/max: on keys with the order of the floats (finite values;
// -0 sorts below +0) for an arbitrary range, or on the raw patterns where
// the range holds 0 (group_minmax).  The key map is its own inverse.
__device__ __forceinline__ int order_key(float f)
{
    const int b = __builtin_bit_cast(int, f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float from_order_key(int k)
{
    return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}

// Every lane has a valid source under the four patterns used here (quad_perm
// and row_ror stay inside a 16-lane row) and every lane of the wave is active
// where the group reduction runs, so bound_ctrl's zero fill never applies; it
// lets the backend fold the move into the consuming min/max.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// min and max over the lanes of a group (16 lanes, or 32 for GROUP = 256);
// every lane ends with the result.  Only the sign of a zero result can differ
// from a sequential min/max, and no quantizer's output depends on it.
//
// Where the range holds 0 (zero-aware and MSE: every lane's lo <= 0 <= hi)
// the raw bit patterns already sort and the key map is skipped: a lo is a
// zero or a negative float, whose pattern read as an unsigned integer grows
// with its magnitude (+0 is the smallest), so the smallest lo is the largest
// unsigned pattern; a hi is a zero or a positive float, and those order as
// signed integers (-0 is the smallest).  The symmetric grid reduces only hi
// (max |v|, never negative); the naive range is any pair of floats.
template <int GROUP, int QUANT>
__device__ __forceinline__ void group_minmax(float& lo, float& hi)
{
    constexpr bool kRaw = QUANT != kNaive;
    constexpr bool kLo = QUANT != kSymmetric;
    int l = kRaw ? __builtin_bit_cast(int, lo) : order_key(lo);
    int h = kRaw ? __builtin_bit_cast(int, hi) : order_key(hi);
    auto take = [&](int ol, int oh) {
        if constexpr (kLo) l = kRaw ? (int)max((uint32_t)l, (uint32_t)ol) : min(l, ol);
        h = max(h, oh);
    };
    take(kLo ? dpp_i<0xB1>(l) : 0, dpp_i<0xB1>(h));     // quad_perm [1,0,3,2]
    take(kLo ? dpp_i<0x4E>(l) : 0, dpp_i<0x4E>(h));     // quad_perm [2,3,0,1]
    take(kLo ? dpp_i<0x124>(l) : 0, dpp_i<0x124>(h));   // row_ror:4
    take(kLo ? dpp_i<0x128>(l) : 0, dpp_i<0x128>(h));   // row_ror:8
    if constexpr (GROUP == 256) {
        // rows 0<->1 and 2<->3: ds_swizzle in swap-16 mode hands every lane
        // the value of lane ^ 16 (through the LDS crossbar, no LDS memory)
        take(kLo ? __builtin_amdgcn_ds_swizzle(l, 0x401F) : 0, __builtin_amdgcn_ds_swizzle(h, 0x401F));
    }
    lo = kRaw ? __builtin_bit_cast(float, l) : from_order_key(l);
    hi = kRaw ? __builtin_bit_cast(float, h) : from_order_key(h);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float* v)
{
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Keeps an fp32 value as computed: the backend may otherwise fold an fp32
// product straight into the binary16 conversion (one v_fma_mix rounding
// instead of the fp32 rounding and then the binary16 one that the definition
// asks for).  The empty register constraint emits no instruction.
__device__ __forceinline__ float as_f32(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// binary16 scale with the clamps shared by all quantizers: a zero result
// becomes 2^-24, an infinite one 65504
__device__ __forceinline__ uint32_t scale_bits(float s32)
{
    uint32_t sb = f32_to_f16_bits(s32);
    sb = (sb == 0u) ? 1u : sb;
    sb = (sb == 0x7C00u) ? 0x7BFFu : sb;
    return sb;
}

// Group parameters (one binary16 scale and one binary16 zero point per group)
// (For an all-zero group the zero-aware, MSE and symmetric quantizers keep
// s = 2^-24 here while the word stores scale 0; the codes and errors are the
// same either way.)
struct QParams {
    float s;        // scale as fp32 (exact binary16 value)
    float inv;      // 1/s, correctly rounded
    float zf;       // zero point as fp32 (exact binary16 value)
    uint32_t word;  // binary16 scale | binary16 zero << 16
};

// Per-lane statistics feeding the parameters: zero-aware uses min/max with
// 0 included, naive plain min/max, symmetric max |v| (carried in hi).
template <int QUANT>
__device__ __forceinline__ void lane_stats(const float* u, float& lo, float& hi)
{
    if constexpr (QUANT == kZeroAware || QUANT == kMse) {
        lo = 0.0f; hi = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { lo = fminf(lo, u[i]); hi = fmaxf(hi, u[i]); }
    } else if constexpr (QUANT == kNaive) {
        lo = u[0]; hi = u[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) { lo = fminf(lo, u[i]); hi = fmaxf(hi, u[i]); }
    } else {
        lo = 0.0f; hi = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) hi = fmaxf(hi, fabsf(u[i]));
    }
}

// x / Q, correctly rounded, for x >= 0 and the quantizers' constant
// divisors Q = 15, 255 (2^b - 1) and 7, 127 (2^(b-1) - 1), without a
// division: q0 = x * RN(1/Q); the remainder x - q0 * Q is exact by fma; the
// quotient is q0 + r * RN(1/Q), rounded once.  For these four Q the result
// equals IEEE x / Q for every finite x >= 0, subnormals included (checked
// over all 2^31 inputs on the host).  An infinite x would give NaN, so the
// range is first clamped at 2^100: every quotient above 65520 rounds to the
// same binary16 infinity, which the scale clamp turns into 65504.
template <int Q>
__device__ __forceinline__ float div_by_const(float x)
{
    constexpr float kInv = 1.0f / (float)Q;
    x = fminf(x, 0x1p100f);
    const float q0 = x * kInv;
    const float r = __builtin_fmaf(-q0, (float)Q, x);
    // the fp32 quotient is kept as such: the backend would otherwise fuse the
    // last fma with the binary16 conversion (v_fma_mixlo_f16, one rounding)
    return as_f32(__builtin_fmaf(r, kInv, q0));
}

// 1/s, correctly rounded, for a binary16 scale s (2^-24 <= s <= 65504): one
// Newton step from the hardware reciprocal r0 (within one ulp of 1/s).  With
// s = M 2^k, M an integer below 2^11, the product s r0 has at most 35
// significant bits, so e = 1 - s r0 (|e| <= 2^-23) is exact; r0 + r0 e is
// (1 - e^2)/s, within 2^-46 of 1/s relative.  Unless M is a power of two,
// 1/s lies at least 2^-36 (relative) from every midpoint between fp32
// values (2^24 - (2t + 1) M 2^j is a nonzero integer), so the fma's one
// rounding gives RN(1/s); for M a power of two 1/s is a float and 2^-46 is
// far inside its rounding interval.  Three instructions instead of the
// division's eleven.
__device__ __forceinline__ float recip_scale(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, r0, 1.0f);
    return __builtin_fmaf(r0, e, r0);
}

template <int BITS, int QUANT>
__device__ __forceinline__ QParams make_params(float lo, float hi)
{
    constexpr float kQm = (float)((1 << BITS) - 1);
    QParams p;
    if constexpr (QUANT == kZeroAware || QUANT == kMse) {
        // range holds 0; integer zero point, so 0 is exactly code z
        const uint32_t sb = scale_bits(div_by_const<(1 << BITS) - 1>(hi - lo));
        const float s = f16_bits_to_f32(sb);
        const float inv = recip_scale(s);
        const float zr = __builtin_amdgcn_fmed3f(__builtin_rintf(-lo * inv), 0.0f, kQm);
        const float zf = zr + 0.0f;             // a -0 becomes +0
        // An all-zero group (hi == lo, both zeros) stores the word 0.  Its
        // quotient is +0 (div_by_const maps -0 to +0), so s is the clamped
        // 2^-24, inv 2^24 and z 0: every code is 0 and every error +0, as
        // with s = 0, and only the word needs the special case.
        p.s = s;
        p.inv = inv;
        p.zf = zf;
        p.word = (hi == lo) ? 0u : (sb | (f32_to_f16_bits(zf) << 16));
    } else if constexpr (QUANT == kNaive) {
        // plain min/max range; real-valued zero point -lo/s in binary16
        const uint32_t sb = scale_bits(div_by_const<(1 << BITS) - 1>(hi - lo));
        const float s = f16_bits_to_f32(sb);
        const float inv = recip_scale(s);
        // 0 - lo, not -lo: +0 for a zero minimum.  Pinned in a register, as
        // the backend otherwise turns (0 - lo) * inv into (-lo) * inv.
        const float nlo = as_f32(0.0f - lo);
        uint32_t zb = f32_to_f16_bits(as_f32(nlo * inv));
        zb = ((zb & 0x7FFFu) == 0x7C00u) ? ((zb & 0x8000u) | 0x7BFFu) : zb;   // overflow -> +-65504
        const bool zero = (hi == lo);          // constant group
        p.s = zero ? 0.0f : s;
        p.inv = zero ? 0.0f : inv;
        p.zf = zero ? 0.0f : f16_bits_to_f32(zb);
        p.word = zero ? 0u : (sb | (zb << 16));
    } else {
        // symmetric grid about 0, zero point fixed at the middle code
        constexpr float kMid = (float)(1 << (BITS - 1));
        const uint32_t sb = scale_bits(div_by_const<(1 << (BITS - 1)) - 1>(hi));
        const float s = f16_bits_to_f32(sb);
        const float inv = recip_scale(s);
        // an all-zero group (hi == 0) stores scale 0; with the clamped s =
        // 2^-24 its codes are kMid and its errors +0, as with s = 0
        p.s = s;
        p.inv = inv;
        p.zf = kMid;
        p.word = ((hi == 0.0f) ? 0u : sb) | (f32_to_f16_bits(kMid) << 16);
    }
    return p;
}

// code of one value as an integer-valued float
template <int BITS, int QUANT>
__device__ __forceinline__ float quant1(float u, const QParams& p)
{
    constexpr float kQm = (float)((1 << BITS) - 1);
    if constexpr (QUANT == kNaive)   // zero point added before rounding
        return __builtin_amdgcn_fmed3f(__builtin_rintf(u * p.inv + p.zf), 0.0f, kQm);
    else                             // integer zero point added after rounding
        return __builtin_amdgcn_fmed3f(__builtin_rintf(u * p.inv) + p.zf, 0.0f, kQm);
}

// Codes as binary16 values 1024 + q: v_perm_b32 puts two code bytes of b
// (bytes 0, 1 with kPermLo, bytes 2, 3 with kPermHi) under the exponent
// byte 0x64 of binary16 1024, one per 16-bit half.  A value is widened where
// it is used, which folds into a v_fma_mix operand (see decode_peer).
constexpr uint32_t kBias16 = 0x64646464u;
constexpr uint32_t kPermLo = 0x04010400u;
constexpr uint32_t kPermHi = 0x04030402u;
__device__ __forceinline__ float half_lo(uint32_t h) { return f16_bits_to_f32(h & 0xFFFFu); }
__device__ __forceinline__ float half_hi(uint32_t h) { return f16_bits_to_f32(h >> 16); }

// the 8 codes of a lane, packed (4-bit: one dword, 8-bit: two dwords)
template <int BITS>
struct Packed;
template <>
struct Packed<4> {
    uint32_t w;
    // q holds integer-valued floats in [0, 15]: the even codes go to the low
    // nibbles of bytes 0..3 and the odd codes to the high nibbles
    __device__ __forceinline__ void pack(const float* q)
    {
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ev = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * i], i, ev);
            od = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * i + 1], i, od);
        }
        w = ev | (od << 4);
    }
    // e0: element offset from `codes`' element 0 (a 32-bit lane offset from a
    // block's base, or a 64-bit message offset)
    template <typename Off>
    __device__ __forceinline__ void store(uint8_t* codes, Off e0) const
    {
        st_stream((uint32_t*)(codes + (e0 >> 1)), w);
    }
    template <typename Off>
    __device__ __forceinline__ void load(const uint8_t* codes, Off e0)
    {
        w = ld_stream((const uint32_t*)(codes + (e0 >> 1)));
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t codes, uint32_t e0)
    {
        w = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(codes, (int)(e0 >> 1), 0, 2);
    }
    __device__ __forceinline__ void unpack(float* q) const
    {
        uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
        // opaque to the optimizer, so that each code converts with one
        // v_cvt_f32_ubyte<i> instead of a bit-field extract and a convert
        asm volatile("" : "+v"(ev), "+v"(od));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[2 * i] = (float)((ev >> (8 * i)) & 0xFFu);
            q[2 * i + 1] = (float)((od >> (8 * i)) & 0xFFu);
        }
    }
    // 1024 + q of the 8 codes (even codes from the low nibbles, odd from the high)
    __device__ __forceinline__ void biased(float* qb) const
    {
        const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
        const uint32_t e0 = __builtin_amdgcn_perm(kBias16, ev, kPermLo), e1 = __builtin_amdgcn_perm(kBias16, ev, kPermHi);
        const uint32_t o0 = __builtin_amdgcn_perm(kBias16, od, kPermLo), o1 = __builtin_amdgcn_perm(kBias16, od, kPermHi);
        qb[0] = half_lo(e0); qb[2] = half_hi(e0); qb[4] = half_lo(e1); qb[6] = half_hi(e1);
        qb[1] = half_lo(o0); qb[3] = half_hi(o0); qb[5] = half_lo(o1); qb[7] = half_hi(o1);
    }
};
template <>
struct Packed<8> {
    u32x2 w;
    __device__ __forceinline__ void pack(const float* q)
    {
        uint32_t x = 0, y = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x = __builtin_amdgcn_cvt_pk_u8_f32(q[i], i, x);
            y = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + i], i, y);
        }
        w.x = x;
        w.y = y;
    }
    template <typename Off>
    __device__ __forceinline__ void store(uint8_t* codes, Off e0) const
    {
        st_stream((u32x2*)(codes + e0), w);
    }
    template <typename Off>
    __device__ __forceinline__ void load(const uint8_t* codes, Off e0)
    {
        w = ld_stream((const u32x2*)(codes + e0));
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t codes, uint32_t e0)
    {
        w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(codes, (int)e0, 0, 2));
    }
    __device__ __forceinline__ void unpack(float* q) const
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (float)((w.x >> (8 * i)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[4 + i] = (float)((w.y >> (8 * i)) & 0xFFu);
    }
    // 1024 + q of the 8 codes
    __device__ __forceinline__ void biased(float* qb) const
    {
        const uint32_t h[4] = {__builtin_amdgcn_perm(kBias16, w.x, kPermLo), __builtin_amdgcn_perm(kBias16, w.x, kPermHi),
                               __builtin_amdgcn_perm(kBias16, w.y, kPermLo), __builtin_amdgcn_perm(kBias16, w.y, kPermHi)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qb[2 * i] = half_lo(h[i]);
            qb[2 * i + 1] = half_hi(h[i]);
        }
    }
};

// decode of one parameter word: v = (q - z) * s (the same for every quantizer)
__device__ __forceinline__ void decode8(const float* q, uint32_t word, float* v)
{
    const float s = f16_bits_to_f32(word & 0xFFFFu);
    const float zf = f16_bits_to_f32(word >> 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (q[i] - zf) * s;
}

// The same decode of a peer's codes where the zero point is an integer
// (zero-aware, symmetric and MSE quantizers), from the biased codes 1024 + q:
// z <= 255 and s is a binary16 value (11 significant bits), so (1024 + z) s
// and (1024 + q) s fit in 22 bits and (q - z) s in 19, all exact in fp32;
// one fma (1024 + q) s + (-(1024 + z) s) then rounds an exact, representable
// value and gives the bits of the two-step form, +0 included when q == z.
// The naive quantizer's zero point carries a fraction, so there q - z can
// round and only the two-step form is right.
template <int BITS, int QUANT>
__device__ __forceinline__ void decode_peer(const Packed<BITS>& pk, uint32_t word, float* v)
{
    if constexpr (QUANT == kNaive) {
        float q[8];
        pk.unpack(q);
        decode8(q, word, v);
    } else {
        float qb[8];
        pk.biased(qb);
        const float s = f16_bits_to_f32(word & 0xFFFFu);
        // 1024 + z in binary16 (exact below 2048), then -(1024 + z) s; the
        // fma with 0 keeps both operands in their binary16 registers
        const _Float16 zb = __builtin_bit_cast(_Float16, (uint16_t)(word >> 16)) + (_Float16)1024.0f;
        const float c = __builtin_fmaf(-(float)zb, s, 0.0f);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(qb[i], s, c);
    }
}

// ------------------------------------------------------ zero-point search --
// The zero point of the kMse quantizer: the z in [0, Qm] that minimizes the
// group's squared error in units of s, sum_i (clamp(r_i + z, 0, Qm) - z - t_i)^2
// with t_i = u_i * (1/s) and r_i = rint(t_i) as the codes use them, the
// smallest z on ties.  z moves codes only through the clamp, so the search
// compares D(z) = sum_i (c_i - r_i)(c_i + r_i - 2 t_i), c_i = clamp(r_i, -z,
// Qm - z), which differs from the squared error by a constant.  A term is
// nonzero only for a clamped element, whose |t_i| >= 1/2 makes it a multiple
// of 2^-24 below 2^19 in magnitude; in fp64 every term and every partial sum
// is exact, so the cross-lane sum cannot depend on its order.  D is convex
// in z (every term is 0 on an interval and a convex quadratic outside it),
// so a descent from the closed-form zero point reaches the smallest
// minimizer: down while D does not increase, else up while D decreases.

// sum over the lanes of a group (16 lanes, or 32 for GROUP = 256) of an exact fp64 value
template <int GROUP>
__device__ __forceinline__ double group_sum_f64(double d)
{
    auto step = [&](auto mov) {
        const uint64_t b = __builtin_bit_cast(uint64_t, d);
        const int lo = mov((int)(uint32_t)b), hi = mov((int)(uint32_t)(b >> 32));
        d += __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    };
    step([](int v) { return dpp_i<0xB1>(v); });    // quad_perm [1,0,3,2]
    step([](int v) { return dpp_i<0x4E>(v); });    // quad_perm [2,3,0,1]
    step([](int v) { return dpp_i<0x124>(v); });   // row_ror:4
    step([](int v) { return dpp_i<0x128>(v); });   // row_ror:8
    if constexpr (GROUP == 256) step([](int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); });
    return d;
}

template <int BITS, int GROUP>
__device__ __forceinline__ double clamp_cost(const float* t, const float* r, float z)
{
    constexpr float kQm = (float)((1 << BITS) - 1);
    double d = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float c = __builtin_amdgcn_fmed3f(r[i], -z, kQm - z);
        if (c != r[i]) {
            const double cr = (double)c + (double)r[i];
            d += ((double)c - (double)r[i]) * (cr - 2.0 * (double)t[i]);
        }
    }
    return group_sum_f64<GROUP>(d);
}

template <int BITS, int GROUP>
__device__ __forceinline__ float search_zero(const float* u, float inv, float z0)
{
    constexpr float kQm = (float)((1 << BITS) - 1);
    float t[8], r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        t[i] = u[i] * inv;
        r[i] = __builtin_rintf(t[i]);
    }
    float z = z0;
    double dz = clamp_cost<BITS, GROUP>(t, r, z);
    bool down = false;
    if (z > 0.0f) {
        const double dm = clamp_cost<BITS, GROUP>(t, r, z - 1.0f);
        if (dm <= dz) { z -= 1.0f; dz = dm; down = true; }
    }
    if (down) {
        while (z > 0.0f) {
            const double dm = clamp_cost<BITS, GROUP>(t, r, z - 1.0f);
            if (!(dm <= dz)) break;
            z -= 1.0f; dz = dm;
        }
    } else {
        while (z < kQm) {
            const double dp = clamp_cost<BITS, GROUP>(t, r, z + 1.0f);
            if (!(dp < dz)) break;
            z += 1.0f; dz = dp;
        }
    }
    return z;
}

// Quantize the lane's 8 values of one group (the whole group cooperates),
// store codes and parameters, and return the codes (as integer-valued floats)
// in q and the group's parameters.  `lane` is the lane within the wavefront.
// codes, params and e0 as for Packed: e0 counts elements from the element
// that codes[0] and params[0] describe.
template <int BITS, int QUANT, int GROUP, typename Off>
__device__ __forceinline__ QParams quantize_group(const float* u, bool active, uint32_t lane, Off e0,
                                                  uint8_t* codes, uint32_t* params, float* q)
{
    float lo, hi;
    lane_stats<QUANT>(u, lo, hi);
    group_minmax<GROUP, QUANT>(lo, hi);
    QParams p = make_params<BITS, QUANT>(lo, hi);
    if constexpr (QUANT == kMse) {
        if (p.word != 0u) {         // an all-zero group keeps z = 0 (word 0)
            p.zf = search_zero<BITS, GROUP>(u, p.inv, p.zf);
            p.word = (p.word & 0xFFFFu) | (f32_to_f16_bits(p.zf) << 16);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant1<BITS, QUANT>(u[i], p);
    if (active) {
        Packed<BITS> pk;
        pk.pack(q);
        pk.store(codes, e0);
        if ((lane & (GROUP / kEPL - 1)) == 0) params[e0 / GROUP] = p.word;
    }
    return p;
}

// the quantization error (q - z) * s - u of the lane's 8 values, or its
// negation; only computed where a kernel writes it out or updates with it
__device__ __forceinline__ void group_error(const float* q, const QParams& p, const float* u, bool negate, float* e)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = (q[i] - p.zf) * p.s - u[i];
        e[i] = negate ? -v : v;
    }
}

// Addressing: a block works on rows [rb, rb + 16 U) of its tile (rows of 128
// elements).  Its loads and stores go through wave-uniform base pointers at
// the block's first element plus a 32-bit lane offset (a block spans at most
// 16 U * 128 elements), so the per-lane address needs no 64-bit arithmetic.
//
// Where the lane-contiguous fp32 accesses of a wave land: half h (0/1) of the
// wave's 512-element chunk covers rows 2h and 2h+1; lane l moves the float4 at
// offset (4 l) mod 128 of row 2h + l/32.  Rows past the tile re-read the last
// row (clamped) and are never stored.
// Row of a block, from the block's row 0.  A block spans 16 U rows (U a
// power of two) and every row it touches lies in [rb, rb + 16 U), so the
// mask changes nothing; it shows the compiler that the lane offsets stay
// small, which lets every access use a scalar base and a 32-bit lane offset.
template <int U>
__device__ __forceinline__ uint32_t block_row(uint32_t row, uint32_t rb)
{
    static_assert((U & (U - 1)) == 0, "passes per block must be a power of two");
    return (row - rb) & (uint32_t)(kRowsPerBlock * U - 1);
}

struct WaveMap {
    uint32_t rb;           // row index (within the tile) of the block's row 0
    uint32_t gw;           // row index (within the tile) of the wave's row 0
    uint32_t last;         // tile_rows - 1
    uint32_t lane;
    uint32_t mask;         // rows per block - 1 (a power of two minus one)
    __device__ __forceinline__ uint32_t row(uint32_t r) const { return gw + r; }
    // element offset from the block's first element of this lane's float4 of half h
    __device__ __forceinline__ uint32_t contig(uint32_t h) const
    {
        const uint32_t g = min(gw + 2u * h + (lane >> 5), last);
        return ((g - rb) & mask) * kRow + ((4u * lane) & (kRow - 1));
    }
    __device__ __forceinline__ bool contig_active(uint32_t h) const { return gw + 2u * h + (lane >> 5) <= last; }
};

// natural 8-float view of a lane <-> lane-contiguous float4 pairs, via LDS
__device__ __forceinline__ void stage_in(float* slice, uint32_t lane, const f32x4& h0, const f32x4& h1)
{
    *(f32x4*)(slice + 4 * lane) = h0;
    *(f32x4*)(slice + 256 + 4 * lane) = h1;
}
__device__ __forceinline__ void natural_read(const float* slice, uint32_t lane, float* v)
{
    const f32x4 a = *(const f32x4*)(slice + 8 * lane);
    const f32x4 b = *(const f32x4*)(slice + 8 * lane + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void natural_write(float* slice, uint32_t lane, const float* v)
{
    *(f32x4*)(slice + 8 * lane) = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(slice + 8 * lane + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// ------------------------------------------- fp32 stream I/O of a wavefront --
// Loads the compensation (and, for UPD, the slow memory) of U passes, and
// writes back either the error (err) or the updated compensation and slow
// memory, lane-contiguously through the wave's LDS slices.  The pointers are
// the block's bases (its first element).

template <int U, bool UPD>
struct Fp32Io {
    static constexpr int kSlices = UPD ? 2 : 1;
    static constexpr int kPassStride = (kBlock / 64) * kWaveChunk;       // floats per pass (4 waves)
    static constexpr int kLdsFloats = U * kSlices * kPassStride;

    f32x4 c0[U], c1[U], m0[U], m1[U];

    __device__ __forceinline__ static float* slice(float* lds, int k, int which, uint32_t wave)
    {
        return lds + (k * kSlices + which) * kPassStride + wave * kWaveChunk;
    }

    __device__ __forceinline__ void load(int k, const WaveMap& wm, const float* comp, const float* slow)
    {
        c0[k] = ld_stream((const f32x4*)(comp + wm.contig(0)));
        c1[k] = ld_stream((const f32x4*)(comp + wm.contig(1)));
        if (UPD) {
            m0[k] = ld_stream((const f32x4*)(slow + wm.contig(0)));
            m1[k] = ld_stream((const f32x4*)(slow + wm.contig(1)));
        }
    }

    __device__ __forceinline__ void stage(float* lds, uint32_t wave, uint32_t lane)
    {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            stage_in(slice(lds, k, 0, wave), lane, c0[k], c1[k]);
            if (UPD) stage_in(slice(lds, k, 1, wave), lane, m0[k], m1[k]);
        }
        wave_lds_fence();
    }

    // the lane's 8 natural values of pass k (which = 0: comp, 1: slow)
    __device__ __forceinline__ void natural(float* lds, int k, int which, uint32_t wave, uint32_t lane, float* v) const
    {
        natural_read(slice(lds, k, which, wave), lane, v);
    }

    // stage the 8 natural outputs of pass k for slice `which`
    __device__ __forceinline__ void put(float* lds, int k, int which, uint32_t wave, uint32_t lane, const float* v)
    {
        natural_write(slice(lds, k, which, wave), lane, v);
    }

    // after all passes: the staged outputs go out lane-contiguously
    __device__ __forceinline__ void flush(float* lds, uint32_t wave, uint32_t lane, const WaveMap* wm,
                                          float* dst0, float* dst1)
    {
        wave_lds_fence();
#pragma unroll
        for (int k = 0; k < U; ++k) {
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h) {
                if (!wm[k].contig_active(h)) continue;
                const uint32_t g = wm[k].contig(h);
                st_stream((f32x4*)(dst0 + g), *(const f32x4*)(slice(lds, k, 0, wave) + 256 * h + 4 * lane));
                if (UPD) st_stream((f32x4*)(dst1 + g), *(const f32x4*)(slice(lds, k, 1, wave) + 256 * h + 4 * lane));
            }
        }
    }
};

// ------------------------------------------------------- push (entry pass) --

// Fused two-timescale update (UPD kernels): instead of writing e, the kernel
// applies c' = -(alpha*e + beta*M), M' = (1-beta)*M + (1-alpha)*e in place on
// the compensation and slow-memory buffers -- the same IEEE operations, in the
// same order, as compensate_kernel, so the results are bit-identical.
struct UpdArgs {
    float alpha, beta, one_minus_alpha, one_minus_beta;
};

__device__ __forceinline__ void update1(const UpdArgs& a, float e, float m, float& c_out, float& m_out)
{
    const float fa = a.alpha * e;
    const float fb = a.beta * m;
    c_out = -(fa + fb);
    const float m1 = a.one_minus_beta * m;
    const float m2 = a.one_minus_alpha * e;
    m_out = m1 + m2;
}

// One launch serves one rank or several: blockIdx.z picks slot z of the
// per-rank arrays, for rank rank0 + z.
struct PushArgs {
    const uint16_t* x[kMaxP];
    const float* comp[kMaxP];   // nullable (the same for every slot)
    uint8_t* codes[kMaxP];
    uint32_t* params[kMaxP];
    float* err[kMaxP];          // nullable, may alias comp
    float* slow[kMaxP];         // UPD kernels only
    int64_t S;                  // segment length
    int64_t tile_begin;         // tile start inside each segment
    uint32_t tile_rows;         // 128-element rows per segment tile (>= 1)
    int rank0;
    int negate;
    UpdArgs upd;                // UPD kernels only: comp and slow are updated in place
};

// grid: (ceil(tile_rows / (16 U)), P - 1, ranks); blockIdx.y = index among the
// segments the rank does not own.  UPD: comp and slow are required and
// updated in place (err unused).
template <int BITS, int U, bool UPD, int QUANT, int GROUP>
__global__ __launch_bounds__(kBlock) void push_kernel(const PushArgs a)
{
    using Io = Fp32Io<U, UPD>;
    __shared__ float lds[Io::kLdsFloats];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t l16 = lane & 15u;
    const uint32_t rw = lane >> 4;                       // this lane's row in the wave
    const uint32_t z = blockIdx.z;
    const uint32_t rank = (uint32_t)a.rank0 + z;
    const uint32_t si = blockIdx.y;
    const uint32_t seg = si + (si >= rank ? 1u : 0u);
    const int64_t seg0 = (int64_t)seg * a.S + a.tile_begin;
    const uint32_t last = a.tile_rows - 1u;
    // block bases (the block's first element) and 32-bit lane offsets from them
    const uint32_t rb = blockIdx.x * (uint32_t)(kRowsPerBlock * U);
    const int64_t blk0 = seg0 + (int64_t)rb * kRow;
    const uint16_t* const x = a.x[z] + blk0;
    float* const comp = a.comp[z] ? (float*)a.comp[z] + blk0 : nullptr;
    float* const slow = UPD ? a.slow[z] + blk0 : nullptr;
    float* const err = a.err[z] ? a.err[z] + blk0 : nullptr;
    uint8_t* const codes = a.codes[z] + blk0 * BITS / 8;
    uint32_t* const params = a.params[z] + blk0 / GROUP;
    const bool has_comp = UPD || comp != nullptr;
    const bool has_out = UPD || err != nullptr;

    WaveMap wm[U];
    u32x4 xv[U];
    Io io;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        wm[k].rb = rb;
        wm[k].mask = (uint32_t)(kRowsPerBlock * U - 1);
        wm[k].gw = rb + (uint32_t)k * kRowsPerBlock + 4u * wave;
        wm[k].last = last;
        wm[k].lane = lane;
        const uint32_t o = block_row<U>(min(wm[k].row(rw), last), rb) * kRow + l16 * kEPL;
        xv[k] = ld_stream((const u32x4*)(x + o));
        if (has_comp) io.load(k, wm[k], comp, slow);
    }
    if (has_comp) io.stage(lds, wave, lane);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t graw = wm[k].row(rw);
        const bool active = graw <= last;
        const uint32_t e0 = block_row<U>(min(graw, last), rb) * kRow + l16 * kEPL;
        float u[8];
        unpack_bf16x8(xv[k], u);
        if (has_comp) {
            float c[8];
            io.natural(lds, k, 0, wave, lane, c);
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] += c[i];
        }
        float q[8], e[8];
        const QParams p = quantize_group<BITS, QUANT, GROUP>(u, active, lane, e0, codes, params, q);
        if (UPD) {
            group_error(q, p, u, false, e);
            float m[8], cn[8], mn[8];
            io.natural(lds, k, 1, wave, lane, m);
#pragma unroll
            for (int i = 0; i < 8; ++i) update1(a.upd, e[i], m[i], cn[i], mn[i]);
            io.put(lds, k, 0, wave, lane, cn);
            io.put(lds, k, 1, wave, lane, mn);
        } else if (has_out) {
            group_error(q, p, u, a.negate != 0, e);
            io.put(lds, k, 0, wave, lane, e);
        }
    }
    if (has_out) io.flush(lds, wave, lane, wm, UPD ? comp : err, slow);
}

// ------------------------------------------------------------ owner reduce --

// One launch serves one owner or several: blockIdx.y picks slot y of the
// per-owner arrays, for owner owner0 + y.
struct ReduceArgs {
    const uint16_t* x[kMaxP];       // owner's partial sums
    const float* comp[kMaxP];       // owner's compensation, nullable
    float* err[kMaxP];              // owner's error, nullable, may alias comp
    float* slow[kMaxP];             // UPD kernels only
    const uint8_t* pc[kMaxP];       // push codes of each rank (the owner's own entry unused)
    const uint32_t* pp[kMaxP];      // push parameters of each rank
    uint8_t* sc;                    // sum codes (message-shaped)
    uint32_t* sp;                   // sum parameters
    int64_t S;
    int64_t tile_begin;
    uint32_t tile_rows;
    int P;
    int owner0;
    int negate;
    UpdArgs upd;                    // UPD kernels only
};

// grid: (ceil(tile_rows / (16 U)), owners).  UPD as for push_kernel.  The
// peer loop is unrolled to MAXP (4 or 8, at least P) with uniform guards on
// the runtime P: the registers that hold the peers' codes in flight are
// sized for MAXP ranks, so a launch with P <= 4 takes the 4-rank instance.
// OWNER >= 0 fixes P = MAXP and the owner (a one-owner launch) at compile
// time: the rank-order sum is then straight-line code, without the register
// moves that merge the owner's and the peers' branches.
//
// LDS is dynamic: the launcher sizes it (at least Io::kLdsFloats floats
// whenever an fp32 stream is staged), which also sets how many blocks share a
// CU.
template <int BITS, int U, bool UPD, int QUANT, int GROUP, int MAXP, int OWNER>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(BITS == 4 && !UPD && QUANT != kMse ? 6 : 1))) void reduce_kernel(const ReduceArgs a)
{
    constexpr bool kFixed = OWNER >= 0;
    using Io = Fp32Io<U, UPD>;
    extern __shared__ float lds[];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t l16 = lane & 15u;
    const uint32_t rw = lane >> 4;
    const uint32_t y = kFixed ? 0u : blockIdx.y;
    const int owner = kFixed ? OWNER : a.owner0 + (int)y;
    const int nranks = kFixed ? MAXP : a.P;
    const int64_t seg0 = (int64_t)owner * a.S + a.tile_begin;
    const uint32_t last = a.tile_rows - 1u;
    // block bases (the block's first element) and 32-bit lane offsets from them
    const uint32_t rb = blockIdx.x * (uint32_t)(kRowsPerBlock * U);
    const int64_t blk0 = seg0 + (int64_t)rb * kRow;
    const uint16_t* const x = a.x[y] + blk0;
    float* const comp = a.comp[y] ? (float*)a.comp[y] + blk0 : nullptr;
    float* const slow = UPD ? a.slow[y] + blk0 : nullptr;
    float* const err = a.err[y] ? a.err[y] + blk0 : nullptr;
    const bool has_comp = UPD || comp != nullptr;
    const bool has_out = UPD || err != nullptr;

    WaveMap wm[U];
    u32x4 xv[U];
    Io io;
    Packed<BITS> pk[U][MAXP];
    uint32_t pw[U][MAXP];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        wm[k].rb = rb;
        wm[k].mask = (uint32_t)(kRowsPerBlock * U - 1);
        wm[k].gw = rb + (uint32_t)k * kRowsPerBlock + 4u * wave;
        wm[k].last = last;
        wm[k].lane = lane;
        const uint32_t o = block_row<U>(min(wm[k].row(rw), last), rb) * kRow + l16 * kEPL;
        xv[k] = ld_stream((const u32x4*)(x + o));
        if (has_comp) io.load(k, wm[k], comp, slow);
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            if (j < nranks && j != owner) {
                pk[k][j].load(stream_rsrc(a.pc[j] + blk0 * BITS / 8), o);
                pw[k][j] = (a.pp[j] + blk0 / GROUP)[o / GROUP];
            }
        }
    }
    if (has_comp) io.stage(lds, wave, lane);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t graw = wm[k].row(rw);
        const bool active = graw <= last;
        const uint32_t e0 = block_row<U>(min(graw, last), rb) * kRow + l16 * kEPL;
        float own[8];
        unpack_bf16x8(xv[k], own);
        if (has_comp) {
            float c[8];
            io.natural(lds, k, 0, wave, lane, c);
#pragma unroll
            for (int i = 0; i < 8; ++i) own[i] += c[i];
        }
        // fp32 sum in rank order; the owner's own term enters unquantized
        float acc[8];
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            if (j >= nranks) break;
            if (j == owner) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = (j == 0) ? own[i] : acc[i] + own[i];
            } else {
                float t[8];
                decode_peer<BITS, QUANT>(pk[k][j], pw[k][j], t);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = (j == 0) ? t[i] : acc[i] + t[i];
            }
        }
        float q[8], e[8];
        const QParams p = quantize_group<BITS, QUANT, GROUP>(acc, active, lane, e0, a.sc + blk0 * BITS / 8,
                                                             a.sp + blk0 / GROUP, q);
        if (UPD) {
            group_error(q, p, acc, false, e);
            float m[8], cn[8], mn[8];
            io.natural(lds, k, 1, wave, lane, m);
#pragma unroll
            for (int i = 0; i < 8; ++i) update1(a.upd, e[i], m[i], cn[i], mn[i]);
            io.put(lds, k, 0, wave, lane, cn);
            io.put(lds, k, 1, wave, lane, mn);
        } else if (has_out) {
            group_error(q, p, acc, a.negate != 0, e);
            io.put(lds, k, 0, wave, lane, e);
        }
    }
    if (has_out) io.flush(lds, wave, lane, wm, UPD ? comp : err, slow);
}

// ------------------------------------------------------ gather / tail decode --

// One launch serves one rank or several: blockIdx.z picks the output.
struct GatherArgs {
    const uint8_t* sc;
    const uint32_t* sp;
    void* out[kMaxP];
    int64_t S;
    int64_t tile_begin;
    uint32_t tile_rows;
};

// grid: (ceil(tile_rows / (16 U)), P, ranks); blockIdx.y = segment.  bf16
// output is already lane-contiguous (16 B per lane, 1 KB per wave); fp32
// output (32 B per lane) goes through the wave's LDS slice like the fp32
// streams of push and reduce, so that each store instruction writes 1 KB
// contiguously.
template <int BITS, bool OUT_BF16, int U, int GROUP>
__global__ __launch_bounds__(kBlock) void gather_kernel(const GatherArgs a)
{
    __shared__ float lds[OUT_BF16 ? 1 : U * (kBlock / 64) * kWaveChunk];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t l16 = threadIdx.x & 15u;
    const uint32_t row = threadIdx.x >> 4;
    const int64_t seg0 = (int64_t)blockIdx.y * a.S + a.tile_begin;
    // block bases (the block's first element) and 32-bit lane offsets from them
    const uint32_t rb = blockIdx.x * (uint32_t)(kRowsPerBlock * U);
    const int64_t blk0 = seg0 + (int64_t)rb * kRow;
    const uint32_t g0 = rb + row;
    const uint8_t* const sc = a.sc + blk0 * BITS / 8;
    const uint32_t* const sp = a.sp + blk0 / GROUP;
    void* const out = OUT_BF16 ? (void*)((uint16_t*)a.out[blockIdx.z] + blk0) : (void*)((float*)a.out[blockIdx.z] + blk0);

    Packed<BITS> pk[U];
    uint32_t pw[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t gi = min(g0 + (uint32_t)(k * kRowsPerBlock), a.tile_rows - 1u);
        const uint32_t o = block_row<U>(gi, rb) * kRow + l16 * kEPL;
        pk[k].load(sc, o);
        pw[k] = sp[o / GROUP];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t graw = g0 + (uint32_t)(k * kRowsPerBlock);
        if (graw >= a.tile_rows) continue;
        const uint32_t o = block_row<U>(graw, rb) * kRow + l16 * kEPL;
        float q[8], v[8];
        pk[k].unpack(q);
        decode8(q, pw[k], v);
        if (OUT_BF16) {
            u32x4 w;
            w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2));
            w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2));
            w.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[4], v[5]}), bf16x2));
            w.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[6], v[7]}), bf16x2));
            st_stream((u32x4*)((uint16_t*)out + o), w);
        } else {
            natural_write(lds + (k * (kBlock / 64) + wave) * kWaveChunk, lane, v);
        }
    }
    if constexpr (!OUT_BF16) {
        // rows past the tile were not decoded and are not stored
        wave_lds_fence();
#pragma unroll
        for (int k = 0; k < U; ++k) {
            WaveMap wm;
            wm.rb = rb;
            wm.mask = (uint32_t)(kRowsPerBlock * U - 1);
            wm.gw = rb + (uint32_t)k * kRowsPerBlock + 4u * wave;
            wm.last = a.tile_rows - 1u;
            wm.lane = lane;
            const float* sl = lds + (k * (kBlock / 64) + wave) * kWaveChunk;
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h) {
                if (!wm.contig_active(h)) continue;
                st_stream((f32x4*)((float*)out + wm.contig(h)), *(const f32x4*)(sl + 256 * h + 4 * lane));
            }
        }
    }
}

// ------------------------------------------------------------- compensator --

struct CompArgs {
    const float* err;
    float* comp;
    float* slow;        // nullable (beta == 0)
    int64_t n;
    UpdArgs upd;
};

// grid-stride over float4 chunks, then a scalar tail.  Without a slow memory
// (beta == 0) the update is c' = -(alpha*e).
template <bool SLOW>
__global__ __launch_bounds__(kBlock) void compensate_kernel(const CompArgs a)
{
    const int64_t n4 = a.n >> 2;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += stride) {
        const f32x4 e = ld_stream((const f32x4*)(a.err + 4 * i));
        float c[4];
        if (SLOW) {
            const f32x4 m = ld_stream((const f32x4*)(a.slow + 4 * i));
            float mo[4];
            update1(a.upd, e.x, m.x, c[0], mo[0]);
            update1(a.upd, e.y, m.y, c[1], mo[1]);
            update1(a.upd, e.z, m.z, c[2], mo[2]);
            update1(a.upd, e.w, m.w, c[3], mo[3]);
            st_stream((f32x4*)(a.slow + 4 * i), f32x4{mo[0], mo[1], mo[2], mo[3]});
        } else {
            c[0] = -(a.upd.alpha * e.x); c[1] = -(a.upd.alpha * e.y);
            c[2] = -(a.upd.alpha * e.z); c[3] = -(a.upd.alpha * e.w);
        }
        st_stream((f32x4*)(a.comp + 4 * i), f32x4{c[0], c[1], c[2], c[3]});
    }
    if (blockIdx.x == 0) {
        const int64_t i = 4 * n4 + threadIdx.x;
        if (i < a.n) {
            const float e = a.err[i];
            if (SLOW) {
                float c, mo;
                update1(a.upd, e, a.slow[i], c, mo);
                a.slow[i] = mo;
                a.comp[i] = c;
            } else {
                a.comp[i] = -(a.upd.alpha * e);
            }
        }
    }
}

// -------------------------------------------------------- one-pass call --
// A whole call in one launch, for small messages, where a launch per stage
// costs more than the stage's work (a single call of 64 x 1024 per rank is
// bound by launch latency).  The stages work group by group, so each
// wavefront takes 512 elements of one segment (four groups of 128, or two of
// 256) through all of them in the call's order: every other rank's push of
// those elements (codes and parameters into that rank's push buffer), the
// owner's reduce (the peers' codes read back from their push buffers, the
// fp32 sum in rank order, the sum quantized once), and every rank's tail
// (each rank reads the sum codes back and decodes them into its output).
// Every rank's reads and writes are its own, as in the per-stage kernels; a
// workgroup barrier between stages makes one lane's stores (the group's
// parameters) visible to the others.
struct OnePassArgs {
    const uint16_t* x[kMaxP];
    float* comp[kMaxP];     // compensation (null with feedback off); UPD rewrites it
    float* err[kMaxP];      // error output (comp itself when negate), or null
    float* slow[kMaxP];     // slow memory, UPD only
    void* out[kMaxP];
    uint8_t* pc[kMaxP];     // each rank's push codes and parameters, message-shaped
    uint32_t* pp[kMaxP];
    uint8_t* sc;            // sum codes and parameters, message-shaped
    uint32_t* sp;
    UpdArgs upd;
    int64_t S;
    uint32_t seg_chunks;    // 512-element chunks per segment: ceil(S / 512)
    int P;
    int negate;
};

constexpr uint32_t kChunkElems = 64 * kEPL;   // one wavefront's 512 elements

// The whole call in one launch, for small messages.  Block b takes chunk
// b mod seg_chunks of segment (owner) o = b / seg_chunks, and its four
// wavefronts split the ranks: wavefront w serves ranks w and w + 4.  Each
// wavefront pushes its ranks' copies of the chunk (every rank but the
// owner), the owner's wavefront (o mod 4) reduces the chunk, and each
// wavefront decodes the sum into its ranks' outputs.  Workgroup barriers
// between the stages make the codes and parameters one wavefront stored
// visible to the others.  Every rank still writes and reads its own buffers.
template <int BITS, int QUANT, int GROUP, bool UPD, bool OUT_BF16>
__global__ __launch_bounds__(kBlock) void onepass_kernel(const OnePassArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const int wave = (int)(threadIdx.x >> 6);
    const int o = (int)(blockIdx.x / a.seg_chunks);          // the grid holds exactly P * seg_chunks blocks
    const int64_t so = (int64_t)(blockIdx.x - (uint32_t)o * a.seg_chunks) * kChunkElems + lane * kEPL;
    const bool active = so < a.S;
    // an inactive lane reads the segment's last 8 elements; segments hold
    // whole groups, so its group is inactive as a whole and stores nothing
    const int64_t e0 = (int64_t)o * a.S + (active ? so : a.S - kEPL);
    const bool reducer = wave == (o & 3);

    // one rank's inputs at this lane's 8 elements: x, and the compensation
    // and slow memory when they are read
    struct In {
        u32x4 x;
        f32x4 c0, c1, m0, m1;
    };
    auto load_in = [&](int r) {
        In v;
        v.x = *(const u32x4*)(a.x[r] + e0);
        v.c0 = v.c1 = v.m0 = v.m1 = f32x4{};
        if (a.comp[r]) { v.c0 = *(const f32x4*)(a.comp[r] + e0); v.c1 = *(const f32x4*)(a.comp[r] + e0 + 4); }
        if (UPD) { v.m0 = *(const f32x4*)(a.slow[r] + e0); v.m1 = *(const f32x4*)(a.slow[r] + e0 + 4); }
        return v;
    };
    auto to_u = [&](int r, const In& v, float* u, float* m) {
        unpack_bf16x8(v.x, u);
        if (a.comp[r]) {
            u[0] += v.c0.x; u[1] += v.c0.y; u[2] += v.c0.z; u[3] += v.c0.w;
            u[4] += v.c1.x; u[5] += v.c1.y; u[6] += v.c1.z; u[7] += v.c1.w;
        }
        m[0] = v.m0.x; m[1] = v.m0.y; m[2] = v.m0.z; m[3] = v.m0.w;
        m[4] = v.m1.x; m[5] = v.m1.y; m[6] = v.m1.z; m[7] = v.m1.w;
    };
    // the error of rank r's quantization: the compensator's new state
    // (UPD), or the error (negated for the next call's compensation)
    auto finish = [&](int r, const float* q, const QParams& p, const float* u, const float* m) {
        if (!active) return;
        float e[8];
        if (UPD) {
            float cn[8], mn[8];
            group_error(q, p, u, false, e);
#pragma unroll
            for (int i = 0; i < 8; ++i) update1(a.upd, e[i], m[i], cn[i], mn[i]);
            *(f32x4*)(a.comp[r] + e0) = f32x4{cn[0], cn[1], cn[2], cn[3]};
            *(f32x4*)(a.comp[r] + e0 + 4) = f32x4{cn[4], cn[5], cn[6], cn[7]};
            *(f32x4*)(a.slow[r] + e0) = f32x4{mn[0], mn[1], mn[2], mn[3]};
            *(f32x4*)(a.slow[r] + e0 + 4) = f32x4{mn[4], mn[5], mn[6], mn[7]};
        } else if (a.err[r]) {
            group_error(q, p, u, a.negate != 0, e);
            *(f32x4*)(a.err[r] + e0) = f32x4{e[0], e[1], e[2], e[3]};
            *(f32x4*)(a.err[r] + e0 + 4) = f32x4{e[4], e[5], e[6], e[7]};
        }
    };

    // push: this wavefront's ranks other than the owner quantize their copy
    // of the chunk (both ranks' inputs requested first); the owner's
    // wavefront also requests the owner's inputs for the reduce
    const int r0 = wave, r1 = wave + 4;
    const bool push0 = r0 < a.P && r0 != o, push1 = r1 < a.P && r1 != o;
    In in0 = {}, in1 = {}, own_in = {};
    if (push0) in0 = load_in(r0);
    if (push1) in1 = load_in(r1);
    if (reducer) own_in = load_in(o);
    if (push0) {
        float u[8], m[8], q[8];
        to_u(r0, in0, u, m);
        const QParams p = quantize_group<BITS, QUANT, GROUP>(u, active, lane, e0, a.pc[r0], a.pp[r0], q);
        finish(r0, q, p, u, m);
    }
    if (push1) {
        float u[8], m[8], q[8];
        to_u(r1, in1, u, m);
        const QParams p = quantize_group<BITS, QUANT, GROUP>(u, active, lane, e0, a.pc[r1], a.pp[r1], q);
        finish(r1, q, p, u, m);
    }
    __syncthreads();

    // owner reduce: fp32 sum in rank order, the owner's term unquantized;
    // every peer's codes are requested before the sum starts
    if (reducer) {
        Packed<BITS> pk[kMaxP];
        uint32_t pw[kMaxP];
#pragma unroll
        for (int j = 0; j < kMaxP; ++j) {
            if (j < a.P && j != o) {
                pk[j].load(a.pc[j], e0);
                pw[j] = a.pp[j][e0 / GROUP];
            }
        }
        float own[8], m[8], acc[8], q[8];
        to_u(o, own_in, own, m);
#pragma unroll
        for (int j = 0; j < kMaxP; ++j) {
            if (j >= a.P) break;
            if (j == o) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = (j == 0) ? own[i] : acc[i] + own[i];
            } else {
                float t[8];
                decode_peer<BITS, QUANT>(pk[j], pw[j], t);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = (j == 0) ? t[i] : acc[i] + t[i];
            }
        }
        const QParams p = quantize_group<BITS, QUANT, GROUP>(acc, active, lane, e0, a.sc, a.sp, q);
        finish(o, q, p, acc, m);
    }
    __syncthreads();

    // tail: each of this wavefront's ranks reads the sum codes (both reads
    // issued before the first output is stored) and decodes them.  The
    // reads are identical, so a compiler memory barrier after each keeps
    // them from being merged into one: each rank reads for itself, as in the
    // per-stage tail.
    Packed<BITS> sk[2];
    uint32_t sw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (wave + 4 * k < a.P) {
            sk[k].load(a.sc, e0);
            sw[k] = a.sp[e0 / GROUP];
            asm volatile("" ::: "memory");
        }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = wave + 4 * k;
        if (r >= a.P) break;
        float q[8], v[8];
        sk[k].unpack(q);
        decode8(q, sw[k], v);
        if (!active) continue;
        if (OUT_BF16) {
            u32x4 w;
            w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2));
            w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2));
            w.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[4], v[5]}), bf16x2));
            w.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[6], v[7]}), bf16x2));
            *(u32x4*)((uint16_t*)a.out[r] + e0) = w;
        } else {
            *(f32x4*)((float*)a.out[r] + e0) = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4*)((float*)a.out[r] + e0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
    }
}

}  // namespace echo
