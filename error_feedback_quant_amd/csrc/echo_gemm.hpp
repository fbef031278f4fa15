// echo_gemm.hpp — gfx950 row-parallel GEMM with the all-reduce's entry pass
// (push quantization) fused into its epilogue.
//
// Method: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for LLM
// Training and Inference" (arXiv 2610.14277), paper card Fig. 2(a) (each rank
// quantizes its partial sums for the segments it does not own); PhantomByte
// article on Echo, "The cancellation rule" (the compensator is folded into
// the entry pass of the all-reduce, next to the matmul that produces the
// partial sums, without changing the computed values).
//
// One launch computes one rank's partial sums X = A W^T (A: M x K, W: N x K,
// both bf16 with K contiguous, fp32 accumulation), rounds them to bf16 and,
// instead of writing X and reading it back, runs the push step on each 128 x
// 128 output tile while it is still on chip:
//   * rows of the rank's own segment: X (bf16) is written out, for the owner
//     reduce;
//   * every other row: u = f32(x) + c, one quantization group per 128
//     consecutive columns, codes + parameters and the error (or its negation)
//     written exactly as echo_quantize_ef writes them.
// The values are those of "GEMM to bf16, then echo_quantize_ef" for the same
// accumulation; only the HBM round trip of X for the pushed segments is gone.
//
// Main loop: 256 threads (2 x 2 wavefronts, 64 x 64 outputs each) per
// 128 x 128 tile, K in steps of 64, v_mfma_f32_32x32x16_bf16 (2 x 2 per
// wavefront per 16-deep step).  Tiles of A and W are staged through LDS in two
// buffers; 16-byte chunks are XOR-swizzled by row so that the 32 rows read by
// one MFMA operand load spread over the LDS banks.  The tile order is
// XCD-aware: the 8 XCDs each take a compact block of tiles, so that the A and
// W panels a tile needs are shared in that XCD's L2.
#pragma once

#include "echo_kernels.hpp"

namespace echo {

constexpr int kGBM = 128;   // tile rows (M)
constexpr int kGBN = 128;   // tile columns (N) = one quantization group per row
constexpr int kGBK = 64;    // K per stage
constexpr int kGChunks = kGBK / 8;                     // 16-byte chunks per tile row
constexpr int kGStageBytes = (kGBM + kGBN) * kGBK * 2; // A + W, one stage
constexpr int kGXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmPushArgs {
    const uint16_t* a;      // [M][K] bf16
    const uint16_t* w;      // [N][K] bf16
    const float* comp;      // [M*N], nullable
    uint8_t* codes;         // message-shaped codes
    uint32_t* params;       // one word per group of 128
    float* err;             // [M*N], nullable, may alias comp
    uint16_t* x_out;        // [M*N] bf16: own segment (and every segment if x_all)
    int64_t M, N, K;
    int64_t seg_rows;       // rows per segment (M / P), a multiple of kGBM
    uint32_t tiles_m, tiles_n;
    int rank;
    int negate;
    int x_all;
};

// byte offset of 16-byte chunk c of tile row r in a stage buffer
__device__ __forceinline__ uint32_t gemm_swz(uint32_t r, uint32_t c)
{
    return (r * kGChunks + (c ^ (r & 7u))) * 16u;
}

// tile of linear block b: each XCD (b mod 8) takes a contiguous range of a
// grouped row-major order (groups of 8 tile rows), i.e. a compact block of
// tiles whose A and W panels stay in its L2
__device__ __forceinline__ void gemm_tile_of(uint32_t b, uint32_t tm_n, uint32_t tn_n, uint32_t& tm, uint32_t& tn)
{
    const uint32_t T = tm_n * tn_n;
    const uint32_t t = (T % kGXcds == 0) ? (b % kGXcds) * (T / kGXcds) + b / kGXcds : b;
    const uint32_t gm = 8u;
    const uint32_t group = t / (gm * tn_n);
    const uint32_t first = group * gm;
    const uint32_t rows = min(tm_n - first, gm);
    const uint32_t in = t - group * gm * tn_n;
    tm = first + in % rows;
    tn = in / rows;
}

template <int BITS, int QUANT>
__global__ __launch_bounds__(256) void gemm_push_kernel(const GemmPushArgs a)
{
    __shared__ __align__(16) uint8_t smem[2 * kGStageBytes];   // 64 KB; the epilogue reuses it
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    uint32_t tm, tn;
    gemm_tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kGBM, n0 = (int64_t)tn * kGBN;

    // global -> LDS: thread t moves chunk t % 8 of tile rows t / 8 + 32 i
    const uint32_t lc = tid & 7u, lr = tid >> 3;
    const uint16_t* ga = a.a + (m0 + lr) * a.K + 8 * lc;
    const uint16_t* gw = a.w + (n0 + lr) * a.K + 8 * lc;
    const int64_t row32 = 32 * a.K;
    u32x4 ra[4], rw[4];

    // plain loads: A and W panels are shared by the tiles of an XCD through L2
    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *(const u32x4*)(ga + i * row32 + k0);
            rw[i] = *(const u32x4*)(gw + i * row32 + k0);
        }
    };
    auto store_stage = [&](int buf) {
        uint8_t* sa = smem + buf * kGStageBytes;
        uint8_t* sw = sa + kGBM * kGBK * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)(sa + gemm_swz(lr + 32 * i, lc)) = ra[i];
            *(u32x4*)(sw + gemm_swz(lr + 32 * i, lc)) = rw[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int64_t KT = a.K / kGBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    // MFMA operand rows of this lane (A rows for i, W rows for j) and its
    // 8-element half of each 16-deep step
    const uint32_t orow = lane & 31u, ohalf = lane >> 5;
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < KT) load_stage((kt + 1) * kGBK);
        const uint8_t* sa = smem + buf * kGStageBytes;
        const uint8_t* sw = sa + kGBM * kGBK * 2;
#pragma unroll
        for (uint32_t kk = 0; kk < kGBK / 16; ++kk) {
            const uint32_t c = 2 * kk + ohalf;
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = *(const bf16x8*)(sa + gemm_swz(wm * 64 + 32 * i + orow, c));
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = *(const bf16x8*)(sw + gemm_swz(wn * 64 + 32 * j + orow, c));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: x = bf16(acc) into LDS as fp32 rows of 128, then the push
    // step on 16 rows per pass (one 16-lane DPP row per tile row)
    float* xt = (float*)smem;   // [128][128] fp32 = 64 KB
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * ohalf + (v & 3);
                const uint32_t col = wn * 64 + 32 * j + orow;
                xt[r * kGBN + col] = (float)(__bf16)acc[i][j][v];
            }
    __syncthreads();

    const int64_t seg = m0 / a.seg_rows;        // the tile lies inside one segment
    const bool own = seg == a.rank;
    const uint32_t l16 = tid & 15u;
    const bool has_comp = a.comp != nullptr;
    for (uint32_t p = 0; p < kGBM / kRowsPerBlock; ++p) {
        const uint32_t r = p * kRowsPerBlock + (tid >> 4);
        const int64_t e0 = (m0 + r) * a.N + n0 + kEPL * l16;
        float u[8];
        {
            const f32x4 x0 = *(const f32x4*)(xt + r * kGBN + kEPL * l16);
            const f32x4 x1 = *(const f32x4*)(xt + r * kGBN + kEPL * l16 + 4);
            u[0] = x0.x; u[1] = x0.y; u[2] = x0.z; u[3] = x0.w;
            u[4] = x1.x; u[5] = x1.y; u[6] = x1.z; u[7] = x1.w;
        }
        if (own || a.x_all) {
            u32x4 w;
            w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{u[0], u[1]}), bf16x2));
            w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{u[2], u[3]}), bf16x2));
            w.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{u[4], u[5]}), bf16x2));
            w.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{u[6], u[7]}), bf16x2));
            st_stream((u32x4*)(a.x_out + e0), w);
        }
        if (own) continue;                     // uniform over the block
        if (has_comp) {
            const f32x4 c0 = ld_stream((const f32x4*)(a.comp + e0));
            const f32x4 c1 = ld_stream((const f32x4*)(a.comp + e0 + 4));
            u[0] += c0.x; u[1] += c0.y; u[2] += c0.z; u[3] += c0.w;
            u[4] += c1.x; u[5] += c1.y; u[6] += c1.z; u[7] += c1.w;
        }
        float q[8];
        const QParams prm = quantize_group<BITS, QUANT, kGBN>(u, true, lane, e0, a.codes, a.params, q);
        if (a.err) {
            float e[8];
            group_error(q, prm, u, a.negate != 0, e);
            st_stream((f32x4*)(a.err + e0), f32x4{e[0], e[1], e[2], e[3]});
            st_stream((f32x4*)(a.err + e0 + 4), f32x4{e[4], e[5], e[6], e[7]});
        }
    }
}

}  // namespace echo
