// echo_gemm.hpp — gfx950 row-parallel GEMM with the all-reduce's entry pass
// (push quantization) fused into its epilogue.
//
// Method: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for LLM
// Training and Inference" (arXiv 2610.14277), paper card Fig. 2(a) (each rank
// quantizes its partial sums for the segments owned by others); PhantomByte
// article on Echo, "The cancellation rule" (adding the compensation moves
// into the all-reduce's first pass, beside the matmul whose partial sums it
// sends, and the results stay the same).
//
// One launch computes one rank's partial sums X = A W^T (A: M x K, W: N x K,
// both bf16 with K contiguous, fp32 accumulation), rounds them to bf16 and,
// instead of writing X and reading it back, runs the push step on each 256 x
// 256 output tile while it is still on chip:
//   * rows of the rank's own segment: X (bf16) is written out, for the owner
//     reduce;
//   * every other row: u = f32(x) + c, one quantization group per 128
//     consecutive columns, codes + parameters and the error (or its negation)
//     written exactly as echo_quantize_ef writes them.
// The values are those of "GEMM to bf16, then echo_quantize_ef" for the same
// accumulation; only the HBM round trip of X for the pushed segments is gone.
//
// Main loop: 512 threads per 256 x 256 tile as 2 x 4 wavefronts of 128 x 64
// outputs (4 x 2 tiles of v_mfma_f32_32x32x16_bf16, 128 accumulators per
// lane), K in stages of 64, so each 16-deep step reads 6 operand fragments
// from LDS for 8 MFMAs.  Stages are filled with buffer_load_dwordx4 ... lds
// through a buffer resource over the tile's A (or W) panel: one instruction
// of a wavefront moves 8 rows x 128 B and lane i lands at the wave-uniform
// LDS base + 16 i (row i / 8, physical chunk i % 8), so the lane fetches the
// logical chunk that the XOR swizzle puts there.  (The global_load_lds form
// of the same load, a FLAT-encoded instruction, slowed the MFMA loop by
// about 13 %, and the compiler counts it as an LDS event, which turns every
// LDS wait in the loop into a wait for zero.)  Two 64 KB stages, 128 KB of
// LDS; the epilogue reuses it for the bf16 tile.  The tile order is
// XCD-aware: the 8 XCDs each take a compact block of tiles, so that the A and
// W panels a tile needs are shared in that XCD's L2.
#pragma once

#include "echo_kernels.hpp"

namespace echo {

constexpr int kGTile = 256;                            // tile rows = tile columns
constexpr int kGHalf = 128;                            // columns of one 16-lane row in the epilogue
constexpr int kGBK = 64;                               // K per stage
constexpr int kGThreads = 512;                         // 8 wavefronts
constexpr int kGChunks = kGBK / 8;                     // 16-byte chunks per stage row
constexpr int kGStageBytes = 2 * kGTile * kGBK * 2;    // A + W, one stage (64 KB)
constexpr int kGXcds = 8;
constexpr int64_t kGMaxK = (int64_t(1) << 22) - kGBK;  // a 256-row panel stays below 2^31 bytes

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
    int64_t seg_rows;       // rows per segment (M / P), a multiple of 16
    uint32_t tiles_m, tiles_n;
    int rank;
    int negate;
    int x_all;
};

// Byte offset of 16-byte chunk c of tile row r in a stage buffer.  A row is
// 128 B, so without a swizzle every row of an operand fragment (one row per
// lane) would start on the same bank.  The chunk is XORed with
// (r mod 8) ^ ((r / 8) mod 2): any 8 consecutive rows then use 8 distinct
// chunk positions, and so do the 8 even and the 8 odd rows of any aligned
// group of 16, which keeps a 16-lane phase of ds_read_b128 on distinct banks
// whether the LDS serves 8 lanes x 16 B or 16 lanes x 16 B per clock.
__device__ __forceinline__ uint32_t gemm_swz_key(uint32_t r)
{
    return (r & 7u) ^ ((r >> 3) & 1u);
}
__device__ __forceinline__ uint32_t gemm_swz(uint32_t r, uint32_t c)
{
    return (r * kGChunks + (c ^ gemm_swz_key(r))) * 16u;
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

// buffer resource over `rows` rows of a [.][K] bf16 matrix starting at p:
// stride 0, so the record count is in bytes; dword 3 selects 32-bit raw
// data.  A lane's offset is below rows*K*2 < 2^31 (K < 2^22 is checked on
// the host), and an offset past the record count would read 0, not fault.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_panel_rsrc(const uint16_t* p, int64_t rows, int64_t K)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(rows * K * 2), 0x00020000);
}

__device__ __forceinline__ void gemm_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint8_t* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, byte_off, 0, 0, 0);
}

template <int BITS, int QUANT, int GROUP>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm256_push_kernel(const GemmPushArgs a)
{
    __shared__ __align__(16) uint8_t smem[2 * kGStageBytes];   // 128 KB
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t wm = wave >> 2, wn = wave & 3u;
    uint32_t tm, tn;
    gemm_tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kGTile, n0 = (int64_t)tn * kGTile;

    // this lane's share of a stage: rows wave*8 + 64 i + lane/8 (i = 0..3) of
    // A and of W, lane % 8 is the physical chunk, so it fetches the logical
    // chunk (lane % 8) ^ key(row); key(row) is the same for every i
    const uint32_t lrow = lane >> 3;
    const uint32_t lchunk = (lane & 7u) ^ gemm_swz_key(wave * 8 + lrow);
    const __amdgpu_buffer_rsrc_t ra = gemm_panel_rsrc(a.a + m0 * a.K, kGTile, a.K);
    const __amdgpu_buffer_rsrc_t rw = gemm_panel_rsrc(a.w + n0 * a.K, kGTile, a.K);
    const uint32_t lane_off = (uint32_t)(((wave * 8 + lrow) * a.K + 8 * lchunk) * 2);
    const uint32_t row64 = (uint32_t)(64 * a.K * 2);
    auto issue = [&](int buf, int64_t k0) {
        uint8_t* sa = smem + buf * kGStageBytes;
        uint8_t* sw = sa + kGTile * kGBK * 2;
        const uint32_t off = lane_off + (uint32_t)(k0 * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t r0 = wave * 8 + 64 * i;
            gemm_load_lds16(ra, off + i * row64, sa + r0 * (kGChunks * 16));
            gemm_load_lds16(rw, off + i * row64, sw + r0 * (kGChunks * 16));
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int64_t KT = a.K / kGBK;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t orow = lane & 31u, ohalf = lane >> 5;
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < KT) issue(buf ^ 1, (kt + 1) * kGBK);
        const uint8_t* sa = smem + buf * kGStageBytes;
        const uint8_t* sw = sa + kGTile * kGBK * 2;
#pragma unroll
        for (uint32_t kk = 0; kk < kGBK / 16; ++kk) {
            const uint32_t c = 2 * kk + ohalf;
            bf16x8 fa[4], fb[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(sa + gemm_swz(wm * 128 + 32 * i + orow, c));
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = *(const bf16x8*)(sw + gemm_swz(wn * 64 + 32 * j + orow, c));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        // the backend's interleaving of LDS reads and MFMAs for small-tile
        // GEMMs (strategy 1): -3 to -7 % per call against its default order
        __builtin_amdgcn_iglp_opt(1);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's share of the next stage has landed
        __syncthreads();
    }

    // ---- epilogue: x = bf16(acc) as a [256][256] tile in LDS, then the push
    // step on 16 rows (32 groups) per pass
    uint16_t* xt = (uint16_t*)smem;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t r = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * ohalf + (v & 3);
                const uint32_t col = wn * 64 + 32 * j + orow;
                xt[r * kGTile + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
            }
    __syncthreads();

    const uint32_t l16 = tid & 15u;
    const uint32_t gcol = ((tid >> 4) & 1u) * kGHalf + kEPL * l16;
    const bool has_comp = a.comp != nullptr;
    for (uint32_t p = 0; p < kGTile / 16; ++p) {
        const uint32_t r = p * 16 + (tid >> 5);
        const int64_t grow = m0 + r;
        const bool own = grow / a.seg_rows == a.rank;   // uniform: segments hold whole 16-row passes
        const int64_t e0 = grow * a.N + n0 + gcol;
        const u32x4 xw = *(const u32x4*)(xt + r * kGTile + gcol);
        if (own || a.x_all) st_stream((u32x4*)(a.x_out + e0), xw);
        if (own) continue;
        float u[8];
        unpack_bf16x8(xw, u);
        // the fp32 streams here go as two float4 per lane at a 32-byte stride,
        // so each 128-byte line is touched by two instructions: plain cache
        // policy lets the second one hit the line the first brought in (with
        // the non-temporal hint the call measured 7 % slower)
        if (has_comp) {
            const f32x4 c0 = *(const f32x4*)(a.comp + e0);
            const f32x4 c1 = *(const f32x4*)(a.comp + e0 + 4);
            u[0] += c0.x; u[1] += c0.y; u[2] += c0.z; u[3] += c0.w;
            u[4] += c1.x; u[5] += c1.y; u[6] += c1.z; u[7] += c1.w;
        }
        float q[8];
        const QParams prm = quantize_group<BITS, QUANT, GROUP>(u, true, lane, e0, a.codes, a.params, q);
        if (a.err) {
            float e[8];
            group_error(q, prm, u, a.negate != 0, e);
            *(f32x4*)(a.err + e0) = f32x4{e[0], e[1], e[2], e[3]};
            *(f32x4*)(a.err + e0 + 4) = f32x4{e[4], e[5], e[6], e[7]};
        }
    }
}


}  // namespace echo
