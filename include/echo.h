/*
 * echo.h — C ABI of libecho: the per-call hot path of Echo's
 * error-compensated low-bit all-reduce, on one MI355X (gfx950).
 *
 * Sources: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for
 * LLM Training and Inference" (arXiv 2610.14277), paper card: abstract,
 * Fig. 1, Fig. 2(a)/(b), Table 8, appendix Fig. 4; and the PhantomByte article
 * "Your All-Reduce Is 4x Overpriced: Echo's 4-Bit Error-Feedback Trick for
 * Tensor-Parallel Training", section "The cancellation rule".
 *
 * The problem: P tensor-parallel ranks each hold a partial sum x_r of n
 * bfloat16 values; the all-reduce returns sum_r x_r to every rank.  Echo
 * splits the message into P equal contiguous segments, segment s owned by
 * rank s.  Each rank adds its compensation, quantizes the P-1 segments that
 * belong to other ranks and sends those codes to the segments' owners; an
 * owner decodes the P-1 copies it received, adds its own copy (never
 * quantized) in fp32 and quantizes the total a single time; every rank
 * decodes that same code.  The errors the sum reveals feed a
 * compensator whose output is added at the next call.
 *
 * Here the P ranks are P sets of buffers on one GPU: "push" and "gather"
 * move no bytes between devices; each simulated rank still performs its own
 * reads and writes.
 *
 * Conventions for every call:
 *  - Pointers marked (device) are device memory, (host) are host memory.  The
 *    caller owns every buffer and keeps it alive until the enqueued work is
 *    done.  The library never allocates or frees device memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue;
 *    they do not synchronize.
 *  - Arguments are checked on the host before anything is enqueued; a call
 *    that returns an error other than ECHO_EHIP has enqueued nothing.
 *  - Data pointers must be 16-byte aligned (ECHO_EALIGN otherwise).
 *  - Messages: n elements per rank, 0 <= n <= 2^34, n a multiple of P*group.
 *    S = n / P is the segment length.  Tiles are element ranges *inside each
 *    segment*: [tile_begin, tile_begin + tile_len), both multiples of group,
 *    tile_begin + tile_len <= S.  (0, S) means whole segments.
 *  - bits is 4 or 8; group is 128 or 256 (ECHO_EUNSUP otherwise).  P is 1..8.
 *  - Codes: unsigned, 0 .. 2^bits - 1.  bits = 4: element i's code is in byte
 *    i/2, the low nibble when i is even; bits = 8: byte i.  Code arrays are
 *    message-shaped: n*bits/8 bytes, segment s at byte offset s*S*bits/8.
 *  - Per-group parameters: one echo_qparam per group of `group` consecutive
 *    message elements (n/group entries, message-shaped): IEEE binary16 scale s
 *    and binary16 zero point z.  Decoding is v = (q - z) * s in fp32: exact
 *    when z is an integer (the zero-aware quantizer and the symmetric-grid
 *    ablation); the naive-zero-point ablation's z carries a fraction, so
 *    there q - z may round.
 *  - Non-finite inputs give unspecified (but memory-safe) results.
 *  - Thread safety: calls are reentrant.  Calls that write the same buffers
 *    must be ordered by the caller.
 */
#ifndef ECHO_H
#define ECHO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum echo_status {
    ECHO_OK = 0,
    ECHO_EINVAL = -1, /* null required pointer, bad P/rank/owner/constants */
    ECHO_EALIGN = -2, /* a data pointer is not 16-byte aligned */
    ECHO_EUNSUP = -3, /* bits not 4/8, group not 128/256, unknown output dtype */
    ECHO_ESHAPE = -4, /* n or tile not a valid multiple / out of range */
    ECHO_EHIP = -5,   /* a HIP launch or runtime call failed; see echo_last_hip_error */
    ECHO_ETOOBIG = -6 /* echo_allreduce_sim_noalloc: the message needs more workspace than
                         echo_noalloc_scratch_bytes() */
};

enum echo_out_dtype { ECHO_OUT_F32 = 0, ECHO_OUT_BF16 = 1 };

/* flags for echo_quantize_ef / echo_reduce_segment / echo_gemm_quantize_ef
 * (and echo_sim_args.quant for the two quantizer bits) */
enum {
    ECHO_ERR_NEGATED = 1,      /* write -e (the next call's compensation) instead of e */
    ECHO_QUANT_NAIVE = 2,      /* Table 8 ablation: naive zero point */
    ECHO_QUANT_SYMMETRIC = 4,  /* Table 8 ablation: symmetric grid */
    ECHO_X_ALL = 8,            /* echo_gemm_quantize_ef only: write x for every segment */
    ECHO_QUANT_MSE = 16        /* full method with its zero point searched for the least squared error */
};

#define ECHO_MAX_P 8

typedef struct echo_qparam {
    uint16_t scale_f16; /* binary16 bits of s */
    uint16_t zero_f16;  /* binary16 bits of the zero point z (an integer except
                           for the naive-zero-point ablation) */
} echo_qparam;

/*
 * echo_quantize_ef — entry pass and push quantization for one rank.
 * Paper card Fig. 2(a) and Fig. 4 (each rank quantizes the segments it does
 * not own, keeps its own); article "The cancellation rule" (the compensation
 * is added in the entry pass; parameters are half precision per group);
 * Table 8 (zero-aware asymmetric quantizer, g = 128).
 *
 * For every segment s != rank and every group of the tile inside it:
 *   u = float(x) + comp            (u = float(x) when comp is NULL)
 *   lo = min(0, min u), hi = max(0, max u)
 *   s = binary16((hi - lo) / (2^bits - 1)), round to nearest even; a zero
 *       result becomes 2^-24 and an infinite one 65504; hi == lo (an all-zero
 *       group) gives s = +0, z = 0 and all codes 0
 *   z = clamp(rint(-lo * (1/s)), 0, 2^bits - 1)
 *   q = clamp(rint(u * (1/s)) + z, 0, 2^bits - 1)
 *   err = (q - z) * s - u          (or its negation with ECHO_ERR_NEGATED)
 * All float operations are single IEEE fp32 operations (no contraction);
 * 1/s and the scale division are correctly rounded; rint rounds half to even.
 *
 * The quantizer above is the full method's (zero-aware asymmetric, Table 8).
 * The flag bits select one of Table 8's ablations instead (same parameter
 * word, same decode v = (q - z) * s):
 *   ECHO_QUANT_NAIVE      lo = min u, hi = max u (no widening to 0);
 *                         s as above; z = binary16((0 - lo) * (1/s)), a real
 *                         value (+0 when the minimum is a zero of either sign;
 *                         an overflow becomes +-65504); q = clamp(rint(u *
 *                         (1/s) + z), 0, Qm); hi == lo gives s = +0, z = 0,
 *                         codes 0.
 *   ECHO_QUANT_SYMMETRIC  a = max |u|; s = binary16(a / (2^(bits-1) - 1))
 *                         with the clamps above; z = 2^(bits-1);
 *                         q = clamp(rint(u * (1/s)) + z, 0, Qm); a == 0 gives
 *                         s = +0 and all codes z.
 * ECHO_QUANT_MSE keeps the full method's s and codes rule and searches the
 * integer zero point instead of taking the closed form: the z in [0, Qm]
 * minimizing sum_i (clamp(rint(t_i) + z, 0, Qm) - z - t_i)^2 with
 * t_i = u_i * (1/s), the smallest z on ties (it differs from the closed form
 * only where the rounded codes span more than 2^bits levels).
 * Setting more than one quantizer bit is ECHO_EINVAL.
 *
 *   x_bf16 (device, in)   bfloat16 bits [n] of this rank's partial sums
 *   comp   (device, in)   fp32 [n] compensation, or NULL (no feedback)
 *   codes  (device, out)  this rank's push codes (message-shaped)
 *   params (device, out)  this rank's push parameters (message-shaped)
 *   err    (device, out)  fp32 [n] revealed error, or NULL.  May alias comp:
 *                         each element is read before it is overwritten.
 * Elements of segment `rank` and outside the tile are not touched.
 */
int echo_quantize_ef(const uint16_t* x_bf16, const float* comp, int64_t n, int P, int rank,
                     int64_t tile_begin, int64_t tile_len, int bits, int group,
                     uint8_t* codes, echo_qparam* params, float* err, int flags, void* stream);

/*
 * echo_reduce_segment — the owner's high-precision sum and single
 * requantization.  Paper card Fig. 2(a) (decode of the peers' codes, the
 * owner's own copy added without quantization, one quantization of the total
 * before the all-gather), Fig. 4, abstract (the sum reveals each injected
 * error).
 *
 * For every group of segment `owner` inside the tile:
 *   t_j = float(own_x) + own_comp       when j == owner (no quantization)
 *   t_j = (q_j - z_j) * s_j              from peer j's push codes otherwise
 *   acc = t_0 + t_1 + ... + t_{P-1}      in fp32, left to right in rank order
 *   sum codes / params = Q(acc)          (the quantizer of echo_quantize_ef)
 *   own_err = (q - z) * s - acc          (or its negation with ECHO_ERR_NEGATED)
 *
 *   own_x_bf16, own_comp (device, in)  the owner's x and comp (comp nullable)
 *   peer_codes, peer_params (host arrays of P device pointers, in)
 *                                      each rank's push codes/params, made by
 *                                      echo_quantize_ef with the same
 *                                      quantizer flag; entry [owner] is not
 *                                      read and may be NULL
 *   sum_codes, sum_params (device, out) message-shaped; only segment `owner`
 *                                      inside the tile is written
 *   own_err (device, out, nullable)    fp32 [n]; may alias own_comp
 */
int echo_reduce_segment(const uint16_t* own_x_bf16, const float* own_comp,
                        const uint8_t* const* peer_codes, const echo_qparam* const* peer_params,
                        int P, int owner, int64_t n, int64_t tile_begin, int64_t tile_len,
                        int bits, int group, uint8_t* sum_codes, echo_qparam* sum_params,
                        float* own_err, int flags, void* stream);

/*
 * echo_gather_dequant — quantized all-gather and tail decode for one rank.
 * Paper card Fig. 2(a) (every rank, the owner included, decodes the same
 * code, so all outputs are identical), Fig. 4.
 *
 * For every segment and every element of the tile inside it:
 *   out[i] = (q_i - z) * s   as fp32, or rounded to bfloat16 (nearest even)
 *
 *   sum_codes, sum_params (device, in)  the owners' sum codes (message-shaped)
 *   out (device, out)  fp32 [n] (ECHO_OUT_F32) or bfloat16 bits [n] (ECHO_OUT_BF16)
 */
int echo_gather_dequant(const uint8_t* sum_codes, const echo_qparam* sum_params, int64_t n,
                        int64_t tile_begin, int64_t tile_len, int P, int bits, int group,
                        void* out, int out_dtype, void* stream);

/*
 * echo_compensate — the two-timescale compensator update, elementwise.
 * Paper card abstract (a revealed error is returned in a later call, which
 * cancels it); article "The cancellation rule" (a two-timescale compensator,
 * updated off the critical path while the next matmul runs).  The
 * pages give no equation; the reading is an error debt with a fast fraction
 * alpha returned at the next call and a slow memory M released at rate beta:
 *   comp_next = -(alpha*e + beta*M)
 *   M         = (1-beta)*M + (1-alpha)*e
 * (products rounded, then the sum, then the negation).  With slow == NULL
 * (beta must be 0): comp_next = -(alpha*e); alpha = 1 is classic error feedback.
 *
 *   err (device, in)        fp32 [n] revealed errors of the last call
 *   comp_next (device, out) fp32 [n]; may alias err
 *   slow (device, in/out)   fp32 [n] slow memory M, or NULL
 * Constraints: 0 < alpha <= 1, 0 <= beta <= 1, beta > 0 iff slow != NULL,
 * alpha < 1 requires beta > 0 (ECHO_EINVAL otherwise).
 */
int echo_compensate(const float* err, float* comp_next, float* slow, int64_t n,
                    float alpha, float beta, void* stream);

/*
 * echo_gemm_quantize_ef — one rank's row-parallel matmul with the entry pass
 * and push quantization fused into its epilogue.  Paper card Fig. 2(a) (each
 * rank quantizes its partial sums for the segments owned by other ranks);
 * article "The cancellation rule" (the compensator is folded into the entry
 * pass, beside the matmul, and the results stay as they were).
 *
 * Computes this rank's partial sums x = bf16(A W^T), i.e.
 *   x[m*N + j] = bfloat16(sum_k A[m][k] * W[j][k])   (fp32 accumulation,
 *                                                     round to nearest even)
 * and then does exactly what echo_quantize_ef(x, comp, M*N, P, rank, 0,
 * M*N/P, bits, group, codes, params, err, flags) does, without writing x for
 * the pushed segments: the message is x in row-major order, segment s is
 * rows [s*M/P, (s+1)*M/P), one group is `group` consecutive columns of a row.
 * The rank's own segment of x is written to x_out (bf16), for the owner
 * reduce; with ECHO_X_ALL, x_out receives every segment.  The fp32 sum order
 * is the kernel's own (K in steps of 16, MFMA accumulation), so x matches a
 * separate GEMM only up to fp32 rounding of the sum; everything after x is
 * bit-exact.
 * Performance: measured at a Llama-3-8B MLP down projection at TP = 4
 * (M = N = 4096, K = 3584), this call is usually slower than a library
 * matmul (hipBLASLt) followed by echo_quantize_ef, by about 3 to 10 %
 * depending on the GPU (on one it was 3 % faster): its matmul core is
 * slower than the library's, and its epilogue (the push) cannot overlap the
 * matrix cores when every CU holds one output tile.  Prefer the separate
 * pair where speed matters.
 *
 *   a_bf16 (device, in)   bfloat16 bits [M][K], row-major (K contiguous)
 *   w_bf16 (device, in)   bfloat16 bits [N][K], row-major (K contiguous): the
 *                         weight of y = a w^T
 *   comp   (device, in)   fp32 [M*N] compensation, or NULL (no feedback)
 *   codes, params, err    as for echo_quantize_ef (message-shaped; err may
 *                         alias comp or be NULL)
 *   x_out  (device, out)  bfloat16 bits [M*N]; rows of segment `rank` (all
 *                         rows with ECHO_X_ALL) are written, others untouched
 * Constraints: group 128 or 256 (ECHO_EUNSUP otherwise); M and N multiples of
 * 256, K a positive multiple of 64 below 2^22, M a multiple of P with
 * M/P a multiple of 16, M*N <= 2^34 (ECHO_ESHAPE); M or N of 0 enqueues nothing.  Flags: those
 * of echo_quantize_ef and ECHO_X_ALL.
 * Pointers as for echo_quantize_ef (codes and params may be NULL when P == 1,
 * as nothing is pushed), plus a_bf16, w_bf16 and x_out required.
 */
int echo_gemm_quantize_ef(const uint16_t* a_bf16, const uint16_t* w_bf16, int64_t M, int64_t N,
                          int64_t K, const float* comp, int P, int rank, int bits, int group,
                          uint8_t* codes, echo_qparam* params, float* err, uint16_t* x_out,
                          int flags, void* stream);

/*
 * echo_allreduce_sim — one whole call for P simulated ranks: push, owner
 * reduce, gather, tail decode and (if on) the compensator update, with each
 * segment split into `tiles` tiles whose stages overlap on several streams.
 * Paper card Fig. 2(b) (the stages of successive tiles overlap in time;
 * events order the work inside a GPU).
 *
 * Stage k of every tile runs on streams[k % nstreams] (push 0, reduce 1,
 * tail 2, compensator 3); events order tile t's reduce after its pushes and
 * its tail after its reduce.  Tile t's tail is enqueued after tile t+1's
 * push, so with two streams (the tail sharing the push's stream) the reduce
 * of a tile still runs beside the push of the next.  The gather moves no bytes here: the tail reads
 * the owners' sum codes directly.  All streams start after the work already
 * enqueued on streams[0], and streams[0] waits for all of them before the
 * call returns, so the caller may treat the call as enqueued on streams[0].
 * streams may be NULL (null stream only).  Results do not depend on tiles or
 * streams (bit for bit).
 *
 * One tile and at most 2^20 elements per rank: the whole call is one launch
 * on streams[0] (each block takes one 512-element chunk of one segment, and
 * its four wavefronts split the ranks: they push their ranks' copies, the
 * owner's wavefront reduces, and each decodes the sum into its ranks'
 * outputs; every stage still writes and reads its own buffers), followed by
 * echo_compensate when err[r] are given.
 * Such a call is bound by launch latency, and one launch instead of one per
 * stage cuts it; the results are the same bit for bit.
 *
 * Feedback (ef = 1): every rank's comp is added at the entry pass.  With
 * err[r] == NULL for every rank the update is fused into the push and reduce
 * kernels: they write -e straight into comp (alpha = 1, beta = 0, classic
 * error feedback) or apply the two-timescale update to comp and slow in place
 * (beta > 0).  Both are bit-identical to writing e and running
 * echo_compensate, which is what happens when err[r] are given: err[r]
 * receives e, and echo_compensate turns it into comp[r] (and slow[r]) after
 * the call's last reduce.
 *
 * The workspace (device, caller-allocated, >= echo_allreduce_sim_workspace_bytes)
 * holds every rank's push codes/params and the sum codes/params.
 */
typedef struct echo_sim_args {
    int P;          /* ranks, 1..8 */
    int bits;       /* 4 or 8 */
    int group;      /* 128 or 256 */
    int tiles;      /* tiles per segment, >= 1 (capped at S/group and at 4096) */
    int out_dtype;  /* ECHO_OUT_F32 or ECHO_OUT_BF16 */
    int ef;         /* 0: no compensation; 1: compensation on */
    int quant;      /* 0 (zero-aware), ECHO_QUANT_NAIVE, ECHO_QUANT_SYMMETRIC or ECHO_QUANT_MSE */
    float alpha;    /* fast fraction, 0 < alpha <= 1 */
    float beta;     /* slow release rate, 0 <= beta <= 1 */
    int64_t n;      /* elements per rank */
    const uint16_t* x[ECHO_MAX_P]; /* (device) bf16 bits [n] per rank */
    float* comp[ECHO_MAX_P];       /* (device) fp32 [n] per rank (ef = 1) */
    float* slow[ECHO_MAX_P];       /* (device) fp32 [n] per rank (beta > 0) */
    float* err[ECHO_MAX_P];        /* (device) fp32 [n] per rank, or NULL (update fused) */
    void* out[ECHO_MAX_P];         /* (device) [n] fp32 or bf16 bits per rank */
    void* workspace;               /* (device) */
    size_t workspace_bytes;
} echo_sim_args;

/* Bytes of workspace echo_allreduce_sim needs; 0 for invalid arguments. */
size_t echo_allreduce_sim_workspace_bytes(int P, int64_t n, int bits, int group);

/* streams: host array of nstreams hipStream_t handles, or NULL. */
int echo_allreduce_sim(const echo_sim_args* args, void* const* streams, int nstreams);

/*
 * echo_allreduce_sim_noalloc — echo_allreduce_sim for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: the push and sum
 * codes go to a static device array of echo_noalloc_scratch_bytes() bytes
 * (64 MiB) that the library holds on every device it runs on until the
 * process ends; args->workspace and args->workspace_bytes are ignored.  Every
 * stage runs on `stream` (hipStream_t, NULL = the null stream), tile after
 * tile, so no events are created either; results are those of
 * echo_allreduce_sim, bit for bit.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.
 *
 * Errors: those of echo_allreduce_sim (except the workspace checks), and
 * ECHO_ETOOBIG, with nothing enqueued, when
 * echo_allreduce_sim_workspace_bytes(P, n, bits, group) exceeds the array:
 * at 4-bit codes and g = 128 that is n above about 25 million elements per
 * rank for P = 4.  Calls on one device share the array: calls that overlap
 * in time on one device race and must be ordered by the caller (for example
 * by issuing them on one stream).  Nothing in the array needs clearing
 * between calls: every byte a call reads was written earlier in that call.
 */
int echo_allreduce_sim_noalloc(const echo_sim_args* args, void* stream);

/* Size in bytes of the static scratch array of echo_allreduce_sim_noalloc. */
size_t echo_noalloc_scratch_bytes(void);

/* Static description of a status code. */
const char* echo_status_str(int status);

/* The hipError_t behind the calling thread's last ECHO_EHIP (0 if none). */
int echo_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ECHO_H */
