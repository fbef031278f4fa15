// echo_api.hip — host side of libecho: argument checks, kernel launches and
// the tile-staged multi-stream schedule of one simulated all-reduce call (a
// small call asked for in one tile runs as a single launch instead).
//
// The calls follow the problem statement of "Echo: Error-Compensated 4-Bit
// Tensor-Parallel Communication for LLM Training and Inference" (arXiv
// 2610.14277): Fig. 2(a) (push, owner reduce, quantized all-gather, decode),
// Fig. 2(b) (the push, reduce, gather and tail of successive tiles overlap,
// with events ordering the work inside one GPU), and the PhantomByte article's
// "The cancellation rule" (compensator fused into the entry pass, update run
// beside the next matmul).  Semantics, layouts and error behaviour are
// specified in include/echo.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "echo.h"
#include "echo_gemm.hpp"
#include "echo_kernels.hpp"

namespace {

thread_local int t_last_hip_error = 0;

constexpr int64_t kMaxN = int64_t(1) << 34;
// passes of 16 groups per block (each DPP row handles this many groups),
// per kernel; chosen by measurement at the 1 GiB workload
constexpr int kUPush = 2;
constexpr int kURed = 2;
constexpr int kUGath = 2;
constexpr size_t kReduceCompLds = 32 * 1024;
// tiles per segment in one simulated call: results do not depend on the
// tiling, and each tile takes two events from the pool
constexpr int64_t kMaxTiles = 4096;
// below this many push blocks per rank launch, one launch serves all ranks
constexpr int64_t kBatchBelowBlocks = 4096;
// one-tile calls of at most this many elements per rank run as one launch (onepass_kernel)
constexpr int64_t kOnePassMaxElems = int64_t(1) << 20;

int hip_fail(hipError_t e)
{
    t_last_hip_error = (int)e;
    return ECHO_EHIP;
}

int check_launch()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? ECHO_OK : hip_fail(e);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t code_bytes(int64_t n, int bits) { return bits == 4 ? n / 2 : n; }

int check_common(int64_t n, int P, int64_t tile_begin, int64_t tile_len, int bits, int group)
{
    if (P < 1 || P > ECHO_MAX_P) return ECHO_EINVAL;
    if (bits != 4 && bits != 8) return ECHO_EUNSUP;
    if (group != 128 && group != 256) return ECHO_EUNSUP;
    if (n < 0 || n > kMaxN || n % ((int64_t)P * group) != 0) return ECHO_ESHAPE;
    const int64_t S = n / P;
    // tile_begin + tile_len could overflow for huge arguments: compare by subtraction
    if (tile_begin < 0 || tile_len < 0 || tile_begin % group || tile_len % group || tile_begin > S ||
        tile_len > S - tile_begin)
        return ECHO_ESHAPE;
    return ECHO_OK;
}

// alpha, beta ranges; alpha < 1 needs a slow memory to keep the rest of the debt
int check_alpha_beta(float alpha, float beta)
{
    if (!(alpha > 0.0f && alpha <= 1.0f)) return ECHO_EINVAL;
    if (!(beta >= 0.0f && beta <= 1.0f)) return ECHO_EINVAL;
    if (alpha < 1.0f && beta == 0.0f) return ECHO_EINVAL;
    return ECHO_OK;
}

// the slow memory is given exactly when it is released (beta > 0)
int check_slow(float beta, bool has_slow) { return has_slow == (beta > 0.0f) ? ECHO_OK : ECHO_EINVAL; }

unsigned blocks_for(uint32_t tile_rows, int u)
{
    return (tile_rows + echo::kRowsPerBlock * u - 1) / (echo::kRowsPerBlock * u);
}

// quantizer selected by the flag bits (-1: more than one asked for)
int quant_of(int flags)
{
    const bool naive = flags & ECHO_QUANT_NAIVE, sym = flags & ECHO_QUANT_SYMMETRIC, mse = flags & ECHO_QUANT_MSE;
    if ((int)naive + (int)sym + (int)mse > 1) return -1;
    return naive ? echo::kNaive : (sym ? echo::kSymmetric : (mse ? echo::kMse : echo::kZeroAware));
}

constexpr int kQuantFlags = ECHO_QUANT_NAIVE | ECHO_QUANT_SYMMETRIC | ECHO_QUANT_MSE;
constexpr int kKnownFlags = ECHO_ERR_NEGATED | kQuantFlags;

// Runtime (bits, update, quantizer, group) -> kernel template instance.
template <template <int, bool, int, int> class L, typename A>
void dispatch(int bits, bool upd, int quant, int group, const A& a, dim3 grid, hipStream_t st)
{
#define ECHO_D3(B, UP, Q)                                             \
    if (group == 128) L<B, UP, Q, 128>::go(a, grid, st);              \
    else L<B, UP, Q, 256>::go(a, grid, st);
#define ECHO_D2(B, UP)                                                \
    if (quant == echo::kNaive) { ECHO_D3(B, UP, echo::kNaive) }       \
    else if (quant == echo::kSymmetric) { ECHO_D3(B, UP, echo::kSymmetric) } \
    else if (quant == echo::kMse) { ECHO_D3(B, UP, echo::kMse) }      \
    else { ECHO_D3(B, UP, echo::kZeroAware) }
#define ECHO_D1(B)                                                    \
    if (upd) { ECHO_D2(B, true) } else { ECHO_D2(B, false) }
    if (bits == 4) { ECHO_D1(4) } else { ECHO_D1(8) }
#undef ECHO_D1
#undef ECHO_D2
#undef ECHO_D3
}

template <int B, bool UP, int Q, int G>
struct PushL {
    static void go(const echo::PushArgs& a, dim3 grid, hipStream_t st)
    {
        hipLaunchKernelGGL((echo::push_kernel<B, kUPush, UP, Q, G>), grid, dim3(echo::kBlock), 0, st, a);
    }
};
template <int B, bool UP, int Q, int G>
struct ReduceL {
    static void go(const echo::ReduceArgs& a, dim3 grid, hipStream_t st)
    {
        // LDS: the staging slices when an fp32 stream is read or written, and
        // at least kReduceCompLds when the compensation is read.  32 KB holds
        // residency to five blocks per CU (160 KB of LDS): with the
        // compensation stream that measured faster than the six that the
        // registers allow, while the reduce without it wants every wave it
        // can get and takes no LDS at all.  Every slot of a launch has the
        // same streams, so slot 0 decides.
        using Io = echo::Fp32Io<kURed, UP>;
        const bool comp = a.comp[0] != nullptr, err = a.err[0] != nullptr;
        size_t lds = (UP || comp || err) ? Io::kLdsFloats * sizeof(float) : 0;
        if ((UP || comp) && lds < kReduceCompLds) lds = kReduceCompLds;
        // one owner at P = 4: the instance with that owner's sum order fixed
        const int fixed = (a.P == 4 && grid.y == 1) ? a.owner0 : -1;
#define ECHO_RED(MAXP, OWNER) \
    hipLaunchKernelGGL((echo::reduce_kernel<B, kURed, UP, Q, G, MAXP, OWNER>), grid, dim3(echo::kBlock), lds, st, a)
        switch (fixed) {
        case 0: ECHO_RED(4, 0); break;
        case 1: ECHO_RED(4, 1); break;
        case 2: ECHO_RED(4, 2); break;
        case 3: ECHO_RED(4, 3); break;
        default:
            if (a.P <= 4) ECHO_RED(4, -1);
            else ECHO_RED(8, -1);
        }
#undef ECHO_RED
    }
};

// ---------------------------------------------------------------- launchers --
// Each assumes validated arguments and tile_len > 0.  One launch covers
// `slots` ranks (or owners): slot k of the pointer arrays belongs to rank
// (owner) rank0 + k.

echo::UpdArgs make_upd(float alpha, float beta)
{
    echo::UpdArgs u;
    u.alpha = alpha;
    u.beta = beta;
    u.one_minus_alpha = 1.0f - alpha;
    u.one_minus_beta = 1.0f - beta;
    return u;
}

// The scalar fields of a push launch over the tile [tb, tb + tl) of every segment.
echo::PushArgs push_args(int64_t n, int P, int64_t tb, int64_t tl, int rank0, int flags)
{
    echo::PushArgs a;
    std::memset(&a, 0, sizeof(a));
    a.S = n / P; a.tile_begin = tb; a.tile_rows = (uint32_t)(tl / echo::kRow);
    a.rank0 = rank0; a.negate = (flags & ECHO_ERR_NEGATED) ? 1 : 0;
    return a;
}

// upd: the fused two-timescale update (comp and slow in place, err unused)
int launch_push(const echo::PushArgs& a, int P, int slots, int bits, int group, int flags, bool upd,
                hipStream_t st)
{
    if (P == 1) return ECHO_OK;   // a single rank owns everything: nothing to push
    dim3 grid(blocks_for(a.tile_rows, kUPush), (unsigned)(P - 1), (unsigned)slots);
    dispatch<PushL>(bits, upd, quant_of(flags), group, a, grid, st);
    return check_launch();
}

echo::ReduceArgs reduce_args(int64_t n, int P, int64_t tb, int64_t tl, int owner0, int flags)
{
    echo::ReduceArgs a;
    std::memset(&a, 0, sizeof(a));
    a.S = n / P; a.tile_begin = tb; a.tile_rows = (uint32_t)(tl / echo::kRow);
    a.P = P; a.owner0 = owner0; a.negate = (flags & ECHO_ERR_NEGATED) ? 1 : 0;
    return a;
}

int launch_reduce(const echo::ReduceArgs& a, int slots, int bits, int group, int flags, bool upd, hipStream_t st)
{
    dim3 grid(blocks_for(a.tile_rows, kURed), (unsigned)slots);
    dispatch<ReduceL>(bits, upd, quant_of(flags), group, a, grid, st);
    return check_launch();
}

template <int B, bool BF, int G>
void gather_go(const echo::GatherArgs& a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((echo::gather_kernel<B, BF, kUGath, G>), grid, dim3(echo::kBlock), 0, st, a);
}

echo::GatherArgs gather_args(const uint8_t* sc, const echo_qparam* sp, int64_t n, int P, int64_t tb, int64_t tl)
{
    echo::GatherArgs a;
    std::memset(&a, 0, sizeof(a));
    a.sc = sc; a.sp = (const uint32_t*)sp;
    a.S = n / P; a.tile_begin = tb; a.tile_rows = (uint32_t)(tl / echo::kRow);
    return a;
}

int launch_gather(const echo::GatherArgs& a, int P, int slots, int bits, int group, int out_dtype, hipStream_t st)
{
    dim3 grid(blocks_for(a.tile_rows, kUGath), (unsigned)P, (unsigned)slots);
    const bool bf = out_dtype == ECHO_OUT_BF16;
    if (bits == 4) {
        if (group == 128) { if (bf) gather_go<4, true, 128>(a, grid, st); else gather_go<4, false, 128>(a, grid, st); }
        else { if (bf) gather_go<4, true, 256>(a, grid, st); else gather_go<4, false, 256>(a, grid, st); }
    } else {
        if (group == 128) { if (bf) gather_go<8, true, 128>(a, grid, st); else gather_go<8, false, 128>(a, grid, st); }
        else { if (bf) gather_go<8, true, 256>(a, grid, st); else gather_go<8, false, 256>(a, grid, st); }
    }
    return check_launch();
}

template <int B, int Q, int G, bool UP, bool BF>
void onepass_go(const echo::OnePassArgs& a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((echo::onepass_kernel<B, Q, G, UP, BF>), grid, dim3(echo::kBlock), 0, st, a);
}

// the whole call in one launch: one block per 512-element chunk of every segment
int launch_onepass(const echo::OnePassArgs& a, int bits, int group, int quant, bool upd, bool bf16, hipStream_t st)
{
    const dim3 grid((unsigned)((uint64_t)a.P * a.seg_chunks));
#define ECHO_O4(B, Q, G, UP) \
    if (bf16) onepass_go<B, Q, G, UP, true>(a, grid, st); else onepass_go<B, Q, G, UP, false>(a, grid, st);
#define ECHO_O3(B, Q, G) \
    if (upd) { ECHO_O4(B, Q, G, true) } else { ECHO_O4(B, Q, G, false) }
#define ECHO_O2(B, Q) \
    if (group == 128) { ECHO_O3(B, Q, 128) } else { ECHO_O3(B, Q, 256) }
#define ECHO_O1(B)                                                          \
    if (quant == echo::kNaive) { ECHO_O2(B, echo::kNaive) }                 \
    else if (quant == echo::kSymmetric) { ECHO_O2(B, echo::kSymmetric) }    \
    else if (quant == echo::kMse) { ECHO_O2(B, echo::kMse) }                \
    else { ECHO_O2(B, echo::kZeroAware) }
    if (bits == 4) { ECHO_O1(4) } else { ECHO_O1(8) }
#undef ECHO_O1
#undef ECHO_O2
#undef ECHO_O3
#undef ECHO_O4
    return check_launch();
}

int launch_compensate(const float* err, float* comp, float* slow, int64_t n, float alpha, float beta,
                      hipStream_t st)
{
    if (n == 0) return ECHO_OK;
    echo::CompArgs a;
    a.err = err; a.comp = comp; a.slow = slow; a.n = n;
    a.upd = make_upd(alpha, beta);
    int64_t chunks = (n + 3) / 4;
    int64_t blocks = (chunks + echo::kBlock - 1) / echo::kBlock;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (slow) hipLaunchKernelGGL((echo::compensate_kernel<true>), dim3((unsigned)blocks), dim3(echo::kBlock), 0, st, a);
    else hipLaunchKernelGGL((echo::compensate_kernel<false>), dim3((unsigned)blocks), dim3(echo::kBlock), 0, st, a);
    return check_launch();
}

// ------------------------------------------------------------- event pool --
// Cross-stream ordering inside one call uses events from a per-thread,
// per-device pool (created once, reused by later calls of the same thread).

// The pool is not destroyed at thread exit: the HIP runtime may already be
// torn down by then, and the process releases the events anyway.
struct EventPool {
    int device = -1;
    std::vector<hipEvent_t> ev;
};
thread_local EventPool t_pool;

int get_events(size_t count, hipEvent_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (t_pool.device != dev) {
        for (hipEvent_t ev : t_pool.ev) (void)hipEventDestroy(ev);
        t_pool.ev.clear();
        t_pool.device = dev;
    }
    while (t_pool.ev.size() < count) {
        hipEvent_t ev;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e);
        t_pool.ev.push_back(ev);
    }
    *out = t_pool.ev.data();
    return ECHO_OK;
}

struct SimLayout {
    int64_t cb, pbytes, cb_al, pb_al;
    size_t total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

SimLayout sim_layout(int P, int64_t n, int bits, int group)
{
    SimLayout L;
    L.cb = code_bytes(n, bits);
    L.pbytes = (n / group) * (int64_t)sizeof(echo_qparam);
    L.cb_al = (int64_t)align256((size_t)L.cb);
    L.pb_al = (int64_t)align256((size_t)L.pbytes);
    L.total = (size_t)(P + 1) * (size_t)(L.cb_al + L.pb_al);
    return L;
}

// ------------------------------------------------------------ static scratch --
// The allocation-free call keeps the push and sum codes in this array.  In
// host code `scratch` names a host-side stand-in, not device memory: kernels
// get the device address that hipGetSymbolAddress returns, taken once per
// device (each device holds its own copy of the array until the process ends).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_device(uint8_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return ECHO_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!p) return ECHO_EHIP;
        g_scratch_ptr[dev] = (uint8_t*)p;
    }
    *out = g_scratch_ptr[dev];
    return ECHO_OK;
}

}  // namespace

// ======================================================================= ABI

extern "C" {

const char* echo_status_str(int status)
{
    switch (status) {
    case ECHO_OK: return "ok";
    case ECHO_EINVAL: return "invalid argument";
    case ECHO_EALIGN: return "pointer not 16-byte aligned";
    case ECHO_EUNSUP: return "unsupported bits, group or output dtype";
    case ECHO_ESHAPE: return "invalid message or tile shape";
    case ECHO_EHIP: return "HIP runtime error";
    case ECHO_ETOOBIG: return "message needs more workspace than the static scratch of the allocation-free call";
    default: return "unknown status";
    }
}

int echo_last_hip_error(void) { return t_last_hip_error; }

int echo_quantize_ef(const uint16_t* x_bf16, const float* comp, int64_t n, int P, int rank,
                     int64_t tile_begin, int64_t tile_len, int bits, int group, uint8_t* codes,
                     echo_qparam* params, float* err, int flags, void* stream)
{
    int rc = check_common(n, P, tile_begin, tile_len, bits, group);
    if (rc) return rc;
    if (rank < 0 || rank >= P) return ECHO_EINVAL;
    if ((flags & ~kKnownFlags) || quant_of(flags) < 0) return ECHO_EINVAL;
    if (n == 0 || tile_len == 0 || P == 1) return ECHO_OK;
    if (!x_bf16 || !codes || !params) return ECHO_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(params) ||
        (comp && !aligned16(comp)) || (err && !aligned16(err)))
        return ECHO_EALIGN;
    echo::PushArgs a = push_args(n, P, tile_begin, tile_len, rank, flags);
    a.x[0] = x_bf16; a.comp[0] = comp; a.codes[0] = codes; a.params[0] = (uint32_t*)params; a.err[0] = err;
    return launch_push(a, P, 1, bits, group, flags, false, (hipStream_t)stream);
}

int echo_gemm_quantize_ef(const uint16_t* a_bf16, const uint16_t* w_bf16, int64_t M, int64_t N,
                          int64_t K, const float* comp, int P, int rank, int bits, int group,
                          uint8_t* codes, echo_qparam* params, float* err, uint16_t* x_out,
                          int flags, void* stream)
{
    if (P < 1 || P > ECHO_MAX_P) return ECHO_EINVAL;
    if (bits != 4 && bits != 8) return ECHO_EUNSUP;
    if (group != 128 && group != 256) return ECHO_EUNSUP;   // one group = 128 or 256 columns of a row
    if (M < 0 || N < 0 || K < 0) return ECHO_ESHAPE;
    if (N % echo::kGTile || M % echo::kGTile || M % P || (M / P) % 16) return ECHO_ESHAPE;
    if (M != 0 && N != 0 && (K == 0 || K % echo::kGBK || K > echo::kGMaxK)) return ECHO_ESHAPE;
    if (N != 0 && M > kMaxN / N) return ECHO_ESHAPE;
    if (rank < 0 || rank >= P) return ECHO_EINVAL;
    if ((flags & ~(kKnownFlags | ECHO_X_ALL)) || quant_of(flags) < 0) return ECHO_EINVAL;
    if (M == 0 || N == 0) return ECHO_OK;
    // with P == 1 nothing is pushed and codes / params may be NULL
    if (!a_bf16 || !w_bf16 || !x_out || (P > 1 && (!codes || !params))) return ECHO_EINVAL;
    if (!aligned16(a_bf16) || !aligned16(w_bf16) || (codes && !aligned16(codes)) ||
        (params && !aligned16(params)) || !aligned16(x_out) || (comp && !aligned16(comp)) ||
        (err && !aligned16(err)))
        return ECHO_EALIGN;
    echo::GemmPushArgs g;
    g.a = a_bf16; g.w = w_bf16; g.comp = comp; g.codes = codes; g.params = (uint32_t*)params;
    g.err = err; g.x_out = x_out;
    g.M = M; g.N = N; g.K = K; g.seg_rows = M / P;
    g.rank = rank; g.negate = (flags & ECHO_ERR_NEGATED) ? 1 : 0; g.x_all = (flags & ECHO_X_ALL) ? 1 : 0;
    const hipStream_t st = (hipStream_t)stream;
    const int q = quant_of(flags);
    g.tiles_m = (uint32_t)(M / echo::kGTile); g.tiles_n = (uint32_t)(N / echo::kGTile);
    const dim3 grid(g.tiles_m * g.tiles_n);
#define ECHO_GEMM_GO(B, Q)                                                                                  \
    do {                                                                                                    \
        if (group == 128)                                                                                   \
            hipLaunchKernelGGL((echo::gemm256_push_kernel<B, Q, 128>), grid, dim3(echo::kGThreads), 0, st, g); \
        else                                                                                                \
            hipLaunchKernelGGL((echo::gemm256_push_kernel<B, Q, 256>), grid, dim3(echo::kGThreads), 0, st, g); \
    } while (0)
    if (bits == 4) {
        if (q == echo::kZeroAware) ECHO_GEMM_GO(4, echo::kZeroAware);
        else if (q == echo::kNaive) ECHO_GEMM_GO(4, echo::kNaive);
        else if (q == echo::kMse) ECHO_GEMM_GO(4, echo::kMse);
        else ECHO_GEMM_GO(4, echo::kSymmetric);
    } else {
        if (q == echo::kZeroAware) ECHO_GEMM_GO(8, echo::kZeroAware);
        else if (q == echo::kNaive) ECHO_GEMM_GO(8, echo::kNaive);
        else if (q == echo::kMse) ECHO_GEMM_GO(8, echo::kMse);
        else ECHO_GEMM_GO(8, echo::kSymmetric);
    }
#undef ECHO_GEMM_GO
    return check_launch();
}

int echo_reduce_segment(const uint16_t* own_x_bf16, const float* own_comp,
                        const uint8_t* const* peer_codes, const echo_qparam* const* peer_params, int P,
                        int owner, int64_t n, int64_t tile_begin, int64_t tile_len, int bits, int group,
                        uint8_t* sum_codes, echo_qparam* sum_params, float* own_err, int flags,
                        void* stream)
{
    int rc = check_common(n, P, tile_begin, tile_len, bits, group);
    if (rc) return rc;
    if (owner < 0 || owner >= P) return ECHO_EINVAL;
    if ((flags & ~kKnownFlags) || quant_of(flags) < 0) return ECHO_EINVAL;
    if (n == 0 || tile_len == 0) return ECHO_OK;
    if (!own_x_bf16 || !sum_codes || !sum_params) return ECHO_EINVAL;
    if (P > 1 && (!peer_codes || !peer_params)) return ECHO_EINVAL;
    for (int j = 0; j < P; ++j) {
        if (j == owner) continue;
        if (!peer_codes[j] || !peer_params[j]) return ECHO_EINVAL;
        if (!aligned16(peer_codes[j]) || !aligned16(peer_params[j])) return ECHO_EALIGN;
    }
    if (!aligned16(own_x_bf16) || !aligned16(sum_codes) || !aligned16(sum_params) ||
        (own_comp && !aligned16(own_comp)) || (own_err && !aligned16(own_err)))
        return ECHO_EALIGN;
    echo::ReduceArgs a = reduce_args(n, P, tile_begin, tile_len, owner, flags);
    a.x[0] = own_x_bf16; a.comp[0] = own_comp; a.err[0] = own_err;
    for (int j = 0; j < P; ++j) {
        a.pc[j] = j == owner ? nullptr : peer_codes[j];
        a.pp[j] = j == owner ? nullptr : (const uint32_t*)peer_params[j];
    }
    a.sc = sum_codes; a.sp = (uint32_t*)sum_params;
    return launch_reduce(a, 1, bits, group, flags, false, (hipStream_t)stream);
}

int echo_gather_dequant(const uint8_t* sum_codes, const echo_qparam* sum_params, int64_t n,
                        int64_t tile_begin, int64_t tile_len, int P, int bits, int group, void* out,
                        int out_dtype, void* stream)
{
    int rc = check_common(n, P, tile_begin, tile_len, bits, group);
    if (rc) return rc;
    if (out_dtype != ECHO_OUT_F32 && out_dtype != ECHO_OUT_BF16) return ECHO_EUNSUP;
    if (n == 0 || tile_len == 0) return ECHO_OK;
    if (!sum_codes || !sum_params || !out) return ECHO_EINVAL;
    if (!aligned16(sum_codes) || !aligned16(sum_params) || !aligned16(out)) return ECHO_EALIGN;
    echo::GatherArgs a = gather_args(sum_codes, sum_params, n, P, tile_begin, tile_len);
    a.out[0] = out;
    return launch_gather(a, P, 1, bits, group, out_dtype, (hipStream_t)stream);
}

int echo_compensate(const float* err, float* comp_next, float* slow, int64_t n, float alpha, float beta,
                    void* stream)
{
    if (n < 0 || n > kMaxN) return ECHO_ESHAPE;
    int rc = check_alpha_beta(alpha, beta);
    if (rc) return rc;
    if (n == 0) return ECHO_OK;
    if ((rc = check_slow(beta, slow != nullptr))) return rc;
    if (!err || !comp_next) return ECHO_EINVAL;
    if (!aligned16(err) || !aligned16(comp_next) || (slow && !aligned16(slow))) return ECHO_EALIGN;
    return launch_compensate(err, comp_next, slow, n, alpha, beta, (hipStream_t)stream);
}

size_t echo_allreduce_sim_workspace_bytes(int P, int64_t n, int bits, int group)
{
    if (check_common(n, P, 0, 0, bits, group)) return 0;
    return sim_layout(P, n, bits, group).total;
}

}  // extern "C"

namespace {

// The whole simulated call.  With noalloc the push and sum codes live in the
// static scratch array of this device (a->workspace is ignored) and every
// stage runs on the first stream, so the call creates no events either.
int sim_impl(const echo_sim_args* a, void* const* streams, int nstreams, bool noalloc)
{
    if (!a) return ECHO_EINVAL;
    const int P = a->P;
    int rc = check_common(a->n, P, 0, 0, a->bits, a->group);
    if (rc) return rc;
    if (a->out_dtype != ECHO_OUT_F32 && a->out_dtype != ECHO_OUT_BF16) return ECHO_EUNSUP;
    if (a->tiles < 1) return ECHO_EINVAL;
    if (a->ef != 0 && a->ef != 1) return ECHO_EINVAL;
    if ((a->quant & ~kQuantFlags) || quant_of(a->quant) < 0) return ECHO_EINVAL;
    if (streams && nstreams < 1) return ECHO_EINVAL;
    const int64_t n = a->n;
    if (n == 0) return ECHO_OK;
    const int64_t S = n / P;
    bool fused = false;
    if (a->ef) {
        bool any_err = false, all_err = true;
        for (int r = 0; r < P; ++r) {
            any_err = any_err || a->err[r] != nullptr;
            all_err = all_err && a->err[r] != nullptr;
        }
        if (any_err && !all_err) return ECHO_EINVAL;
        fused = !any_err;
        bool slow_all = true, slow_any = false;
        for (int r = 0; r < P; ++r) {
            slow_all = slow_all && a->slow[r] != nullptr;
            slow_any = slow_any || a->slow[r] != nullptr;
        }
        if (slow_any && !slow_all) return ECHO_EINVAL;
        if ((rc = check_alpha_beta(a->alpha, a->beta))) return rc;
        if ((rc = check_slow(a->beta, slow_all))) return rc;
    }
    for (int r = 0; r < P; ++r) {
        if (!a->x[r] || !a->out[r]) return ECHO_EINVAL;
        if (a->ef && !a->comp[r]) return ECHO_EINVAL;
        if (!aligned16(a->x[r]) || !aligned16(a->out[r])) return ECHO_EALIGN;
        if (a->ef && (!aligned16(a->comp[r]) || (a->err[r] && !aligned16(a->err[r])) ||
                      (a->slow[r] && !aligned16(a->slow[r]))))
            return ECHO_EALIGN;
    }
    const SimLayout L = sim_layout(P, n, a->bits, a->group);
    uint8_t* ws = nullptr;
    if (noalloc) {
        if (L.total > kScratchBytes) return ECHO_ETOOBIG;
        if ((rc = scratch_on_device(&ws))) return rc;
        nstreams = 1;
    } else {
        if (!a->workspace || a->workspace_bytes < L.total) return ECHO_EINVAL;
        if (!aligned16(a->workspace)) return ECHO_EALIGN;
        ws = (uint8_t*)a->workspace;
    }

    // workspace: push codes of every rank, push params of every rank, sum codes, sum params
    const uint8_t* pc[ECHO_MAX_P];
    const echo_qparam* pp[ECHO_MAX_P];
    for (int r = 0; r < P; ++r) {
        pc[r] = ws + (size_t)r * L.cb_al;
        pp[r] = (const echo_qparam*)(ws + (size_t)P * L.cb_al + (size_t)r * L.pb_al);
    }
    uint8_t* sc = ws + (size_t)P * (L.cb_al + L.pb_al);
    echo_qparam* sp = (echo_qparam*)(sc + L.cb_al);

    // tiles: equal lengths (multiples of the group), the last one ragged
    const int64_t groups_per_seg = S / a->group;
    int64_t T = a->tiles;
    if (T > groups_per_seg) T = groups_per_seg;
    if (T > kMaxTiles) T = kMaxTiles;   // bounds the events this call needs
    const int64_t tile_groups = (groups_per_seg + T - 1) / T;
    const int64_t tile_len = tile_groups * a->group;
    T = (S + tile_len - 1) / tile_len;

    const int nst = streams ? nstreams : 1;
    hipStream_t st_main = streams ? (hipStream_t)streams[0] : (hipStream_t)0;
    auto stage_stream = [&](int stage) -> hipStream_t {
        return streams ? (hipStream_t)streams[stage % nst] : (hipStream_t)0;
    };
    const hipStream_t s_push = stage_stream(0), s_red = stage_stream(1), s_tail = stage_stream(2),
                      s_comp = stage_stream(3);
    const bool multi = nst > 1;

    // feedback forms: classic fused (-e written into comp), two-timescale
    // fused (comp and slow updated in the kernels), or unfused (e into err,
    // then echo_compensate after the last reduce)
    const bool two_fused = a->ef && fused && a->beta > 0.0f;
    const int flags = ((fused && !two_fused) ? ECHO_ERR_NEGATED : 0) | a->quant;
    const echo::UpdArgs upd = make_upd(a->alpha, a->beta);
    // Small tiles: one launch per stage serves every rank (the per-rank
    // launches would be too small to fill the GPU, and the call is bound by
    // launch latency).  Large tiles: one launch per rank, which measured
    // faster than one launch over all ranks.
    const bool batch = (int64_t)blocks_for((uint32_t)(tile_len / echo::kRow), kUPush) * (P - 1) < kBatchBelowBlocks;
    const int per_launch = batch ? P : 1;
    auto comp_of = [&](int r) -> float* { return a->ef ? a->comp[r] : nullptr; };
    auto err_of = [&](int r) -> float* {
        return (a->ef && !two_fused) ? (fused ? a->comp[r] : a->err[r]) : nullptr;
    };
    auto slow_of = [&](int r) -> float* { return two_fused ? a->slow[r] : nullptr; };

    // A small message asked for in one tile: the whole call in one launch on
    // the first stream (the stages work group by group, so no stage waits for
    // another launch), then the separate update pass if the feedback is
    // unfused.  More tiles keep the staged schedule the caller asked for.
    if (a->tiles == 1 && n <= kOnePassMaxElems) {
        echo::OnePassArgs oa;
        std::memset(&oa, 0, sizeof(oa));
        for (int r = 0; r < P; ++r) {
            oa.x[r] = a->x[r]; oa.comp[r] = comp_of(r); oa.err[r] = err_of(r); oa.slow[r] = slow_of(r);
            oa.out[r] = a->out[r]; oa.pc[r] = (uint8_t*)pc[r]; oa.pp[r] = (uint32_t*)pp[r];
        }
        oa.sc = sc; oa.sp = (uint32_t*)sp;
        oa.upd = upd;
        oa.S = S;
        oa.seg_chunks = (uint32_t)((S + echo::kChunkElems - 1) / echo::kChunkElems);
        oa.P = P;
        oa.negate = (flags & ECHO_ERR_NEGATED) ? 1 : 0;
        rc = launch_onepass(oa, a->bits, a->group, quant_of(flags), two_fused, a->out_dtype == ECHO_OUT_BF16, st_main);
        if (rc) return rc;
        if (a->ef && !fused) {
            for (int r = 0; r < P; ++r) {
                rc = launch_compensate(a->err[r], a->comp[r], a->slow[r], n, a->alpha, a->beta, st_main);
                if (rc) return rc;
            }
        }
        return ECHO_OK;
    }

    // events: start, per tile push-done and reduce-done, per stream done
    hipEvent_t* ev = nullptr;
    if (multi) {
        rc = get_events((size_t)(1 + 2 * T + 4), &ev);
        if (rc) return rc;
    }
    hipEvent_t ev_start = multi ? ev[0] : nullptr;
    auto ev_push = [&](int64_t t) { return ev[1 + 2 * t]; };
    auto ev_red = [&](int64_t t) { return ev[2 + 2 * t]; };
    hipEvent_t* ev_done = multi ? ev + 1 + 2 * T : nullptr;

    hipError_t he;
    hipStream_t used[4] = {s_push, s_red, s_tail, s_comp};
    if (multi) {
        if ((he = hipEventRecord(ev_start, st_main)) != hipSuccess) return hip_fail(he);
        for (int k = 0; k < 4 && k < nst; ++k)
            if (used[k] != st_main && (he = hipStreamWaitEvent(used[k], ev_start, 0)) != hipSuccess)
                return hip_fail(he);
    }

    // The tail of tile t is enqueued after the push of tile t + 1, so that the
    // reduce of a tile can run beside the next tile's push even when the tail
    // shares the push's stream (two streams).
    auto tile_at = [&](int64_t t, int64_t& tb, int64_t& tl) {
        tb = t * tile_len;
        tl = (tb + tile_len <= S) ? tile_len : S - tb;
    };
    for (int64_t t = 0; t <= T; ++t) {
        int64_t tb, tl;
        if (t < T) {
            tile_at(t, tb, tl);
            // push: every rank quantizes its non-owned segments of this tile
            for (int r0 = 0; r0 < P; r0 += per_launch) {
                echo::PushArgs pa = push_args(n, P, tb, tl, r0, flags);
                pa.upd = upd;
                for (int k = 0; k < per_launch; ++k) {
                    const int r = r0 + k;
                    pa.x[k] = a->x[r]; pa.comp[k] = comp_of(r); pa.err[k] = err_of(r); pa.slow[k] = slow_of(r);
                    pa.codes[k] = (uint8_t*)pc[r]; pa.params[k] = (uint32_t*)pp[r];
                }
                if ((rc = launch_push(pa, P, per_launch, a->bits, a->group, flags, two_fused, s_push))) return rc;
            }
            if (multi) {
                if ((he = hipEventRecord(ev_push(t), s_push)) != hipSuccess) return hip_fail(he);
                if ((he = hipStreamWaitEvent(s_red, ev_push(t), 0)) != hipSuccess) return hip_fail(he);
            }
            // reduce: every owner sums its segment of this tile and requantizes once
            for (int o0 = 0; o0 < P; o0 += per_launch) {
                echo::ReduceArgs ra = reduce_args(n, P, tb, tl, o0, flags);
                ra.upd = upd;
                for (int k = 0; k < per_launch; ++k) {
                    const int o = o0 + k;
                    ra.x[k] = a->x[o]; ra.comp[k] = comp_of(o); ra.err[k] = err_of(o); ra.slow[k] = slow_of(o);
                }
                for (int j = 0; j < P; ++j) { ra.pc[j] = pc[j]; ra.pp[j] = (const uint32_t*)pp[j]; }
                ra.sc = sc; ra.sp = (uint32_t*)sp;
                if ((rc = launch_reduce(ra, per_launch, a->bits, a->group, flags, two_fused, s_red))) return rc;
            }
            if (multi && (he = hipEventRecord(ev_red(t), s_red)) != hipSuccess) return hip_fail(he);
        }
        if (t >= 1) {
            // gather moves no bytes here; tail: every rank decodes tile t - 1 of every segment
            tile_at(t - 1, tb, tl);
            if (multi && (he = hipStreamWaitEvent(s_tail, ev_red(t - 1), 0)) != hipSuccess) return hip_fail(he);
            for (int r0 = 0; r0 < P; r0 += per_launch) {
                echo::GatherArgs ga = gather_args(sc, sp, n, P, tb, tl);
                for (int k = 0; k < per_launch; ++k) ga.out[k] = a->out[r0 + k];
                if ((rc = launch_gather(ga, P, per_launch, a->bits, a->group, a->out_dtype, s_tail))) return rc;
            }
        }
    }
    // compensator update (two-timescale or unfused) after the last reduce
    if (a->ef && !fused) {
        if (multi && s_comp != s_red) {
            if ((he = hipStreamWaitEvent(s_comp, ev_red(T - 1), 0)) != hipSuccess) return hip_fail(he);
        }
        for (int r = 0; r < P; ++r) {
            rc = launch_compensate(a->err[r], a->comp[r], a->slow[r], n, a->alpha, a->beta, s_comp);
            if (rc) return rc;
        }
    }
    if (multi) {
        for (int k = 0; k < 4 && k < nst; ++k) {
            if (used[k] == st_main) continue;
            if ((he = hipEventRecord(ev_done[k], used[k])) != hipSuccess) return hip_fail(he);
            if ((he = hipStreamWaitEvent(st_main, ev_done[k], 0)) != hipSuccess) return hip_fail(he);
        }
    }
    return ECHO_OK;
}

}  // namespace

extern "C" {

int echo_allreduce_sim(const echo_sim_args* a, void* const* streams, int nstreams)
{
    return sim_impl(a, streams, nstreams, false);
}

int echo_allreduce_sim_noalloc(const echo_sim_args* a, void* stream)
{
    void* st[1] = {stream};
    return sim_impl(a, st, 1, true);
}

size_t echo_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
