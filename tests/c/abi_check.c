/* Compiles include/echo.h as strict C99 and exercises libecho's host-side
 * argument checks through the C ABI (no device needed: every call below is
 * rejected before anything would be enqueued). */
#include <stdio.h>
#include <string.h>

#include "echo.h"

static int fails = 0;

static void expect(const char* what, int got, int want)
{
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, got, echo_status_str(got), want);
        ++fails;
    }
}

int main(void)
{
    /* a non-null, 16-byte aligned address that is never dereferenced */
    void* fake = (void*)(size_t)(1u << 20);
    const uint16_t* x = (const uint16_t*)fake;
    uint8_t* codes = (uint8_t*)fake;
    echo_qparam* params = (echo_qparam*)fake;

    expect("bits 3", echo_quantize_ef(x, NULL, 4096, 4, 0, 0, 128, 3, 128, codes, params, NULL, 0, NULL),
           ECHO_EUNSUP);
    expect("group 64", echo_quantize_ef(x, NULL, 4096, 4, 0, 0, 128, 4, 64, codes, params, NULL, 0, NULL),
           ECHO_EUNSUP);
    expect("rank 4", echo_quantize_ef(x, NULL, 4096, 4, 4, 0, 128, 4, 128, codes, params, NULL, 0, NULL),
           ECHO_EINVAL);
    expect("n % (P*g)", echo_quantize_ef(x, NULL, 4096 + 128, 4, 0, 0, 128, 4, 128, codes, params, NULL, 0, NULL),
           ECHO_ESHAPE);
    expect("both quantizers",
           echo_quantize_ef(x, NULL, 4096, 4, 0, 0, 128, 4, 128, codes, params, NULL,
                            ECHO_QUANT_NAIVE | ECHO_QUANT_SYMMETRIC, NULL),
           ECHO_EINVAL);
    expect("misaligned x", echo_quantize_ef((const uint16_t*)((char*)fake + 2), NULL, 4096, 4, 0, 0, 128, 4, 128,
                                            codes, params, NULL, 0, NULL),
           ECHO_EALIGN);
    expect("empty tile", echo_quantize_ef(x, NULL, 4096, 4, 0, 0, 0, 4, 128, codes, params, NULL, 0, NULL),
           ECHO_OK);
    expect("gather dtype", echo_gather_dequant(codes, params, 4096, 0, 128, 4, 4, 128, fake, 7, NULL),
           ECHO_EUNSUP);
    expect("compensate alpha", echo_compensate((const float*)fake, (float*)fake, NULL, 1024, 0.5f, 0.0f, NULL),
           ECHO_EINVAL);
    expect("workspace size", (int)(echo_allreduce_sim_workspace_bytes(4, 4096, 4, 128) == 5 * (2048 + 256)), 1);
    expect("gemm N % 256", echo_gemm_quantize_ef(x, x, 512, 384, 128, NULL, 4, 0, 4, 128, codes, params, NULL,
                                                 (uint16_t*)fake, 0, NULL),
           ECHO_ESHAPE);
    expect("gemm group 64", echo_gemm_quantize_ef(x, x, 512, 256, 128, NULL, 4, 0, 4, 64, codes, params, NULL,
                                                  (uint16_t*)fake, 0, NULL),
           ECHO_EUNSUP);
    expect("gemm x_out NULL", echo_gemm_quantize_ef(x, x, 512, 256, 128, NULL, 4, 0, 4, 128, codes, params, NULL,
                                                    NULL, ECHO_X_ALL, NULL),
           ECHO_EINVAL);
    expect("gemm K = 2^22", echo_gemm_quantize_ef(x, x, 512, 256, (int64_t)1 << 22, NULL, 4, 0, 4, 128, codes,
                                                  params, NULL, (uint16_t*)fake, 0, NULL),
           ECHO_ESHAPE);
    expect("gemm empty", echo_gemm_quantize_ef(x, x, 0, 256, 128, NULL, 4, 0, 4, 128, codes, params, NULL,
                                               (uint16_t*)fake, 0, NULL),
           ECHO_OK);

    echo_sim_args a;
    memset(&a, 0, sizeof a);
    a.P = 4; a.bits = 4; a.group = 128; a.tiles = 0; a.n = 4096;
    expect("sim tiles 0", echo_allreduce_sim(&a, NULL, 0), ECHO_EINVAL);
    a.tiles = 1; a.n = 0;
    expect("sim empty", echo_allreduce_sim(&a, NULL, 0), ECHO_OK);
    expect("noalloc scratch", (int)(echo_noalloc_scratch_bytes() == ((size_t)64 << 20)), 1);
    expect("noalloc null args", echo_allreduce_sim_noalloc(NULL, NULL), ECHO_EINVAL);
    a.n = (int64_t)1 << 25;
    for (int r = 0; r < 4; ++r) { a.x[r] = x; a.out[r] = fake; }
    expect("noalloc too big", echo_allreduce_sim_noalloc(&a, NULL), ECHO_ETOOBIG);
    expect("last hip error", echo_last_hip_error(), 0);

    printf(fails ? "abi_check: %d failures\n" : "abi_check: ok\n", fails);
    return fails ? 1 : 0;
}
