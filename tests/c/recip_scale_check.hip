// Test-only device library: the kernels' reciprocal of a binary16 scale,
// echo::recip_scale, evaluated on the GPU for every binary16 bit pattern.
// tests/test_gpu_recip_scale.py compares the positive finite ones
// (0x0001 .. 0x7BFF) with the IEEE quotient 1/s.  Built with the library's
// own flags by error_feedback_quant_amd/build.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "echo_kernels.hpp"

constexpr uint32_t kPatterns = 0x10000u;

__global__ __launch_bounds__(256) void recip_all(uint32_t* out)
{
    const uint32_t b = blockIdx.x * 256u + threadIdx.x;
    if (b < kPatterns) {
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)b);
        out[b] = __builtin_bit_cast(uint32_t, echo::recip_scale(s));
    }
}

// out: host array of 65536 words (fp32 bit patterns), indexed by the
// binary16 pattern.  Returns 0, or the first HIP error code.
extern "C" int recip_scale_all(uint32_t* out)
{
    uint32_t* d = nullptr;
    hipError_t e = hipMalloc((void**)&d, kPatterns * sizeof(uint32_t));
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(recip_all, dim3(kPatterns / 256u), dim3(256), 0, 0, d);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(out, d, kPatterns * sizeof(uint32_t), hipMemcpyDeviceToHost);
    const hipError_t f = hipFree(d);
    return (int)(e != hipSuccess ? e : f);
}
