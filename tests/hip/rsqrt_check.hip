// Exhaustive check of the library's shorter reciprocal-square-root sequence (rsqrt_rn_large in
// rmsnorm_rope_amd/csrc/h3qk_device.h, used by row_rstd when eps >= 2^-96) against the correctly
// rounded operations it replaces, 1.0f / sqrtf(v), over every binary32 bit pattern in [lo, hi).
// Built with the library's own compiler flags (correctly rounded division and square root).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_device.h"

namespace {

__global__ __launch_bounds__(256) void rsqrt_check_kernel(uint32_t lo, uint32_t hi, unsigned long long *bad,
                                                          uint32_t *first) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += stride) {
        const float v = __uint_as_float((uint32_t)u);
        const float a = h3::rsqrt_rn_large(v);
        const float b = 1.0f / __builtin_sqrtf(v);
        if (__float_as_uint(a) != __float_as_uint(b) && !(a != a && b != b)) {
            const unsigned long long k = atomicAdd(bad, 1ull);
            if (k < 4) first[k] = (uint32_t)u;
        }
    }
}

}  // namespace

// bad: one uint64 (zeroed by the caller), first: four uint32 (the first mismatching inputs).
extern "C" int h3check_rsqrt(uint32_t lo, uint32_t hi, unsigned long long *bad, uint32_t *first, hipStream_t s) {
    hipLaunchKernelGGL(rsqrt_check_kernel, dim3(8192), dim3(256), 0, s, lo, hi, bad, first);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
