// Exhaustive checks of two short sequences of the library's device code against the correctly
// rounded operations they replace, built with the library's own compiler flags (correctly rounded
// division and square root):
//   - rsqrt_rn_large (used by row_rstd when eps >= 2^-96) against 1.0f / sqrtf(v), over every
//     binary32 bit pattern in [lo, hi);
//   - quotient (the cast's RN(y / ds) from rcp = RN(1 / ds) and FMA remainder corrections) against
//     y / ds, for every finite binary32 y in [lo, hi) and one descale ds.
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

// Quotient check, for one descale ds (the fast path's range, [2^-60, 2^60]): with r = y / ds
// correctly rounded, the library's q must have r's bits wherever |r| is in [2^-12, 512); below 2^-12
// it must encode to r's E4M3 code (every such value is a signed zero code); at |r| >= 512 it must be
// NaN (the wave then takes the exact path) or exceed 448 in magnitude with r's sign (clamped to the
// saturated code and counted as clipped).  Non-finite y are skipped: NaN data takes the exact path.
__global__ __launch_bounds__(256) void quotient_check_kernel(uint32_t lo, uint32_t hi, float ds,
                                                             unsigned long long *bad, uint32_t *first) {
    const float rcp = 1.0f / ds;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += stride) {
        const float y = __uint_as_float((uint32_t)u);
        if (!__builtin_isfinite(y)) continue;
        const float q = h3::quotient(y, ds, rcp);
        const float r = y / ds;
        const float a = __builtin_fabsf(r);
        bool ok;
        if (a >= 0x1p-12f && a < 512.0f) ok = __float_as_uint(q) == __float_as_uint(r);
        else if (a < 0x1p-12f) ok = h3::f32_to_e4m3(q) == h3::f32_to_e4m3(r);
        else ok = (q != q) || (__builtin_fabsf(q) > 448.0f && __builtin_signbit(q) == __builtin_signbit(r));
        if (!ok) {
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

// bad: one uint64 (zeroed by the caller), first: four uint32 (the first mismatching y bit patterns).
extern "C" int h3check_quotient(uint32_t lo, uint32_t hi, float ds, unsigned long long *bad, uint32_t *first,
                                hipStream_t s) {
    hipLaunchKernelGGL(quotient_check_kernel, dim3(8192), dim3(256), 0, s, lo, hi, ds, bad, first);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
