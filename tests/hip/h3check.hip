// Exhaustive checks of short sequences of the library's device code (h3qk_device.h) against the
// operations they stand for, built with the library's own compiler flags (correctly rounded
// division and square root, IEEE denormals, no contraction):
//   - rsqrt_rn_large (row_rstd when eps >= 2^-96) against 1.0f / sqrtf(v);
//   - quotient (the cast's RN(y / ds) from rcp = RN(1 / ds) and one FMA remainder correction)
//     against y / ds: every finite y at one descale, and every pair of significands;
//   - the E4M3 encodings: the integer encoder f32_to_e4m3 written out for any range of bit
//     patterns (the test compares it with the oracle on the host), the conversion instruction
//     behind pack_e4m3(hw = true) and the clamp_e4m3 + conversion step against f32_to_e4m3, and
//     the whole wave-level cast cast_e4m3_wave (fast, clip and exact paths, clip count) at
//     descale 1, where the quotient is the value itself.
// Test infrastructure: loaded by the GPU tests only.  Each check counts mismatches into a 64-bit
// word and records the first few failing inputs; every loop is bounded by its arguments.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_device.h"

namespace {

__device__ __forceinline__ void report(unsigned long long *bad, uint32_t *first, uint32_t what) {
    const unsigned long long k = atomicAdd(bad, 1ull);
    if (k < 4) first[k] = what;
}

__global__ __launch_bounds__(256) void rsqrt_check_kernel(uint32_t lo, uint32_t hi, unsigned long long *bad,
                                                          uint32_t *first) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += stride) {
        const float v = __uint_as_float((uint32_t)u);
        const float a = h3::rsqrt_rn_large(v);
        const float b = 1.0f / __builtin_sqrtf(v);
        if (__float_as_uint(a) != __float_as_uint(b) && !(a != a && b != b)) report(bad, first, (uint32_t)u);
    }
}

// Quotient check, for one descale ds (the fast path's range, [2^-60, 2^60]): with r = y / ds
// correctly rounded, the library's q must have r's bits wherever |r| is in [2^-12, 512); below 2^-12
// it must encode to r's E4M3 code (every such value is a signed zero code); at |r| >= 512 it must be
// NaN (the wave then takes the exact path) or exceed 448 in magnitude with r's sign (clamped to the
// saturated code and counted as clipped).  Non-finite y are skipped: NaN data takes the exact path.
__device__ __forceinline__ bool quotient_ok(float y, float ds, float rcp) {
    const float q = h3::quotient(y, ds, rcp);
    const float r = y / ds;
    const float a = __builtin_fabsf(r);
    if (a >= 0x1p-12f && a < 512.0f) return __float_as_uint(q) == __float_as_uint(r);
    if (a < 0x1p-12f) return h3::f32_to_e4m3(q) == h3::f32_to_e4m3(r);
    return (q != q) || (__builtin_fabsf(q) > 448.0f && __builtin_signbit(q) == __builtin_signbit(r));
}

__global__ __launch_bounds__(256) void quotient_check_kernel(uint32_t lo, uint32_t hi, float ds,
                                                             unsigned long long *bad, uint32_t *first) {
    const float rcp = 1.0f / ds;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += stride) {
        const float y = __uint_as_float((uint32_t)u);
        if (!__builtin_isfinite(y)) continue;
        if (!quotient_ok(y, ds, rcp)) report(bad, first, (uint32_t)u);
    }
}

// Every pair of significands: ds = 1 + j 2^-23 for j in [j0, j1), y = 1 + i 2^-23 for every i < 2^23
// (and -y for every 16th i).  Each thread takes one descale and 256 consecutive y; the 2^15 threads
// of a descale cover its 2^23 y.  q = y / ds lies in (1/2, 2), so every comparison is of bits.
// Scaling y and ds by powers of two scales every intermediate of quotient() exactly while they stay
// normal, which they do for descales in [2^-60, 2^60] and |y / ds| in [2^-12, 512); so this sweep
// covers that whole region.  A mismatch records the descale index j and the y significand i.
constexpr int kPairYPerThread = 256;
constexpr int kPairThreadsPerDs = (1 << 23) / kPairYPerThread;

__global__ __launch_bounds__(256) void quotient_pairs_kernel(uint32_t j0, uint32_t j1, unsigned long long *bad,
                                                             uint32_t *first) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t jd = t / kPairThreadsPerDs;
    if (jd >= (uint64_t)(j1 - j0)) return;
    const uint32_t j = j0 + (uint32_t)jd;
    const float ds = __uint_as_float(0x3F800000u + j);
    const float rcp = 1.0f / ds;
    const uint32_t i0 = (uint32_t)(t % kPairThreadsPerDs) * kPairYPerThread;
    for (uint32_t i = i0; i < i0 + kPairYPerThread; ++i) {
        const float y = __uint_as_float(0x3F800000u + i);
        bool ok = quotient_ok(y, ds, rcp);
        if ((i & 15u) == 0u) ok = ok && quotient_ok(-y, ds, rcp);
        if (!ok) {
            const unsigned long long k = atomicAdd(bad, 1ull);
            if (k < 2) {
                first[2 * k] = j;
                first[2 * k + 1] = i;
            }
        }
    }
}

// codes[i] = f32_to_e4m3(bits lo + i) for i < n (lo + n <= 2^32).
__global__ __launch_bounds__(256) void e4m3_codes_kernel(uint32_t lo, uint32_t n, uint8_t *codes) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        codes[i] = (uint8_t)h3::f32_to_e4m3(__uint_as_float(lo + (uint32_t)i));
}

// The conversion instruction against the integer encoder over the bit patterns [lo, hi] (inclusive),
// four consecutive patterns per thread packed by pack_e4m3(hw = true) (the last group repeats hi).
// clamp = 0: the patterns must all have |v| <= 448, the range the fast path hands the instruction
// unclamped.  clamp = 1: any non-NaN pattern (+-inf included), first brought into range by
// clamp_e4m3 as the clip path does; its code must be the integer encoder's code of the unclamped
// value, i.e. the saturated code past 448.
__global__ __launch_bounds__(256) void e4m3_hw_check_kernel(uint32_t lo, uint32_t hi, int clamp,
                                                            unsigned long long *bad, uint32_t *first) {
    const uint64_t groups = ((uint64_t)hi - lo) / 4 + 1;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t gi = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups; gi += stride) {
        float v[4], q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t u = (uint64_t)lo + 4 * gi + k;
            v[k] = __uint_as_float((uint32_t)(u <= hi ? u : hi));
            q[k] = clamp ? h3::clamp_e4m3(v[k]) : v[k];
        }
        uint32_t w[1];
        h3::pack_e4m3<4>(q, true, w);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (((w[0] >> (8 * k)) & 0xFFu) != h3::f32_to_e4m3(v[k])) report(bad, first, __float_as_uint(v[k]));
    }
}

// The wave-level cast at descale 1 over 2^32 bit patterns: lane l of wave w takes the patterns
// map(256 w + 4 l + k), k < 4, with map the identity (order = 0), the bijection
// x -> 0x9E3779B1 x mod 2^32 (order = 1: waves of scattered magnitudes and NaNs), or that bijection
// with NaN patterns turned finite by clearing their exponent's top bit (order = 2: waves that mix
// in-range and clipped values without taking the exact path).  Codes must equal the integer
// encoder's (NaN codes up to their sign, which the contract leaves open); the wave's clip count
// must equal the number of its non-NaN values past 448 in magnitude.  sat_total receives the sum
// of the clip counts.  Waves [w0, w1) of the 2^24.
__global__ __launch_bounds__(256) void cast_wave_check_kernel(uint32_t w0, uint32_t w1, int order,
                                                              unsigned long long *bad, uint32_t *first,
                                                              unsigned long long *sat_total) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t wave = (uint64_t)w0 + (uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (wave >= w1) return;  // wave-uniform
    float y[1][4];
    uint32_t mine = 0;  // this lane's non-NaN values past 448
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t u = (uint32_t)(wave * 256u + 4u * lane + (uint32_t)k);
        if (order >= 1) u *= 0x9E3779B1u;
        if (order == 2 && (u & 0x7FFFFFFFu) > 0x7F800000u) u &= ~0x40000000u;
        y[0][k] = __uint_as_float(u);
        mine += (!(y[0][k] != y[0][k]) && __builtin_fabsf(y[0][k]) > 448.0f) ? 1u : 0u;
    }
    uint32_t nsat = 0, w[1][1];
    h3::cast_e4m3_wave<1, 4>(y, 1.0f, 1.0f, true, true, nsat, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t got = (w[0][0] >> (8 * k)) & 0xFFu;
        const uint32_t ref = h3::f32_to_e4m3(y[0][k]);
        const bool nan = y[0][k] != y[0][k];
        if (nan ? (got & 0x7Fu) != 0x7Fu : got != ref) report(bad, first, __float_as_uint(y[0][k]));
    }
    uint32_t expect = mine;
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) expect += (uint32_t)__shfl_xor((int)expect, o, 64);
    if (lane == 0) {
        if (expect != nsat) report(bad, first, 0xFFFFFFFFu);
        if (nsat) atomicAdd(sat_total, (unsigned long long)nsat);
    }
}

hipError_t launch_status() { return hipGetLastError(); }

}  // namespace

// bad: one uint64 (zeroed by the caller), first: four uint32 (the first mismatching inputs).
extern "C" int h3check_rsqrt(uint32_t lo, uint32_t hi, unsigned long long *bad, uint32_t *first, hipStream_t s) {
    hipLaunchKernelGGL(rsqrt_check_kernel, dim3(8192), dim3(256), 0, s, lo, hi, bad, first);
    return launch_status() == hipSuccess ? 0 : 1;
}

// bad: one uint64 (zeroed by the caller), first: four uint32 (the first mismatching y bit patterns).
extern "C" int h3check_quotient(uint32_t lo, uint32_t hi, float ds, unsigned long long *bad, uint32_t *first,
                                hipStream_t s) {
    hipLaunchKernelGGL(quotient_check_kernel, dim3(8192), dim3(256), 0, s, lo, hi, ds, bad, first);
    return launch_status() == hipSuccess ? 0 : 1;
}

// Descale significands [j0, j1) of [0, 2^23) against every y significand.  first: four uint32, the
// (j, i) pairs of the first two mismatches.
extern "C" int h3check_quotient_pairs(uint32_t j0, uint32_t j1, unsigned long long *bad, uint32_t *first,
                                      hipStream_t s) {
    if (j1 <= j0 || j1 > (1u << 23)) return 2;
    // a dispatch's grid is a 32-bit count of work-items: at most 2^16 descales per launch
    const uint64_t threads = (uint64_t)(j1 - j0) * kPairThreadsPerDs;
    if (threads > (1ull << 31)) return 2;
    const uint64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(quotient_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, j0, j1, bad, first);
    return launch_status() == hipSuccess ? 0 : 1;
}

// codes: n bytes (device).  lo + n must not exceed 2^32.
extern "C" int h3check_e4m3_codes(uint32_t lo, uint32_t n, uint8_t *codes, hipStream_t s) {
    if ((uint64_t)lo + n > (1ull << 32)) return 2;
    hipLaunchKernelGGL(e4m3_codes_kernel, dim3(8192), dim3(256), 0, s, lo, n, codes);
    return launch_status() == hipSuccess ? 0 : 1;
}

extern "C" int h3check_e4m3_hw(uint32_t lo, uint32_t hi, int clamp, unsigned long long *bad, uint32_t *first,
                               hipStream_t s) {
    if (hi < lo) return 2;
    hipLaunchKernelGGL(e4m3_hw_check_kernel, dim3(8192), dim3(256), 0, s, lo, hi, clamp, bad, first);
    return launch_status() == hipSuccess ? 0 : 1;
}

// Waves [w0, w1) of the 2^24 waves that cover every bit pattern; sat_total: one uint64 (zeroed by
// the caller).
extern "C" int h3check_cast_wave(uint32_t w0, uint32_t w1, int order, unsigned long long *bad, uint32_t *first,
                                 unsigned long long *sat_total, hipStream_t s) {
    if (w1 <= w0 || w1 > (1u << 24) || order < 0 || order > 2) return 2;
    const uint32_t blocks = (w1 - w0 + 3) / 4;
    hipLaunchKernelGGL(cast_wave_check_kernel, dim3(blocks), dim3(256), 0, s, w0, w1, order, bad, first, sat_total);
    return launch_status() == hipSuccess ? 0 : 1;
}
