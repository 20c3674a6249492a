// gfx950 kernels for the two elementwise ops of a MiniMax-H3 VAE decoder block that sit beside the
// attention input preparation ([OMNI-6607] "Operations" table, SwiGLU and scaled-residual rows):
//   SwiGLU          y = silu(g) u on the 16-bit w1 output [N, 2F] (g = first F columns, u = the rest),
//                   the binary64 value rounded once to the 16-bit output (a binary32 fast path where
//                   that rounding is certain, binary64 for the other elements);
//   scaled residual out = res + (branch * scale) in binary32, product rounded first (no contraction).
// Both stream with no reuse: 16-byte vectors, two per lane (the second 256 vectors after the first),
// short-lived 256-thread blocks that sweep the tensors in order; outputs bypass the caches
// (nontemporal stores).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_internal.h"

namespace h3 {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kVectorsPerThread = 2;

template <int DT>
__device__ __forceinline__ float h16_to_f32(uint32_t b) {
    if constexpr (DT == H3_BF16) return __uint_as_float(b << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

template <int DT>
__device__ __forceinline__ uint32_t f32_to_h16(float x) {
    if constexpr (DT == H3_BF16) return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    else return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// ------------------------------------------------------------------ SwiGLU
//
// The contract: y = RN16(RN64(RN64(g / RN64(1 + exp(-g))) * u)), the binary64 evaluation rounded
// once to the 16-bit output.  Each element takes a binary32 fast path whose result is used only when
// its rounding to 16 bits is certain to be the contract's; otherwise it is evaluated in binary64.
// Every (g, u) pair of either 16-bit dtype is checked against the CPU oracle by the tests.

// exp(x) for |x| <= 64 in binary32, about one ulp: Cody and Waite's range reduction (W. J. Cody,
// W. Waite, Software Manual for the Elementary Functions, 1980), x = k ln2 + r with |r| <= ln2 / 2,
// ln2 split in two so that k ln2_hi is exact (ln2_hi has 15 significant bits, |k| <= 93), then the
// degree-7 Taylor polynomial of exp(r) (truncation below 2^-26 relative) and a scaling by 2^k.
__device__ __forceinline__ float exp_reduced(float x) {
    constexpr float kLog2e = 1.44269504088896340736f;
    constexpr float kLn2Hi = 0.693145751953125f;         // ln 2 to 15 bits
    constexpr float kLn2Lo = 1.42860676533018700e-06f;    // ln 2 - kLn2Hi, rounded
    const float k = __builtin_rintf(x * kLog2e);
    float r = __builtin_fmaf(k, -kLn2Hi, x);              // exact
    r = __builtin_fmaf(k, -kLn2Lo, r);
    float p = 1.0f / 5040.0f;
    p = __builtin_fmaf(p, r, 1.0f / 720.0f);
    p = __builtin_fmaf(p, r, 1.0f / 120.0f);
    p = __builtin_fmaf(p, r, 1.0f / 24.0f);
    p = __builtin_fmaf(p, r, 1.0f / 6.0f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)k);
}

// The value as a materialised binary32 (the compiler may otherwise fold a product and its
// conversion to binary16 into one mixed-precision FMA).
__device__ __forceinline__ float keep32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// binary64 -> 16-bit float (FRAC fraction bits, smallest normal exponent EMIN, INF / NAN codes) with
// one rounding to nearest even; the conversion instructions go through binary32 and round twice.
template <int FRAC, int EMIN, uint32_t INF, uint32_t QNAN>
__device__ __forceinline__ uint32_t round_f64_to_16(double v) {
    const uint64_t x = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(x >> 48) & 0x8000u;
    const uint64_t a = x & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return sign | QNAN;
    const int E = (int)(a >> 52);
    const uint64_t sig = (a & 0xFFFFFFFFFFFFFull) | (E ? (1ull << 52) : 0ull);
    const int e = E ? E - 1023 : -1022;
    if (e > (int)(INF >> FRAC) + EMIN - 1) return sign | INF;
    const int shift = 52 - FRAC + (e < EMIN ? EMIN - e : 0);
    if (shift > 63) return sign;  // below half the smallest subnormal: rounds to zero
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1ull), half = 1ull << (shift - 1);
    q += (rem > half || (rem == half && (q & 1ull))) ? 1ull : 0ull;
    uint64_t code = (e > EMIN ? (uint64_t)(e - EMIN) << FRAC : 0ull) + q;
    if (code >= INF) code = INF;
    return sign | (uint32_t)code;
}

// The contract's binary64 evaluation.
template <int DT>
__device__ uint32_t silu_mul_f64(float g, float u) {
    const double gd = g, ud = u;
    const double s = gd / (1.0 + exp(-gd));
    const double v = s * ud;
    if constexpr (DT == H3_BF16) return round_f64_to_16<7, -126, 0x7F80u, 0x7FC0u>(v);
    else return round_f64_to_16<10, -14, 0x7C00u, 0x7E00u>(v);
}

// Fast path.  y = RN32(RN32(g * rcp(RN32(1 + e))) * u) with e = exp_reduced(-g) is within a few
// binary32 ulps of the exact silu(g) u (about 1.5 ulp from e, 0.5 from the sum, 1 from the
// hardware reciprocal, 0.5 from each product; over every (g, u) pair of either dtype with
// |g| <= 64 it was never more than 3 ulps from the binary64 value rounded to binary32), and the
// contract's binary64 value is within 2^-50 of the exact one.  So the 16-bit rounding of y is the
// contract's unless a 16-bit rounding boundary lies within that distance of y: the element is
// taken here only when |g| <= 64 and y is zero, or lies in the 16-bit normal range more than
// kNearUlps binary32 ulps from every boundary (there the boundaries are the binary32 values whose
// bits below the 16-bit fraction hold the midpoint pattern, evenly spaced in the bit patterns).
// Otherwise ok is false and the caller evaluates the element in binary64.
constexpr uint32_t kNearUlps = 4;

template <int DT>
__device__ __forceinline__ uint32_t silu_mul_fast(float g, float u, bool &ok) {
    const float e = exp_reduced(-g);
    const float d = 1.0f + e;
    const float s = g * __builtin_amdgcn_rcpf(d);
    const float y = keep32(s * u);
    const uint32_t a = __float_as_uint(y) & 0x7FFFFFFFu;
    constexpr uint32_t kLow = DT == H3_BF16 ? 0xFFFFu : 0x1FFFu;          // bits below the 16-bit fraction
    constexpr uint32_t kMid = (kLow >> 1) + 1u;                            // their midpoint pattern
    constexpr uint32_t kMinNormal = DT == H3_BF16 ? 0x00800000u : 0x38800000u;
    const bool far = ((a & kLow) - (kMid - kNearUlps)) > 2u * kNearUlps;
    ok = (__builtin_fabsf(g) <= 64.0f) & ((a == 0u) | ((a >= kMinNormal) & far));  // no branches
    return f32_to_h16<DT>(y);
}

// One 16-byte vector of outputs (8 elements) from its gate and up vectors.
template <int DT>
__device__ __forceinline__ u32x4 swiglu_vector(const u32x4 gv, const u32x4 uv) {
    uint32_t o[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t gb = (k & 1) ? (gv[k >> 1] >> 16) : (gv[k >> 1] & 0xFFFFu);
        const uint32_t ub = (k & 1) ? (uv[k >> 1] >> 16) : (uv[k >> 1] & 0xFFFFu);
        o[k] = silu_mul_fast<DT>(h16_to_f32<DT>(gb), h16_to_f32<DT>(ub), ok[k]);
    }
    // Rare: the elements the fast path cannot decide, in binary64.  Each pass takes every lane's
    // next pending element at once (one copy of the binary64 code, as many passes as the busiest
    // lane has pending elements), with the element picked and placed by selects, not by indexing.
    uint32_t pend = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) pend |= ok[k] ? 0u : 1u << k;
    while (pend) {
        const int k = __builtin_ctz(pend);
        pend &= pend - 1u;
        uint32_t gw = gv[0], uw = uv[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            gw = (k >> 1) == j ? gv[j] : gw;
            uw = (k >> 1) == j ? uv[j] : uw;
        }
        const uint32_t sh = (k & 1) ? 16u : 0u;
        const uint32_t r = silu_mul_f64<DT>(h16_to_f32<DT>((gw >> sh) & 0xFFFFu), h16_to_f32<DT>((uw >> sh) & 0xFFFFu));
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = k == j ? r : o[j];
    }
    return (u32x4){o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)};
}

// Each vector is loaded, evaluated and stored in turn (issuing both vectors' loads first measured
// 21.4 against 19.4 us on the bench shape).
template <int DT>
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ y,
                                                     uint32_t vectors, DivMagic f8, uint32_t F) {
  for (int v = 0; v < kVectorsPerThread; ++v) {
    const uint32_t t = blockIdx.x * (256u * kVectorsPerThread) + v * 256u + threadIdx.x;  // 8 outputs
    if (t >= vectors) return;
    const uint32_t n = div_apply(t, f8);                  // row
    const uint32_t f = (t - n * f8.d) * 8u;               // column of the first output
    const uint16_t *row = x + (uint64_t)n * (2u * (uint64_t)F);
    const u32x4 gv = *reinterpret_cast<const u32x4 *>(row + f);
    const u32x4 uv = *reinterpret_cast<const u32x4 *>(row + F + f);
    __builtin_nontemporal_store(swiglu_vector<DT>(gv, uv), reinterpret_cast<u32x4 *>(y + (uint64_t)t * 8u));
  }
}

template <int DT, bool PER_CHANNEL>
__global__ __launch_bounds__(256) void scaled_residual_kernel(const float *__restrict__ res,
                                                              const uint16_t *__restrict__ br,
                                                              const float *__restrict__ scale,
                                                              float *__restrict__ out, uint32_t vectors,
                                                              DivMagic c4) {
  for (int v = 0; v < kVectorsPerThread; ++v) {
    const uint32_t t = blockIdx.x * (256u * kVectorsPerThread) + v * 256u + threadIdx.x;  // 4 elements
    if (t >= vectors) return;
    const f32x4 r = *reinterpret_cast<const f32x4 *>(res + (uint64_t)t * 4u);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(br + (uint64_t)t * 4u);
    f32x4 s;
    if constexpr (PER_CHANNEL) {
        const uint32_t n = div_apply(t, c4);
        s = *reinterpret_cast<const f32x4 *>(scale + (t - n * c4.d) * 4u);
    } else {
        s = (f32x4){scale[0], scale[0], scale[0], scale[0]};
    }
    const float b0 = h16_to_f32<DT>(b.x & 0xFFFFu), b1 = h16_to_f32<DT>(b.x >> 16);
    const float b2 = h16_to_f32<DT>(b.y & 0xFFFFu), b3 = h16_to_f32<DT>(b.y >> 16);
    const float p0 = b0 * s.x, p1 = b1 * s.y, p2 = b2 * s.z, p3 = b3 * s.w;
    __builtin_nontemporal_store((f32x4){r.x + p0, r.y + p1, r.z + p2, r.w + p3},
                                reinterpret_cast<f32x4 *>(out + (uint64_t)t * 4u));
  }
}

// vectors < 2^32 (the host's limit): at most 2^23 blocks, and the kernels' 32-bit vector index
// blockIdx.x * 512 + 256 v + threadIdx.x stays below 2^32.
int launch(const void *kern, uint32_t vectors, void **args, hipStream_t stream, std::string *err) {
    const uint64_t blocks = blocks_for(vectors, 256u * kVectorsPerThread);
    if (blocks == 0) return H3_OK;
    const hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3(256), args, 0, stream);
    if (e != hipSuccess) {
        *err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

}  // namespace

int launch_swiglu(int dt, const void *x, void *y, int64_t N, int64_t F, hipStream_t stream, std::string *err) {
    uint32_t vectors = (uint32_t)(N * F / 8);
    DivMagic f8 = div_magic((uint32_t)(F / 8));
    uint32_t F32 = (uint32_t)F;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    uint16_t *yp = static_cast<uint16_t *>(y);
    void *args[] = {&xp, &yp, &vectors, &f8, &F32};
    if (dt == H3_BF16) return launch(reinterpret_cast<const void *>(swiglu_kernel<H3_BF16>), vectors, args, stream, err);
    return launch(reinterpret_cast<const void *>(swiglu_kernel<H3_F16>), vectors, args, stream, err);
}

int launch_scaled_residual(int dt, const float *res, const void *branch, const float *scale, int64_t scale_len,
                           float *out, int64_t N, int64_t C, hipStream_t stream, std::string *err) {
    uint32_t vectors = (uint32_t)(N * C / 4);
    DivMagic c4 = div_magic((uint32_t)(C / 4));
    const uint16_t *bp = static_cast<const uint16_t *>(branch);
    void *args[] = {&res, &bp, &scale, &out, &vectors, &c4};
    const bool pc = scale_len != 1;
    const void *k = dt == H3_BF16 ? (pc ? reinterpret_cast<const void *>(scaled_residual_kernel<H3_BF16, true>)
                                        : reinterpret_cast<const void *>(scaled_residual_kernel<H3_BF16, false>))
                                  : (pc ? reinterpret_cast<const void *>(scaled_residual_kernel<H3_F16, true>)
                                        : reinterpret_cast<const void *>(scaled_residual_kernel<H3_F16, false>));
    return launch(k, vectors, args, stream, err);
}

}  // namespace h3
