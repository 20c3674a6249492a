// gfx950 kernels for the two elementwise ops of a MiniMax-H3 VAE decoder block that sit beside the
// attention input preparation ([OMNI-6607] "Operations" table, SwiGLU and scaled-residual rows):
//   SwiGLU          y = silu(g) u on the 16-bit w1 output [N, 2F] (g = first F columns, u = the rest),
//                   computed in binary32 with the device exp, rounded once to the 16-bit output;
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

// silu(g) u = (g / (1 + exp(-g))) u in binary32 with the hardware exp2 and reciprocal: a few
// binary32 ulps in all (relative error below 1e-6), far under one ulp of the 16-bit output, so the
// rounded result is the exactly rounded one except next to a rounding boundary, where it may be one
// 16-bit ulp away.  exp(-g) overflows to +inf for g below about -88, giving silu = -0.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __expf(-g);
    const float d = 1.0f + e;
    const float s = g * __builtin_amdgcn_rcpf(d);
    return s * u;
}

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
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float y0 = silu_mul(h16_to_f32<DT>(gv[k] & 0xFFFFu), h16_to_f32<DT>(uv[k] & 0xFFFFu));
        const float y1 = silu_mul(h16_to_f32<DT>(gv[k] >> 16), h16_to_f32<DT>(uv[k] >> 16));
        o[k] = f32_to_h16<DT>(y0) | (f32_to_h16<DT>(y1) << 16);
    }
    __builtin_nontemporal_store((u32x4){o[0], o[1], o[2], o[3]},
                                reinterpret_cast<u32x4 *>(y + (uint64_t)t * 8u));
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
