// gfx950 kernels for the MiniMax-H3 QK preparation: per-head RMSNorm + partial 3-axis RoPE +
// head-major permute ([SDCPP-19] fused QKV / ggml_rope_pe_permute_rms commits, [OMNI-6607]
// Operations table), and the FP8 amax and E4M3 cast passes ([TRT-21485] Summary and
// fused_fp8_qk commits).  The numerical contract is stated in include/h3qk.h.
//
// Work decomposition (wave64):
//   * A work item is 8 consecutive tokens of one item and a chunk of its heads.  Lane
//     l = 8 g + c serves token g of the 8 and holds, of every head row it touches, the dims
//     {8W m + W c + k : m < M, k < W} with W = 4, M = 2 for D = 64 and W = 8, M = 2 for D = 128.
//     Loads are then 8 W contiguous bytes per token per instruction, and the f32 Q store of a
//     D = 64 row is two full 128-byte lines.
//   * The halving reduction tree maps onto that layout as: levels o >= 8W fold chunks inside
//     the lane, levels 4W, 2W, W are cross-lane butterflies (lane c with c^4, c^2, c^1, the
//     8 lanes of a token), levels below W fold inside the chunk.  Floating-point addition is
//     commutative, so the butterfly partner computes the same bits as the tree node, and all
//     8 lanes end with ss.
//   * Each lane's rotary pairs depend only on its lane index, so their (axis, frequency) is
//     computed once; the cos/sin entries of a token are loaded once and reused for every head.
//   * Work items are taken grid-stride, so per-lane setup (weights, pair map) is paid once per
//     wave, and the amax pass issues one atomic per wave and tensor.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_internal.h"

namespace h3 {
namespace {

constexpr int DT_F32 = H3_F32, DT_F16 = H3_F16, DT_BF16 = H3_BF16, DT_E4M3 = H3_E4M3FN;

// ------------------------------------------------------------------ element conversions

template <int IN>
__device__ __forceinline__ float in_to_f32(uint32_t bits16) {
    if constexpr (IN == DT_BF16) {
        return __uint_as_float(bits16 << 16);
    } else {
        _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
        return (float)h;  // exact
    }
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even, IEEE denormals
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// binary32 -> OCP E4M3FN, round to nearest even, saturating to +-448 (also +-inf), NaN -> 0x7F
// with the sign.  Integer arithmetic on the encoding.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t E = a >> 23;
    uint32_t sig = (a & 0x7FFFFFu) | (E ? 0x800000u : 0u);
    bool normal = E >= 121u;                       // |f| >= 2^-6
    uint32_t s = normal ? 20u : min(141u - E, 31u);
    uint32_t base = normal ? (E - 121u) << 3 : 0u;
    uint32_t q = sig >> s;
    uint32_t rem = sig & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1u);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    uint32_t code = base + q;
    code = a > 0x43E00000u ? 0x7Eu : code;         // > 448 saturates
    code = a > 0x7F800000u ? 0x7Fu : code;         // NaN
    return code | sign;
}

template <int OT>
__device__ __forceinline__ uint32_t encode_out(float x) {
    if constexpr (OT == DT_F16) return f32_to_f16_bits(x);
    else if constexpr (OT == DT_BF16) return f32_to_bf16_bits(x);
    else return f32_to_e4m3(x);
}

// ------------------------------------------------------------------ cross-lane butterflies

__device__ __forceinline__ float lane_xor1(float v) {  // DPP quad_perm [1,0,3,2]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {  // DPP quad_perm [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor4(float v) {  // ds_swizzle bit mode: and 0x1F, xor 4
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}

// ------------------------------------------------------------------ loads and stores

// W consecutive 16-bit values (W = 4: 8 bytes, W = 8: 16 bytes) as W/2 packed words.
template <int W>
__device__ __forceinline__ void load_chunk(const uint16_t *p, uint32_t (&r)[W / 2]) {
    if constexpr (W == 4) {
        uint2 t = *reinterpret_cast<const uint2 *>(p);
        r[0] = t.x; r[1] = t.y;
    } else {
        uint4 t = *reinterpret_cast<const uint4 *>(p);
        r[0] = t.x; r[1] = t.y; r[2] = t.z; r[3] = t.w;
    }
}

// Store W values of one chunk in output dtype OT at element offset `e` of `base`.
template <int OT, int W>
__device__ __forceinline__ void store_chunk(void *base, int64_t e, const float (&y)[W]) {
    if constexpr (OT == DT_F32) {
        float *p = reinterpret_cast<float *>(base) + e;
#pragma unroll
        for (int k = 0; k < W; k += 4)
            *reinterpret_cast<float4 *>(p + k) = make_float4(y[k], y[k + 1], y[k + 2], y[k + 3]);
    } else if constexpr (OT == DT_E4M3) {
        uint8_t *p = reinterpret_cast<uint8_t *>(base) + e;
        uint32_t w[W / 4];
#pragma unroll
        for (int k = 0; k < W; k += 4)
            w[k / 4] = encode_out<OT>(y[k]) | (encode_out<OT>(y[k + 1]) << 8) |
                       (encode_out<OT>(y[k + 2]) << 16) | (encode_out<OT>(y[k + 3]) << 24);
        if constexpr (W == 4) *reinterpret_cast<uint32_t *>(p) = w[0];
        else *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(base) + e;
        uint32_t w[W / 2];
#pragma unroll
        for (int k = 0; k < W; k += 2) w[k / 2] = encode_out<OT>(y[k]) | (encode_out<OT>(y[k + 1]) << 16);
        if constexpr (W == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int OT, int W>
__device__ __forceinline__ void store_zero_chunk(void *base, int64_t e) {
    float z[W];
#pragma unroll
    for (int k = 0; k < W; ++k) z[k] = 0.0f;
    store_chunk<OT, W>(base, e, z);
}

// ------------------------------------------------------------------ the row

// One Q or K head row held as x[m][k] (dim 8W m + W c + k of lane c): RMS normalisation with
// weight w, then the rotation of the lane's pairs.  Binary32, one rounding per operation, the
// halving reduction tree of the contract, no contraction (built with -ffp-contract=off).
template <int W, int M>
__device__ __forceinline__ void norm_rope_row(float (&x)[M][W], const float (&w)[M][W], float eps,
                                              float inv_d, const float (&cs)[M][W / 2],
                                              const float (&sn)[M][W / 2],
                                              const bool (&rot)[M][W / 2]) {
    float a[M][W];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int k = 0; k < W; ++k) a[m][k] = x[m][k] * x[m][k];
    // tree levels o = 8W M/2 .. 8W: chunk m folds chunk m + om, inside the lane
#pragma unroll
    for (int om = M / 2; om >= 1; om /= 2)
#pragma unroll
        for (int m = 0; m < om; ++m)
#pragma unroll
            for (int k = 0; k < W; ++k) a[m][k] = a[m][k] + a[m + om][k];
    // levels 4W, 2W, W: lanes c and c + 4, c + 2, c + 1 of the token's 8 lanes
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_xor4(a[0][k]);
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_xor2(a[0][k]);
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_xor1(a[0][k]);
    // levels W/2 .. 1 inside the chunk
#pragma unroll
    for (int o = W / 2; o >= 1; o /= 2)
#pragma unroll
        for (int k = 0; k < o; ++k) a[0][k] = a[0][k] + a[0][k + o];
    const float ms = a[0][0] * inv_d;
    const float v = ms + eps;
    const float sq = __builtin_sqrtf(v);  // correctly rounded
    const float r = 1.0f / sq;            // correctly rounded
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const float t = x[m][k] * r;
            x[m][k] = t * w[m][k];
        }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const float e = x[m][2 * q], f = x[m][2 * q + 1];
            const float c = cs[m][q], s = sn[m][q];
            const float ec = e * c, fs = f * s, es = e * s, fc = f * c;
            const float e2 = ec - fs, f2 = es + fc;
            x[m][2 * q] = rot[m][q] ? e2 : e;
            x[m][2 * q + 1] = rot[m][q] ? f2 : f;
        }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// ------------------------------------------------------------------ the kernel

template <int D, int IN, int QT, int KT, int MODE>
__global__ __launch_bounds__(256) void qk_kernel(const QkParams p) {
    constexpr int W = (D == 64) ? 4 : 8;
    constexpr int M = D / (8 * W);
    constexpr int VC = D / 64;  // 16-byte V chunks per lane
    constexpr int U = (D == 64) ? 4 : 2;  // heads whose loads are in flight together
    static_assert(M >= 1 && 8 * W * M == D, "layout");

    const int lane = threadIdx.x & 63;
    const int c = lane & 7;
    const int g = lane >> 3;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const float inv_d = 1.0f / (float)D;

    // pair map of this lane: chunk m, pair q -> (axis, frequency); fixed for the whole kernel
    int paxis[M][W / 2], pj[M][W / 2];
    bool rot[M][W / 2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const int pr = (8 * W * m + W * c + 2 * q) >> 1;
            rot[m][q] = pr < 3 * p.n;
            paxis[m][q] = rot[m][q] ? pr / p.n : 0;
            pj[m][q] = rot[m][q] ? pr - paxis[m][q] * p.n : 0;
        }
    float wq[M][W], wk[M][W];
    {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < W; k += 4) {
                const float4 a = *reinterpret_cast<const float4 *>(p.wq + 8 * W * m + W * c + k);
                const float4 b = *reinterpret_cast<const float4 *>(p.wk + 8 * W * m + W * c + k);
                wq[m][k] = a.x; wq[m][k + 1] = a.y; wq[m][k + 2] = a.z; wq[m][k + 3] = a.w;
                wk[m][k] = b.x; wk[m][k + 1] = b.y; wk[m][k + 2] = b.z; wk[m][k + 3] = b.w;
            }
    }
    float ds[2] = {1.0f, 1.0f};
    if constexpr (MODE == MODE_CAST) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float am = p.amax[s];
            ds[s] = am > 0.0f ? am / 448.0f : 1.0f;
        }
        if (wave0 == 0 && lane == 0) {
            p.descale[0] = ds[0];
            p.descale[1] = ds[1];
        }
    }
    uint32_t mx[2] = {0u, 0u};  // MODE_AMAX: max of |y'| bits (NaN above +inf)

    for (int64_t item = wave0; item < p.items; item += nwaves) {
        const int hc = (int)(item % p.head_chunks);
        const int64_t bgi = item / p.head_chunks;
        const int tg = (int)(bgi % p.groups);
        const int b = (int)(bgi / p.groups);
        const int i = tg * 8 + g;
        if (i >= p.T) continue;  // ragged tail: the token's 8 lanes skip together
        const bool valid = i < p.vlen[b];
        if (MODE == MODE_AMAX && !valid) continue;
        const int h0 = hc * p.heads_per_chunk;
        const int h1 = min(p.H, h0 + p.heads_per_chunk);

        float cs[M][W / 2], sn[M][W / 2];
        if (valid) {
            const int pt = i / (p.Gh * p.Gw) + p.off[b][0];
            const int ph = (i / p.Gw) % p.Gh + p.off[b][1];
            const int pw = i % p.Gw + p.off[b][2];
            const int rowoff[3] = {pt * p.n, (p.base_h + ph) * p.n, (p.base_w + pw) * p.n};
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int q = 0; q < W / 2; ++q) {
                    const int a = paxis[m][q];
                    const int idx = (a == 0 ? rowoff[0] : (a == 1 ? rowoff[1] : rowoff[2])) + pj[m][q];
                    cs[m][q] = rot[m][q] ? p.cos_tab[idx] : 1.0f;
                    sn[m][q] = rot[m][q] ? p.sin_tab[idx] : 0.0f;
                }
        }

        const uint16_t *tok = p.qkv + (int64_t)b * p.batch_stride + (int64_t)i * p.row_stride;
        if (!valid) {
            if constexpr (MODE != MODE_AMAX) {
                for (int h = h0; h < h1; ++h) {
                    const int64_t orow = (((int64_t)b * p.H + h) * p.T + i) * D;
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        store_zero_chunk<QT, W>(p.q, orow + 8 * W * m + W * c);
                        store_zero_chunk<KT, W>(p.k, orow + 8 * W * m + W * c);
                    }
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
                        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.v) + orow + 64 * vc + 8 * c) =
                            make_uint4(0, 0, 0, 0);
                }
            }
            continue;
        }
        // heads in batches of U: every load of the batch is issued before its first use
        for (int hb = h0; hb < h1; hb += U) {
            uint32_t rq[U][M][W / 2], rk[U][M][W / 2];
            uint4 rv[U][VC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = hb + u;
                if (h >= h1) break;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    load_chunk<W>(tok + (int64_t)h * D + 8 * W * m + W * c, rq[u][m]);
                    load_chunk<W>(tok + (int64_t)(p.H + h) * D + 8 * W * m + W * c, rk[u][m]);
                }
                if constexpr (MODE != MODE_AMAX) {
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
                        rv[u][vc] = *reinterpret_cast<const uint4 *>(tok + (int64_t)(2 * p.H + h) * D + 64 * vc + 8 * c);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = hb + u;
                if (h >= h1) break;
                float xq[M][W], xk[M][W];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W / 2; ++k) {
                        xq[m][2 * k] = in_to_f32<IN>(rq[u][m][k] & 0xFFFFu);
                        xq[m][2 * k + 1] = in_to_f32<IN>(rq[u][m][k] >> 16);
                        xk[m][2 * k] = in_to_f32<IN>(rk[u][m][k] & 0xFFFFu);
                        xk[m][2 * k + 1] = in_to_f32<IN>(rk[u][m][k] >> 16);
                    }
                norm_rope_row<W, M>(xq, wq, p.eps, inv_d, cs, sn, rot);
                norm_rope_row<W, M>(xk, wk, p.eps, inv_d, cs, sn, rot);
                if constexpr (MODE == MODE_AMAX) {
#pragma unroll
                    for (int m = 0; m < M; ++m)
#pragma unroll
                        for (int k = 0; k < W; ++k) {
                            mx[0] = max(mx[0], __float_as_uint(xq[m][k]) & 0x7FFFFFFFu);
                            mx[1] = max(mx[1], __float_as_uint(xk[m][k]) & 0x7FFFFFFFu);
                        }
                } else {
                    if constexpr (MODE == MODE_CAST) {
#pragma unroll
                        for (int m = 0; m < M; ++m)
#pragma unroll
                            for (int k = 0; k < W; ++k) {
                                xq[m][k] = xq[m][k] / ds[0];
                                xk[m][k] = xk[m][k] / ds[1];
                            }
                    }
                    const int64_t orow = (((int64_t)b * p.H + h) * p.T + i) * D;
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        store_chunk<QT, W>(p.q, orow + 8 * W * m + W * c, xq[m]);
                        store_chunk<KT, W>(p.k, orow + 8 * W * m + W * c, xk[m]);
                    }
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
                        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.v) + orow + 64 * vc + 8 * c) = rv[u][vc];
                }
            }
        }
    }
    if constexpr (MODE == MODE_AMAX) {
        const uint32_t m0 = wave_max_u32(mx[0]);
        const uint32_t m1 = wave_max_u32(mx[1]);
        if (lane == 0) {
            if (m0) atomicMax(reinterpret_cast<unsigned int *>(p.amax), m0);
            if (m1) atomicMax(reinterpret_cast<unsigned int *>(p.amax) + 1, m1);
        }
    }
}

__global__ void clear2_kernel(float *a) {
    if (threadIdx.x < 2) a[threadIdx.x] = 0.0f;
}

// ------------------------------------------------------------------ dispatch

template <int D, int IN, int QT, int KT, int MODE>
int launch_one(QkParams &p, hipStream_t stream, std::string *err) {
    auto kern = qk_kernel<D, IN, QT, KT, MODE>;
    static int max_blocks = 0;  // resident blocks per CU for this instantiation
    static int cus = 0;
    if (max_blocks == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&max_blocks, kern, 256, 0) != hipSuccess ||
            max_blocks <= 0) {
            max_blocks = 0;
            *err = "device query failed (no HIP device?)";
            return H3_ELAUNCH;
        }
    }
    const int64_t waves_needed = p.items;
    int64_t blocks = (waves_needed + 3) / 4;
    const int64_t cap = (int64_t)max_blocks * cus;
    if (blocks > cap) blocks = cap;
    if (MODE == MODE_AMAX) {
        hipLaunchKernelGGL(clear2_kernel, dim3(1), dim3(64), 0, stream, p.amax);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) {
            *err = std::string("amax clear launch failed: ") + hipGetErrorString(e0);
            return H3_ELAUNCH;
        }
    }
    void *args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3((unsigned)blocks),
                                   dim3(256), args, 0, stream);
    if (e != hipSuccess) {
        *err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

template <int D, int IN, int MODE>
int dispatch_out(int q_dt, int k_dt, QkParams &p, hipStream_t s, std::string *err) {
    if constexpr (MODE == MODE_STORE) {
#define H3_QK(QT, KT) \
    if (q_dt == QT && k_dt == KT) return launch_one<D, IN, QT, KT, MODE>(p, s, err);
        H3_QK(DT_F32, DT_F16) H3_QK(DT_F32, DT_BF16) H3_QK(DT_F32, DT_F32)
        H3_QK(DT_F16, DT_F16) H3_QK(DT_F16, DT_BF16) H3_QK(DT_F16, DT_F32)
        H3_QK(DT_BF16, DT_F16) H3_QK(DT_BF16, DT_BF16) H3_QK(DT_BF16, DT_F32)
#undef H3_QK
    } else {
        return launch_one<D, IN, DT_E4M3, DT_E4M3, MODE>(p, s, err);
    }
    *err = "unsupported output dtype combination";
    return H3_EUNSUPPORTED;
}

template <int D, int MODE>
int dispatch_in(int in_dt, int q_dt, int k_dt, QkParams &p, hipStream_t s, std::string *err) {
    if (in_dt == DT_F16) return dispatch_out<D, DT_F16, MODE>(q_dt, k_dt, p, s, err);
    if (in_dt == DT_BF16) return dispatch_out<D, DT_BF16, MODE>(q_dt, k_dt, p, s, err);
    *err = "unsupported input dtype";
    return H3_EUNSUPPORTED;
}

template <int D>
int dispatch_mode(int mode, int in_dt, int q_dt, int k_dt, QkParams &p, hipStream_t s, std::string *err) {
    switch (mode) {
    case MODE_STORE: return dispatch_in<D, MODE_STORE>(in_dt, q_dt, k_dt, p, s, err);
    case MODE_AMAX: return dispatch_in<D, MODE_AMAX>(in_dt, q_dt, k_dt, p, s, err);
    default: return dispatch_in<D, MODE_CAST>(in_dt, q_dt, k_dt, p, s, err);
    }
}

}  // namespace

int launch_qk(int mode, int D, int in_dt, int q_dt, int k_dt, QkParams &p, hipStream_t stream,
              std::string *err) {
    if (D == 64) return dispatch_mode<64>(mode, in_dt, q_dt, k_dt, p, stream, err);
    if (D == 128) return dispatch_mode<128>(mode, in_dt, q_dt, k_dt, p, stream, err);
    *err = "unsupported head dim";
    return H3_EUNSUPPORTED;
}

}  // namespace h3
