// Device-side building blocks shared by the gfx950 kernels of libh3qk: element conversions,
// DPP butterflies, chunk loads and nontemporal stores, the normalised and rotated row in the
// lane layout described in h3qk_kernels.hip, rotary-table entries, the correctly rounded
// quotient and the E4M3 packing.  Internal: included by the kernel sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_internal.h"

namespace h3 {
namespace {

constexpr int DT_F32 = H3_F32, DT_F16 = H3_F16, DT_BF16 = H3_BF16, DT_E4M3 = H3_E4M3FN;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// The value as a materialised binary32: without this the compiler may fold a binary32 product of a
// 16-bit input and its conversion to binary16 into one mixed-precision FMA (v_fma_mixlo_f16), which
// rounds once where the contract rounds twice.
__device__ __forceinline__ float keep_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int OT>
__device__ __forceinline__ uint32_t encode_out(float x) {
    if constexpr (OT == DT_F16) return f32_to_f16_bits(x);
    else if constexpr (OT == DT_BF16) return f32_to_bf16_bits(x);
    else return f32_to_e4m3(x);
}

// ------------------------------------------------------------------ cross-lane butterflies

// Every source lane of these patterns exists, so bound_ctrl never applies; setting it lets the
// compiler fold the move into the consuming add (v_add_f32 with a DPP source).
__device__ __forceinline__ float lane_xor1(float v) {  // DPP quad_perm [1,0,3,2]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor2(float v) {  // DPP quad_perm [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_mirror8(float v) {  // DPP row_half_mirror: lane l <-> 7 - l
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
}

// Chunk held by lane l of a token's 8 lanes: l for l < 4, 11 - l for l >= 4.  Chunk ch + 4 then
// sits in the half-mirror lane 7 - ch, so the first cross-lane tree level pairs mirror lanes and
// the next two pair lanes l ^ 2 and l ^ 1 (lane l >= 4 stands for node 7 - l = l ^ 7, whose
// partners l ^ 7 ^ 2 and l ^ 7 ^ 1 live in lanes l ^ 2 and l ^ 1).  All three are DPP moves.
__device__ __forceinline__ int chunk_of_lane(int l) { return l < 4 ? l : 11 - l; }

// ------------------------------------------------------------------ loads and stores

// Element e of a wave-uniform 16-bit base, as a 32-bit byte offset (2e < 2^32, which the host's
// stride limits guarantee): the load then takes the scalar base plus a 32-bit lane offset instead of
// a 64-bit per-lane address.
__device__ __forceinline__ const uint16_t *at16(const uint16_t *base, uint32_t e) {
    return reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(base) + e * 2u);
}

// Entry e of a wave-uniform binary32 table, as a 32-bit byte offset (4e < 2^32: the host keeps
// every table under 2^30 entries).
__device__ __forceinline__ const float *atf32(const float *base, uint32_t e) {
    return reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + e * 4u);
}

// W consecutive 16-bit values (W = 4: 8 bytes, W = 8: 16 bytes) as W/2 packed words.
template <int W>
__device__ __forceinline__ void load_chunk(const uint16_t *p, uint32_t (&r)[W / 2]) {
    if constexpr (W == 4) {
        const u32x2 t = *reinterpret_cast<const u32x2 *>(p);
        r[0] = t.x; r[1] = t.y;
    } else {
        const u32x4 t = *reinterpret_cast<const u32x4 *>(p);
        r[0] = t.x; r[1] = t.y; r[2] = t.z; r[3] = t.w;
    }
}

// Raw buffer loads (no format conversion): word 3 of the descriptor, data format 32 bits.
constexpr int kRawBufferFlags = 0x00020000;

// W consecutive 16-bit values at byte offset voff + soff of a raw buffer (voff per lane, soff
// wave-uniform; both below the buffer's size, which bounds every access).
template <int W>
__device__ __forceinline__ void load_chunk_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff, uint32_t (&r)[W / 2]) {
    if constexpr (W == 4) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, soff, 0);
        r[0] = t[0]; r[1] = t[1];
    } else {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, soff, 0);
        r[0] = t[0]; r[1] = t[1]; r[2] = t[2]; r[3] = t[3];
    }
}

__device__ __forceinline__ void st_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(u32x2 *p, u32x2 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(f32x4 *p, f32x4 v) { __builtin_nontemporal_store(v, p); }

// Store W encoded values of one chunk in output dtype OT at element offset `e` of `base`.
template <int OT, int W>
__device__ __forceinline__ void store_codes(void *base, int64_t e, const uint32_t (&w)[W]) {
    if constexpr (OT == DT_E4M3) {
        uint8_t *p = reinterpret_cast<uint8_t *>(base) + e;
        uint32_t pk[W / 4];
#pragma unroll
        for (int k = 0; k < W; k += 4) pk[k / 4] = w[k] | (w[k + 1] << 8) | (w[k + 2] << 16) | (w[k + 3] << 24);
        if constexpr (W == 4) st_nt(reinterpret_cast<uint32_t *>(p), pk[0]);
        else st_nt(reinterpret_cast<u32x2 *>(p), (u32x2){pk[0], pk[1]});
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(base) + e;
        uint32_t pk[W / 2];
#pragma unroll
        for (int k = 0; k < W; k += 2) pk[k / 2] = w[k] | (w[k + 1] << 16);
        if constexpr (W == 4) st_nt(reinterpret_cast<u32x2 *>(p), (u32x2){pk[0], pk[1]});
        else st_nt(reinterpret_cast<u32x4 *>(p), (u32x4){pk[0], pk[1], pk[2], pk[3]});
    }
}

template <int OT, int W>
__device__ __forceinline__ void store_chunk(void *base, int64_t e, const float (&y)[W]) {
    if constexpr (OT == DT_F32) {
        float *p = reinterpret_cast<float *>(base) + e;
#pragma unroll
        for (int k = 0; k < W; k += 4)
            st_nt(reinterpret_cast<f32x4 *>(p + k), (f32x4){y[k], y[k + 1], y[k + 2], y[k + 3]});
    } else {
        uint32_t w[W];
#pragma unroll
        for (int k = 0; k < W; ++k) w[k] = encode_out<OT>(y[k]);
        store_codes<OT, W>(base, e, w);
    }
}

template <int OT, int W>
__device__ __forceinline__ void store_zero_chunk(void *base, int64_t e) {
    if constexpr (OT == DT_F32) {
        float *p = reinterpret_cast<float *>(base) + e;
#pragma unroll
        for (int k = 0; k < W; k += 4) st_nt(reinterpret_cast<f32x4 *>(p + k), (f32x4){0.f, 0.f, 0.f, 0.f});
    } else {
        uint32_t w[W];
#pragma unroll
        for (int k = 0; k < W; ++k) w[k] = 0u;
        store_codes<OT, W>(base, e, w);
    }
}

// Whole-row store of the lane's M = 2 chunks when a chunk is 8 bytes (16-bit outputs with W = 4,
// E4M3 codes with W = 8), given as two packed words per chunk: neighbouring lanes (chunks 2j and
// 2j + 1, always lanes l and l ^ 1 under chunk_of_lane) swap halves with one DPP move per word,
// so the even-chunk lane holds the 16 bytes of chunks 2j, 2j + 1 of the first half-row and the odd
// one those of the second half-row.  One 16-byte store per lane then writes the token's row as
// whole 128-byte lines, which reach HBM without relying on the L2 to merge half-line writes.
template <int EB, int W>
__device__ __forceinline__ void store_words_pairs(void *base, int64_t row_e, int c, const uint32_t (&m0)[2],
                                                  const uint32_t (&m1)[2]) {
    static_assert(EB * W == 8, "8-byte chunks");
    const bool odd = c & 1;
    const uint32_t s0 = odd ? m0[0] : m1[0], s1 = odd ? m0[1] : m1[1];
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0xB1, 0xF, 0xF, true);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0xB1, 0xF, 0xF, true);
    const u32x4 v = odd ? (u32x4){r0, r1, m1[0], m1[1]} : (u32x4){m0[0], m0[1], r0, r1};
    // even chunk 2j: elements [2j W, 2j W + 2W); odd chunk 2j + 1: [8W + 2j W, 8W + 2j W + 2W)
    const int64_t e = row_e + (odd ? 8 * W + (c - 1) * W : c * W);
    st_nt(reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(base) + e * EB), v);
}

// The same trade for 4-byte chunks (E4M3 codes with W = 4, one word per chunk): one 8-byte store per
// lane writes the token's 64-byte row whole, and the wave's 8 tokens 512 contiguous bytes.
__device__ __forceinline__ void store_word_pairs(void *base, int64_t row_e, int c, uint32_t m0, uint32_t m1) {
    const bool odd = c & 1;
    const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? m0 : m1), 0xB1, 0xF, 0xF, true);
    const u32x2 v = odd ? (u32x2){r, m1} : (u32x2){m0, r};
    // even chunk 2j: bytes [8j, 8j + 8); odd chunk 2j + 1: [32 + 8j, 32 + 8j + 8)
    const int64_t e = row_e + (odd ? 32 + 4 * (c - 1) : 4 * c);
    st_nt(reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(base) + e), v);
}

template <int OT, int W>
__device__ __forceinline__ void store_row_pairs(void *base, int64_t row_e, int c, const float (&y)[2][W]) {
    static_assert((OT == DT_F16 || OT == DT_BF16) && W == 4, "16-bit outputs, 4-wide chunks");
    uint32_t m0[2], m1[2];
    m0[0] = encode_out<OT>(y[0][0]) | (encode_out<OT>(y[0][1]) << 16);
    m0[1] = encode_out<OT>(y[0][2]) | (encode_out<OT>(y[0][3]) << 16);
    m1[0] = encode_out<OT>(y[1][0]) | (encode_out<OT>(y[1][1]) << 16);
    m1[1] = encode_out<OT>(y[1][2]) | (encode_out<OT>(y[1][3]) << 16);
    store_words_pairs<2, W>(base, row_e, c, m0, m1);
}

// W E4M3 codes (W / 4 packed words) at element e.
template <int W>
__device__ __forceinline__ void store_code_words(void *base, int64_t e, const uint32_t (&w)[W / 4]) {
    uint8_t *p = reinterpret_cast<uint8_t *>(base) + e;
    if constexpr (W == 4) st_nt(reinterpret_cast<uint32_t *>(p), w[0]);
    else st_nt(reinterpret_cast<u32x2 *>(p), (u32x2){w[0], w[1]});
}

template <int OT, int W, int M>
constexpr bool kPairStore = M == 2 && (OT == DT_F16 || OT == DT_BF16) && W == 4;

// Binary32 rows at W = 8, M = 2 (a chunk is 32 bytes, two 16-byte halves).  Chunk j < 4 (lane j) and
// chunk j + 4 (its half-mirror lane 7 - j) trade halves, so that each of the row's four store
// instructions writes one whole 128-byte quarter of the row across the token's 8 lanes: the low
// lane writes its own first half, then the high lane's first half (32 floats further on); the high
// lane writes the low lane's second half, then its own second half.  Stored chunk by chunk, every
// instruction would write half of each of two lines (measured on the FP8 long-sequence shape with
// binary32 Q and K: 1183 us per store pass).
template <int OT, int W, int M>
constexpr bool kF32PairStore = M == 2 && OT == DT_F32 && W == 8;

// Element offset, from the row's start, of the lane's first 16-byte store for chunk c.
__device__ __forceinline__ uint32_t f32_pair_offset(int c) { return 8u * (uint32_t)(c & 3) + ((c & 4) ? 4u : 0u); }

// `src` from the half-mirror lane for the lanes of the DPP banks in BANKS (4-lane groups of a
// 16-lane row: 0x5 = lanes 0-3 of each 8, 0xA = lanes 4-7); the other lanes keep `old`.
template <int BANKS>
__device__ __forceinline__ float mirror8_into(float old, float src) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), 0x141, 0xF, BANKS, false));
}

template <int W>
__device__ __forceinline__ void store_f32_row_pairs(void *base, int64_t row_e, int c, const float (&y)[2][W]) {
    static_assert(W == 8, "32-byte chunks");
    float *p = reinterpret_cast<float *>(base) + row_e + f32_pair_offset(c);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        f32x4 a, b;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[k] = mirror8_into<0xA>(y[m][k], y[m][k + 4]);  // high lanes: the low lane's second half
            b[k] = mirror8_into<0x5>(y[m][k + 4], y[m][k]);  // low lanes: the high lane's first half
        }
        st_nt(reinterpret_cast<f32x4 *>(p + 64 * m), a);
        st_nt(reinterpret_cast<f32x4 *>(p + 64 * m + 32), b);
    }
}

// A zero binary32 row at W = 8, M = 2, with the same whole-line stores.
__device__ __forceinline__ void store_f32_zero_row_pairs(void *base, int64_t row_e, int c) {
    float *p = reinterpret_cast<float *>(base) + row_e + f32_pair_offset(c);
#pragma unroll
    for (int q = 0; q < 4; ++q) st_nt(reinterpret_cast<f32x4 *>(p + 32 * q), (f32x4){0.f, 0.f, 0.f, 0.f});
}

// ------------------------------------------------------------------ the row

// One Q or K head row is held as x[m][k] (dim 8W m + W c + k, c the lane's chunk).  Binary32,
// one rounding per operation, the halving reduction tree of the contract, no contraction (built
// with -ffp-contract=off).

// Sum of squares of the row over the halving tree; every lane of the token ends with it.
template <int W, int M>
__device__ __forceinline__ float row_sumsq(const float (&x)[M][W]) {
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
    // levels 4W, 2W, W across the token's 8 lanes (see chunk_of_lane)
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_mirror8(a[0][k]);
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_xor2(a[0][k]);
#pragma unroll
    for (int k = 0; k < W; ++k) a[0][k] = a[0][k] + lane_xor1(a[0][k]);
    // levels W/2 .. 1 inside the chunk
#pragma unroll
    for (int o = W / 2; o >= 1; o /= 2)
#pragma unroll
        for (int k = 0; k < o; ++k) a[0][k] = a[0][k] + a[0][k + o];
    return a[0][0];
}

// RN(1 / RN(sqrt(v))) for v >= 2^-96, +inf or NaN, without the rescaling the compiler's correctly
// rounded square root applies to tiny inputs: the hardware square root corrected to its correctly
// rounded neighbour by the signs of the two FMA residuals, then the hardware reciprocal with one
// FMA Newton step.  Checked bit for bit against 1.0f / sqrtf(v) (both correctly rounded) for every
// binary32 v in [2^-96, +inf] and every NaN pattern.  (The reciprocal step alone is not correctly
// rounded where 1/b is subnormal, b >= 2^126; a square root here is at most 2^64.)
// Special inputs need no select: for v = +inf or NaN both residuals are NaN, neither comparison
// holds and q stays the hardware result; for q = +inf the Newton residual -inf * 0 + 1 is NaN, which
// the minimum with 1 (IEEE minNum returns the number) turns into 1, so y1 = y0 = +0.  For finite q
// the residual is below 2^-21 in magnitude and the minimum leaves it alone.
__device__ __forceinline__ float rsqrt_rn_large(float v) {
    const float s = __builtin_amdgcn_sqrtf(v);
    const float sdn = __uint_as_float(__float_as_uint(s) - 1u);
    const float sup = __uint_as_float(__float_as_uint(s) + 1u);
    const float rdn = __builtin_fmaf(-sdn, s, v);
    const float rup = __builtin_fmaf(-sup, s, v);
    float q = rdn <= 0.0f ? sdn : s;
    q = rup > 0.0f ? sup : q;
    const float y0 = __builtin_amdgcn_rcpf(q);
    const float e = __builtin_fminf(__builtin_fmaf(-q, y0, 1.0f), 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// r = 1 / sqrt(ss * (1/D) + eps): correctly rounded sqrt, then correctly rounded division.  With
// eps >= 2^-96 (a kernel-wide condition) v >= eps and the shorter sequence above gives the same bits.
__device__ __forceinline__ float row_rstd(float ss, float inv_d, float eps) {
    const float ms = ss * inv_d;
    const float v = ms + eps;
    if (eps >= 0x1p-96f) return rsqrt_rn_large(v);
    const float sq = __builtin_sqrtf(v);
    return 1.0f / sq;
}

// y = (x r) w, then the rotation of the lane's pairs.
template <int W, int M>
__device__ __forceinline__ void row_scale_rotate(float (&x)[M][W], float r, const float (&w)[M][W],
                                                 const float (&cs)[M][W / 2], const float (&sn)[M][W / 2],
                                                 const bool (&rot)[M][W / 2]) {
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

template <int J>
__device__ __forceinline__ float quad_bcast(float v) {  // DPP quad_perm [J,J,J,J]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), J * 0x55, 0xF, 0xF, true));
}

// The 1/rms of up to 4 rows of a token with one square root and one division per lane: lane l of
// each quad takes row l, and a DPP quad broadcast hands row j's value to every lane.  The 8 lanes
// of a token are two quads, and both compute the same rows.
template <int R>
__device__ __forceinline__ void rows_rstd(const float (&ss)[R], int lane, float inv_d, float eps, float (&r)[R]) {
    static_assert(R >= 1 && R <= 4, "one quad");
    const int lr = lane & 3;
    float mine = ss[0];
#pragma unroll
    for (int j = 1; j < R; ++j) mine = lr == j ? ss[j] : mine;
    const float rm = row_rstd(mine, inv_d, eps);
    r[0] = quad_bcast<0>(rm);
    if constexpr (R > 1) r[1] = quad_bcast<1>(rm);
    if constexpr (R > 2) r[2] = quad_bcast<2>(rm);
    if constexpr (R > 3) r[3] = quad_bcast<3>(rm);
}

template <int W, int M, int IN>
__device__ __forceinline__ void unpack_row(const uint32_t (&r)[M][W / 2], float (&x)[M][W]) {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int k = 0; k < W / 2; ++k) {
            x[m][2 * k] = in_to_f32<IN>(r[m][k] & 0xFFFFu);
            x[m][2 * k + 1] = in_to_f32<IN>(r[m][k] >> 16);
        }
}

template <int W, int M>
__device__ __forceinline__ void load_weights(const float *wsrc, int c, float (&w)[M][W]) {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int k = 0; k < W; k += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(wsrc + 8 * W * m + W * c + k);
            w[m][k] = a.x; w[m][k + 1] = a.y; w[m][k + 2] = a.z; w[m][k + 3] = a.w;
        }
}

// Rotary entries of this lane's pairs for token i of item b.  Pair index pr (the dims 2 pr,
// 2 pr + 1) rotates when pr < 3n, on axis pr / n at frequency pr mod n.  NN is n when it is known
// at compile time (the natural split n = D / 8), else 0 and n is read from the parameters; the
// axis then comes from floor((pr + 1/2) / n) in binary32, exact because pr + 1/2 is never a
// multiple of n and the rounding error is far below the 1/(2n) margin for pr < 128.  With NN
// known, chunks whose pairs all rotate (or none does) need no per-lane test.
// PAIRS = false keeps one 4-byte load per entry (where the pair loads' registers would cost a wave).
template <int W, int M, int NN, bool PAIRS = true>
__device__ __forceinline__ void rotary_entries(const QkParams &p, int b, int i, int c,
                                               float (&cs)[M][W / 2], float (&sn)[M][W / 2],
                                               bool (&rot)[M][W / 2]) {
    const int n = NN ? NN : p.n;
    const uint32_t ui = (uint32_t)i;
    const uint32_t j = div_apply(ui, p.div_gw);   // i / Gw
    const uint32_t tq = div_apply(j, p.div_gh);   // i / (Gh Gw)
    const int row_t = (int)tq + p.off[b][0];
    const int row_h = p.base_h + (int)(j - tq * (uint32_t)p.Gh) + p.off[b][1];
    const int row_w = p.base_w + (int)(ui - j * (uint32_t)p.Gw) + p.off[b][2];
    if constexpr (PAIRS && NN != 0 && NN % 2 == 0 && W == 4) {
        // The lane's two pairs of a chunk start at an even pair index, so they sit on one axis (n is
        // even) and rotate alike (3 n is even); their entries are neighbours at an even table
        // position, which with 8-byte aligned tables load as one 8-byte access per table.
        if (p.tab_pairs) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int pr = 4 * W * m + (W / 2) * c;
                const bool r = (4 * W * m + 4 * W <= 3 * NN) ? true : (4 * W * m >= 3 * NN) ? false : pr < 3 * NN;
                const int axis = pr / NN;
                const int row = axis == 0 ? row_t : (axis == 1 ? row_h : row_w);
                const uint32_t idx = (uint32_t)(row * NN + (pr - axis * NN));  // even; < 2^30
                float2 cv = make_float2(1.0f, 1.0f), sv = make_float2(0.0f, 0.0f);
                if (r) {
                    cv = *reinterpret_cast<const float2 *>(atf32(p.cos_tab, idx));
                    sv = *reinterpret_cast<const float2 *>(atf32(p.sin_tab, idx));
                }
                cs[m][0] = cv.x; cs[m][1] = cv.y;
                sn[m][0] = sv.x; sn[m][1] = sv.y;
                rot[m][0] = r; rot[m][1] = r;
            }
            return;
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const int pr = 4 * W * m + (W / 2) * c + q;  // chunk m spans pairs [4W m, 4W m + 4W)
            if (NN && 4 * W * m + 4 * W <= 3 * NN) rot[m][q] = true;
            else if (NN && 4 * W * m >= 3 * NN) rot[m][q] = false;
            else rot[m][q] = pr < 3 * n;
            const int axis = NN ? pr / (NN ? NN : 1) : (int)(((float)pr + 0.5f) * p.inv_n);
            const int jj = pr - axis * n;
            const int row = axis == 0 ? row_t : (axis == 1 ? row_h : row_w);
            const uint32_t idx = (uint32_t)(row * n + jj);  // < 2^30 (checked on the host)
            cs[m][q] = rot[m][q] ? *atf32(p.cos_tab, idx) : 1.0f;
            sn[m][q] = rot[m][q] ? *atf32(p.sin_tab, idx) : 0.0f;
        }
}

// RN(y / ds) without a division instruction, for a descale ds in [2^-60, 2^60] with
// rcp = RN(1 / ds): q0 = RN(y rcp) is within one ulp of RN(y / ds), and one FMA remainder
// correction, RN(q0 - (q0 ds - y) rcp), gives RN(y / ds) itself: the final step of Markstein's
// division (IBM J. Res. Dev. 34(1), 1990), whose theorem asks for a correctly rounded reciprocal,
// a starting quotient within one ulp of y / ds and an exact remainder.  q0 is not proven faithful
// here; the sequence is instead checked against correctly rounded division for every pair of
// significands of y and ds (2^46 quotients; exact power-of-two scaling carries that over to every
// descale in the range and every quotient in [2^-12, 512)), and for every finite binary32 y at 80
// descales: the same bits wherever |y / ds| is in [2^-12, 512), the same E4M3 code below (every
// value under 2^-10 encodes to a signed zero code), NaN or past 448 above.  The remainder is taken
// negated, e = q0 ds - y (exact, like y - q0 ds), and enters through the FMA's negation modifier:
// a zero y keeps its sign (-0 + -0 = -0), with no fix-up.  The result is a correctly rounded
// division, so the no-contraction rule of the arithmetic chain is untouched.
__device__ __forceinline__ float quotient(float y, float ds, float rcp) {
    const float q0 = y * rcp;
    const float e0 = __builtin_fmaf(q0, ds, -y);
    return __builtin_fmaf(-e0, rcp, q0);
}

// A non-NaN quotient brought into the E4M3 range [-448, 448] (v_med3; +-inf included) ahead of the
// conversion instruction: the encoder saturates everything past 448 to +-448, so the code of the
// clamped value is the code of the value.
__device__ __forceinline__ float clamp_e4m3(float q) { return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f); }

// Codes of W quotients as W/4 packed words.  hw: the conversion instruction, exact for |q| <= 448
// (the caller guarantees that range); otherwise the integer encoder (saturation, NaN).
template <int W>
__device__ __forceinline__ void pack_e4m3(const float (&q)[W], bool hw, uint32_t (&w)[W / 4]) {
#pragma unroll
    for (int k = 0; k < W; k += 4) {
        if (hw) {
            int t = __builtin_amdgcn_cvt_pk_fp8_f32(q[k], q[k + 1], 0, false);
            w[k / 4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[k + 2], q[k + 3], t, true);
        } else {
            w[k / 4] = f32_to_e4m3(q[k]) | (f32_to_e4m3(q[k + 1]) << 8) | (f32_to_e4m3(q[k + 2]) << 16) |
                       (f32_to_e4m3(q[k + 3]) << 24);
        }
    }
}

// Running largest |y| over binary32 values.  gfx950's three-input IEEE 754-2019 maximum takes
// both values through its absolute-value source modifiers, so one instruction folds two values in;
// a NaN operand makes the result NaN (maximum, unlike maxNum, propagates it), +0 and -0 both enter
// as +0, and subnormal magnitudes are compared as they are (the kernels run with binary32
// denormals on).  The result is non-negative, so its bits order like its value, NaN above +inf.
struct MagMax {
    float m = 0.0f;
    // written as the instruction itself: left to itself the compiler may rebuild the unrolled
    // chain into a tree of two-input maxima
    __device__ __forceinline__ void add2(float a, float b) {
        asm("v_maximum3_f32 %0, %0, |%1|, |%2|" : "+v"(m) : "v"(a), "v"(b));
    }
    __device__ __forceinline__ uint32_t bits() const { return __float_as_uint(m) & 0x7FFFFFFFu; }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// E4M3 codes of the M x W values y / ds of one tensor (ds its descale, rcp = RN(1 / ds), fast: ds
// within the quotient's checked range), four codes per word.  The quotients are correctly rounded
// (quotient()); the decisions are wave-uniform: a NaN quotient or a descale outside the checked
// range sends the whole wave through correctly rounded division and the integer encoder; quotients
// past 448 are clamped with v_med3 ahead of the conversion instruction.  With count, the quotients
// past 448 over the wave's active lanes are added to nsat (a wave-uniform value).
template <int M, int W>
__device__ __forceinline__ void cast_e4m3_wave(const float (&y)[M][W], float ds, float rcp, bool fast, bool count,
                                               uint32_t &nsat, uint32_t (&w)[M][W / 4]) {
    float q[M][W];
    MagMax qm;  // the lane's largest |quotient| (NaN if any is NaN): one instruction per two values
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int k = 0; k < W; k += 2) {
            q[m][k] = quotient(y[m][k], ds, rcp);
            q[m][k + 1] = quotient(y[m][k + 1], ds, rcp);
            qm.add2(q[m][k], q[m][k + 1]);
        }
    const bool bad = !(qm.m <= 448.0f);  // a quotient above 448 in magnitude or NaN
    bool exact = !fast, clip = false;
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
        // the running maximum is NaN exactly when one of the lane's quotients is (one compare per
        // lane instead of one per value: the clipping static cast 617 -> 597 us)
        exact = exact || __builtin_amdgcn_ballot_w64(qm.m != qm.m) != 0;
        clip = true;
    }
    if (exact) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < W; ++k)
                if (!fast || !(__builtin_fabsf(q[m][k]) <= 448.0f)) q[m][k] = y[m][k] / ds;
    }
    if (count && (clip || exact)) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < W; ++k)
                nsat += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(q[m][k]) > 448.0f));
    }
    if (clip && !exact) {  // no NaN here
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < W; ++k) q[m][k] = clamp_e4m3(q[m][k]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) pack_e4m3<W>(q[m], !exact, w[m]);
}

}  // namespace
}  // namespace h3
