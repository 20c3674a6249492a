// gfx950 kernels for the MiniMax-H3 QK preparation: per-head RMSNorm + partial 3-axis RoPE +
// head-major permute ([SDCPP-19] fused QKV / ggml_rope_pe_permute_rms commits, [OMNI-6607]
// Operations table), and the FP8 amax and E4M3 cast passes ([TRT-21485] Summary and
// fused_fp8_qk commits).  The numerical contract is stated in include/h3qk.h.
//
// Work decomposition (wave64):
//   * A work item is 8 consecutive tokens of one item and 2 of its heads.  Lane 8 g + l serves
//     token g of the 8 and holds, of every head row it touches, the dims
//     {8W m + W c + k : m < M, k < W} of its chunk c = chunk_of_lane(l), with W = 4, M = 2 for
//     D = 64 and W = 8, M = 2 for D = 128.  Loads are 8 W contiguous bytes per token per instruction, the f32 Q store of a
//     D = 64 row is two full 128-byte lines, V moves in 16-byte lanes.
//   * The halving reduction tree maps onto that layout as: levels o >= 8W fold chunks inside
//     the lane, levels 4W, 2W, W are DPP butterflies across the token's 8 lanes (half-mirror,
//     then xor 2, then xor 1), levels below W fold inside the chunk.  Floating-point addition is
//     commutative, so the butterfly partner computes the same bits as the tree node, and all
//     8 lanes end with ss.
//   * Store and cast passes: one work item per wave, one short-lived 4-wave block per 8 tokens
//     x 8 heads.  Blocks are dispatched in order, so the chip writes a narrow sliding window of
//     each head plane of the [B, H, T, D] outputs; on MI355X that keeps HBM write efficiency
//     well above a persistent grid-stride sweep, which holds a window of every plane open.
//     Each wave issues its data loads first, then decodes positions and fetches weights and
//     rotary entries while the loads are in flight.  Outputs are written once and never read
//     back, so they bypass the caches (nontemporal stores), each row as whole 128-byte lines.
//     At most 3 blocks are resident per CU (see kStoreBlocksPerCU).
//   * Amax pass: persistent waves over the work items with the next item's loads in flight
//     while the current one is reduced, one atomic max per block and tensor.  It stores nothing,
//     so it always takes W = 4 (M = D / 32), which keeps the cross-lane tree levels at 12 DPP adds
//     per row.
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

// r = 1 / sqrt(ss * (1/D) + eps): correctly rounded sqrt, then correctly rounded division.
__device__ __forceinline__ float row_rstd(float ss, float inv_d, float eps) {
    const float ms = ss * inv_d;
    const float v = ms + eps;
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
template <int W, int M, int NN>
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
            const int idx = row * n + jj;
            cs[m][q] = rot[m][q] ? p.cos_tab[idx] : 1.0f;
            sn[m][q] = rot[m][q] ? p.sin_tab[idx] : 0.0f;
        }
}

// RN(y / ds) without a division instruction, for a descale ds in [2^-60, 2^60] with
// rcp = RN(1 / ds): q0 = RN(y rcp) is within 1.5 ulps of y / ds, one FMA remainder correction makes
// it faithful, and a second one then gives the correctly rounded quotient (Markstein's theorem on
// correcting a faithful quotient with a correctly rounded reciprocal; IBM J. Res. Dev. 34(1), 1990).
// Checked against correctly rounded division for every binary32 y with y / ds in [2^-12, 512) and
// 80 descales.  The quotient's sign is that of y (ds > 0), which also fixes y = -0.  Quotients
// below 2^-11 may lose accuracy to underflow in the remainders, but every value under 2^-10
// encodes to a zero code either way.  The result is a correctly rounded division, so the
// no-contraction rule of the arithmetic chain is untouched.
__device__ __forceinline__ float quotient(float y, float ds, float rcp) {
    const float q0 = y * rcp;
    const float r0 = __builtin_fmaf(-q0, ds, y);
    const float q1 = __builtin_fmaf(r0, rcp, q0);
    const float r1 = __builtin_fmaf(-q1, ds, y);
    return __builtin_copysignf(__builtin_fmaf(r1, rcp, q1), y);
}

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

// ------------------------------------------------------------------ store / cast kernel

template <int D, int IN, int QT, int KT, int MODE, int NN, bool VF8>
__global__ __launch_bounds__(256) void qk_kernel(const QkParams p) {
    constexpr int W = (D == 64) ? 4 : 8;
    constexpr int M = D / (8 * W);
    constexpr int VC = D / 64;  // 16-byte V chunks per lane
    constexpr int HPW = kHeadsPerWave;
    static_assert(M >= 1 && 8 * W * M == D, "layout");
    static_assert(MODE == MODE_STORE || MODE == MODE_CAST, "store / cast kernel");
    static_assert(!VF8 || MODE == MODE_CAST, "V codes only in the cast pass");
    constexpr int NS = VF8 ? 3 : 2;  // scaled tensors: Q, K (and V)

    const int lane = threadIdx.x & 63;
    const int c = chunk_of_lane(lane & 7);  // chunk of the row this lane holds
    const int g = lane >> 3;
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    float ds[3] = {1.0f, 1.0f, 1.0f}, rcp[3] = {1.0f, 1.0f, 1.0f};
    bool fast = true;
    if constexpr (MODE == MODE_CAST) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float a = p.amax[s];
            // dynamic: amax / 448 (1 when amax is not > 0); static: the descale itself, 1 when not > 0
            ds[s] = a > 0.0f ? (p.static_scale ? a : a / 448.0f) : 1.0f;
            rcp[s] = 1.0f / ds[s];
            fast = fast && ds[s] >= 0x1p-60f && ds[s] <= 0x1p60f;
        }
        if (p.descale && item == 0 && lane == 0) {
#pragma unroll
            for (int s = 0; s < NS; ++s) p.descale[s] = ds[s];
        }
    }
    if (item >= p.items) return;

    const uint32_t it32 = (uint32_t)item;  // items < 2^31 (checked on the host)
    const uint32_t bgi = it32 / (uint32_t)p.head_chunks;
    const int hc = (int)(it32 - bgi * (uint32_t)p.head_chunks);
    const uint32_t b32 = bgi / (uint32_t)p.groups;
    const int tg = (int)(bgi - b32 * (uint32_t)p.groups);
    const int b = (int)b32;
    const int i = tg * 8 + g;
    if (i >= p.T) return;  // ragged tail: the token's 8 lanes leave together
    const int h0 = hc * HPW;
    const int nh = min(HPW, p.H - h0);
    // Uniform bases (the wave's first token, head h0) and small per-lane offsets, so memory
    // instructions take a scalar base with a 32-bit lane offset.
    const int64_t plane = (int64_t)p.T * D;
    const int64_t obase = (((int64_t)b * p.H + h0) * p.T + (int64_t)tg * 8) * D;  // (b, h0, 8 tg, 0)
    const uint32_t olane = (uint32_t)g * D;

    if (i >= p.vlen[b]) {  // padding token: +0 everywhere
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= nh) break;
            const int64_t o = obase + u * plane;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                store_zero_chunk<QT, W>(p.q, o + (olane + 8 * W * m + W * c));
                store_zero_chunk<KT, W>(p.k, o + (olane + 8 * W * m + W * c));
            }
            if constexpr (VF8) {  // D bytes per token row: 8 or 16 bytes per lane
                if constexpr (VC == 2)
                    st_nt(reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(p.v) + o + (olane + 16 * c)),
                          (u32x4){0u, 0u, 0u, 0u});
                else
                    st_nt(reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(p.v) + o + (olane + 8 * c)),
                          (u32x2){0u, 0u});
            } else {
#pragma unroll
                for (int vc = 0; vc < VC; ++vc)
                    st_nt(reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(p.v) + o + (olane + 64 * vc + 8 * c)),
                          (u32x4){0u, 0u, 0u, 0u});
            }
        }
        return;
    }

    // 1. every data load of the item, before anything that depends on them
    const uint16_t *tokb = p.qkv + (int64_t)b * p.batch_stride + (int64_t)tg * 8 * p.row_stride;
    const uint32_t tlane = (uint32_t)g * (uint32_t)p.row_stride;  // < 2^26 * 8 (checked on the host)
    uint32_t rq[HPW][M][W / 2], rk[HPW][M][W / 2];
    u32x4 rv[HPW][VC];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        if (u < nh) {
            const uint32_t hq = (uint32_t)(h0 + u) * D, hk = (uint32_t)(p.H + h0 + u) * D;
            const uint32_t hv = (uint32_t)(2 * p.H + h0 + u) * D;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                load_chunk<W>(tokb + (tlane + hq + 8 * W * m + W * c), rq[u][m]);
                load_chunk<W>(tokb + (tlane + hk + 8 * W * m + W * c), rk[u][m]);
            }
#pragma unroll
            for (int vc = 0; vc < VC; ++vc)
                rv[u][vc] = *reinterpret_cast<const u32x4 *>(tokb + (tlane + hv + 64 * vc + 8 * c));
        } else {  // absent head of an odd head count: zeros (their rows are never stored)
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int k = 0; k < W / 2; ++k) rq[u][m][k] = rk[u][m][k] = 0u;
        }
    }
    // 2. weights and rotary entries while the loads are in flight
    float wq[M][W], wk[M][W];
    load_weights<W, M>(p.wq, c, wq);
    load_weights<W, M>(p.wk, c, wk);
    float cs[M][W / 2], sn[M][W / 2];
    bool rot[M][W / 2];
    rotary_entries<W, M, NN>(p, b, i, c, cs, sn, rot);
    const float inv_d = 1.0f / (float)D;

    // 3. sums of squares of the 2 HPW rows and their 1/rms.  The ALU-bound cast shares one square
    // root and division per lane among the rows; the store pass keeps one per row, whose
    // independent chains hide latency better at 3 waves per SIMD (measured: shared is 7 % slower
    // on the full latent, 35 % on one tile).
    float x[HPW][2][M][W];
    float ss[2 * HPW], rr[2 * HPW];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        unpack_row<W, M, IN>(rq[u], x[u][0]);
        unpack_row<W, M, IN>(rk[u], x[u][1]);
        ss[2 * u] = row_sumsq<W, M>(x[u][0]);
        ss[2 * u + 1] = row_sumsq<W, M>(x[u][1]);
    }
    if constexpr (MODE == MODE_CAST) {
        rows_rstd<2 * HPW>(ss, lane, inv_d, p.eps, rr);
    } else {
#pragma unroll
        for (int j = 0; j < 2 * HPW; ++j) rr[j] = row_rstd(ss[j], inv_d, p.eps);
    }

    // 4. normalise, rotate, store
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        if (u >= nh) break;
        const int64_t o = obase + u * plane;
        float (&xq)[M][W] = x[u][0];
        float (&xk)[M][W] = x[u][1];
        row_scale_rotate<W, M>(xq, rr[2 * u], wq, cs, sn, rot);
        row_scale_rotate<W, M>(xk, rr[2 * u + 1], wk, cs, sn, rot);
        if constexpr (MODE == MODE_CAST) {
            float qq[2][M][W];
            float xv[VF8 ? VC : 1][8], qv[VF8 ? VC : 1][8];
            bool bad = false;  // a quotient above 448 in magnitude or NaN
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    qq[0][m][k] = quotient(xq[m][k], ds[0], rcp[0]);
                    qq[1][m][k] = quotient(xk[m][k], ds[1], rcp[1]);
                    bad = bad || !(__builtin_fabsf(qq[0][m][k]) <= 448.0f) || !(__builtin_fabsf(qq[1][m][k]) <= 448.0f);
                }
            if constexpr (VF8) {
#pragma unroll
                for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t wd = rv[u][vc][e >> 1];
                        xv[vc][e] = in_to_f32<IN>((e & 1) ? (wd >> 16) : (wd & 0xFFFFu));
                        qv[vc][e] = quotient(xv[vc][e], ds[2], rcp[2]);
                        bad = bad || !(__builtin_fabsf(qv[vc][e]) <= 448.0f);
                    }
            }
            // exact: NaN data or an extreme descale (rare): correctly rounded division where the
            // quotient is out of the checked range, and the integer encoder, for the whole wave.
            // clip: some quotient past the range (a descale below the data's amax / 448): it saturates.
            bool exact = !fast, clip = false;
            if (__builtin_amdgcn_ballot_w64(bad) != 0) {
                bool nan = false;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) nan = nan || qq[0][m][k] != qq[0][m][k] || qq[1][m][k] != qq[1][m][k];
                if constexpr (VF8) {
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                        for (int e = 0; e < 8; ++e) nan = nan || qv[vc][e] != qv[vc][e];
                }
                exact = exact || __builtin_amdgcn_ballot_w64(nan) != 0;
                clip = true;
            }
            if (exact) {
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        if (!fast || !(__builtin_fabsf(qq[0][m][k]) <= 448.0f)) qq[0][m][k] = xq[m][k] / ds[0];
                        if (!fast || !(__builtin_fabsf(qq[1][m][k]) <= 448.0f)) qq[1][m][k] = xk[m][k] / ds[1];
                    }
                if constexpr (VF8) {
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (!fast || !(__builtin_fabsf(qv[vc][e]) <= 448.0f)) qv[vc][e] = xv[vc][e] / ds[2];
                }
            }
            if (p.sat && (clip || exact)) {  // count quotients past the range over the active lanes
                uint32_t n0 = 0, n1 = 0, n2 = 0;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        n0 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(qq[0][m][k]) > 448.0f));
                        n1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(qq[1][m][k]) > 448.0f));
                    }
                if constexpr (VF8) {
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            n2 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_fabsf(qv[vc][e]) > 448.0f));
                }
                if (lane == (int)__builtin_ctzll(__builtin_amdgcn_read_exec())) {
                    // partial counts spread over slots (one 128-byte line each) to keep atomics apart
                    unsigned long long *slot = p.sat + 16 * (1 + (blockIdx.x & (H3_SAT_SLOTS - 1)));
                    if (n0) atomicAdd(slot, (unsigned long long)n0);
                    if (n1) atomicAdd(slot + 1, (unsigned long long)n1);
                    if (n2) atomicAdd(slot + 2, (unsigned long long)n2);
                }
            }
            if (clip && !exact) {  // no NaN here: saturate to +-448 ahead of the conversion instruction
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        qq[0][m][k] = __builtin_amdgcn_fmed3f(qq[0][m][k], -448.0f, 448.0f);
                        qq[1][m][k] = __builtin_amdgcn_fmed3f(qq[1][m][k], -448.0f, 448.0f);
                    }
                if constexpr (VF8) {
#pragma unroll
                    for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                        for (int e = 0; e < 8; ++e) qv[vc][e] = __builtin_amdgcn_fmed3f(qv[vc][e], -448.0f, 448.0f);
                }
            }
            uint32_t cw[2][M][W / 4];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                pack_e4m3<W>(qq[0][m], !exact, cw[0][m]);
                pack_e4m3<W>(qq[1][m], !exact, cw[1][m]);
            }
            if constexpr (W == 8 && M == 2) {
                store_words_pairs<1, W>(p.q, o + olane, c, cw[0][0], cw[0][1]);
                store_words_pairs<1, W>(p.k, o + olane, c, cw[1][0], cw[1][1]);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    store_code_words<W>(p.q, o + (olane + 8 * W * m + W * c), cw[0][m]);
                    store_code_words<W>(p.k, o + (olane + 8 * W * m + W * c), cw[1][m]);
                }
            }
            if constexpr (VF8) {
                uint32_t cv[VC][2];
#pragma unroll
                for (int vc = 0; vc < VC; ++vc) pack_e4m3<8>(qv[vc], !exact, cv[vc]);
                if constexpr (VC == 2) {  // each token's 128-byte row in one instruction
                    store_words_pairs<1, 8>(p.v, o + olane, c, cv[0], cv[1]);
                } else {  // 8 tokens' 64-byte rows: 512 contiguous bytes
                    st_nt(reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(p.v) + o + (olane + 8 * c)),
                          (u32x2){cv[0][0], cv[0][1]});
                }
            }
        } else {
            if constexpr (kPairStore<QT, W, M>) {
                store_row_pairs<QT, W>(p.q, o + olane, c, xq);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_chunk<QT, W>(p.q, o + (olane + 8 * W * m + W * c), xq[m]);
            }
            if constexpr (kPairStore<KT, W, M>) {
                store_row_pairs<KT, W>(p.k, o + olane, c, xk);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_chunk<KT, W>(p.k, o + (olane + 8 * W * m + W * c), xk[m]);
            }
        }
        if constexpr (!VF8) {
#pragma unroll
            for (int vc = 0; vc < VC; ++vc)
                st_nt(reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(p.v) + o + (olane + 64 * vc + 8 * c)), rv[u][vc]);
        }
    }
}

// ------------------------------------------------------------------ amax kernel

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

template <int D, int W, int M, int HPW>
struct AmaxItem {
    uint32_t rq[HPW][M][W / 2], rk[HPW][M][W / 2];
    int b, i, h0, nh;
    bool live;  // a valid token of an existing item
};

template <int D, int W, int M, int HPW>
__device__ __forceinline__ void amax_fetch(const QkParams &p, int64_t item, int g, int c,
                                           AmaxItem<D, W, M, HPW> &it) {
    it.live = false;
    if (item >= p.items) return;
    const uint32_t it32 = (uint32_t)item;  // items < 2^31 (checked on the host)
    const uint32_t bgi = it32 / (uint32_t)p.head_chunks;
    const int hc = (int)(it32 - bgi * (uint32_t)p.head_chunks);
    const uint32_t b32 = bgi / (uint32_t)p.groups;
    it.b = (int)b32;
    it.i = (int)(bgi - b32 * (uint32_t)p.groups) * 8 + g;
    it.h0 = hc * HPW;
    it.nh = min(HPW, p.H - it.h0);
    if (it.i >= p.T || it.i >= p.vlen[it.b]) return;
    it.live = true;
    const uint16_t *tok = p.qkv + (int64_t)it.b * p.batch_stride + (int64_t)it.i * p.row_stride;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const int h = it.h0 + u;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (u < it.nh) {
                load_chunk<W>(tok + (int64_t)h * D + 8 * W * m + W * c, it.rq[u][m]);
                load_chunk<W>(tok + (int64_t)(p.H + h) * D + 8 * W * m + W * c, it.rk[u][m]);
            } else {  // absent head of an odd head count: zeros, never reduced
#pragma unroll
                for (int k = 0; k < W / 2; ++k) it.rq[u][m][k] = it.rk[u][m][k] = 0u;
            }
        }
    }
}

template <int D, int IN, int NN>
__global__ __launch_bounds__(256) void qk_amax_kernel(const QkParams p) {
    // nothing is stored, so 4-wide chunks: fewer cross-lane tree levels per element than W = 8
    constexpr int W = 4;
    constexpr int M = D / (8 * W);
    constexpr int HPW = kHeadsPerWave;
    const int lane = threadIdx.x & 63;
    const int c = chunk_of_lane(lane & 7);  // chunk of the row this lane holds
    const int g = lane >> 3;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
    const float inv_d = 1.0f / (float)D;

    float wq[M][W], wk[M][W];
    load_weights<W, M>(p.wq, c, wq);
    load_weights<W, M>(p.wk, c, wk);
    uint32_t mx0 = 0u, mx1 = 0u;  // max of |y'| bits: NaN above +inf above every finite value

    AmaxItem<D, W, M, HPW> cur, nxt;
    amax_fetch(p, wave0, g, c, cur);
    for (int64_t item = wave0; item < p.items; item += nwaves) {
        amax_fetch(p, item + nwaves, g, c, nxt);  // next item's loads in flight
        if (cur.live) {
            float cs[M][W / 2], sn[M][W / 2];
            bool rot[M][W / 2];
            rotary_entries<W, M, NN>(p, cur.b, cur.i, c, cs, sn, rot);
#pragma unroll
            for (int u = 0; u < HPW; ++u) {
                if (u >= cur.nh) break;
                float xq[M][W], xk[M][W];
                unpack_row<W, M, IN>(cur.rq[u], xq);
                unpack_row<W, M, IN>(cur.rk[u], xk);
                const float rq_ = row_rstd(row_sumsq<W, M>(xq), inv_d, p.eps);
                const float rk_ = row_rstd(row_sumsq<W, M>(xk), inv_d, p.eps);
                row_scale_rotate<W, M>(xq, rq_, wq, cs, sn, rot);
                row_scale_rotate<W, M>(xk, rk_, wk, cs, sn, rot);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        mx0 = max(mx0, __float_as_uint(xq[m][k]) & 0x7FFFFFFFu);
                        mx1 = max(mx1, __float_as_uint(xk[m][k]) & 0x7FFFFFFFu);
                    }
            }
        }
        cur = nxt;
    }
    __shared__ uint32_t red[2][4];
    mx0 = wave_max_u32(mx0);
    mx1 = wave_max_u32(mx1);
    if (lane == 0) {
        red[0][wv] = mx0;
        red[1][wv] = mx1;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const int nw = blockDim.x >> 6;
        uint32_t m = 0u;
        for (int w = 0; w < nw; ++w) m = max(m, red[threadIdx.x][w]);
        if (m) atomicMax(reinterpret_cast<unsigned int *>(p.amax) + threadIdx.x, m);
    }
}

// Zero n words (the amax pair before its reduction, the clip counters before the cast).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *a, int n) {
    for (int i = (int)threadIdx.x; i < n; i += 256) a[i] = 0u;
}

int clear_words(uint32_t *a, int n, hipStream_t stream, const char *what, std::string *err) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, a, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string(what) + " clear launch failed: " + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

// Totals of the clip-counter slots: sat[t] = sum over slots of sat[16 (1 + slot) + t], one wave.
__global__ __launch_bounds__(64) void sat_total_kernel(unsigned long long *sat) {
    const int l = threadIdx.x;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        unsigned long long v = 0;
        for (int s = l; s < H3_SAT_SLOTS; s += 64) v += sat[16 * (1 + s) + t];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (l == 0) sat[t] = v;
    }
}

// ------------------------------------------------------------------ dispatch

// Device facts read once per process (all devices of one process are gfx950 parts).
struct DeviceFacts {
    int cus = 0;
    int lds_per_cu = 0;
};

bool device_facts(DeviceFacts *f, std::string *err) {
    static DeviceFacts facts;
    if (facts.cus == 0) {
        int dev = 0;
        DeviceFacts t;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&t.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&t.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            t.cus <= 0 || t.lds_per_cu <= 0) {
            *err = "device query failed (no HIP device?)";
            return false;
        }
        facts = t;
    }
    *f = facts;
    return true;
}

int launch_kernel(const void *kern, int64_t blocks, size_t lds, QkParams &p, hipStream_t stream, std::string *err) {
    if (blocks <= 0) return H3_OK;
    if (blocks > 0x7FFFFFFF) {
        *err = "problem too large for one launch";
        return H3_EUNSUPPORTED;
    }
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3(256), args, lds, stream);
    if (e != hipSuccess) {
        *err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

// Resident blocks per CU of the store / cast kernels.  They stream with no reuse, and on MI355X
// fewer concurrent blocks keep a narrower window of every output plane open in HBM: 3 blocks
// (12 waves) per CU measured best for the full-latent workload (4-5 within 1 %, 6-7 about 7 %
// slower).  The cap is imposed by reserving a third of the CU's LDS per block (the kernels use none).
constexpr int kStoreBlocksPerCU = 3;

template <int D, int IN, int QT, int KT, int MODE, int NN, bool VF8>
int launch_one(QkParams &p, hipStream_t stream, std::string *err) {
    DeviceFacts f;
    if (!device_facts(&f, err)) return H3_ELAUNCH;
    if constexpr (MODE == MODE_AMAX) {
        auto kern = qk_amax_kernel<D, IN, NN>;
        static int max_blocks = 0;  // resident blocks per CU of this kernel
        if (max_blocks == 0 &&
            (hipOccupancyMaxActiveBlocksPerMultiprocessor(&max_blocks, kern, 256, 0) != hipSuccess || max_blocks <= 0)) {
            max_blocks = 0;
            *err = "occupancy query failed";
            return H3_ELAUNCH;
        }
        const int rc = clear_words(reinterpret_cast<uint32_t *>(p.amax), 2, stream, "amax", err);
        if (rc != H3_OK) return rc;
        // persistent waves, two rounds of resident blocks: one atomic per block and tensor
        int64_t blocks = (p.items + 3) / 4;
        const int64_t cap = 2 * (int64_t)max_blocks * f.cus;
        if (blocks > cap) blocks = cap;
        return launch_kernel(reinterpret_cast<const void *>(kern), blocks, 0, p, stream, err);
    } else {
        auto kern = qk_kernel<D, IN, QT, KT, MODE, NN, VF8>;
        if (MODE == MODE_CAST && p.sat) {
            const int rc = clear_words(reinterpret_cast<uint32_t *>(p.sat), 2 * H3_SAT_WORDS, stream, "clip counter", err);
            if (rc != H3_OK) return rc;
        }
        const size_t lds = (size_t)(f.lds_per_cu / kStoreBlocksPerCU);
        const int rc = launch_kernel(reinterpret_cast<const void *>(kern), (p.items + 3) / 4, lds, p, stream, err);
        if (rc != H3_OK || MODE != MODE_CAST || !p.sat) return rc;
        hipLaunchKernelGGL(sat_total_kernel, dim3(1), dim3(64), 0, stream, p.sat);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            *err = std::string("clip counter total launch failed: ") + hipGetErrorString(e);
            return H3_ELAUNCH;
        }
        return H3_OK;
    }
}

template <int D, int IN, int MODE>
int dispatch_out(int q_dt, int k_dt, QkParams &p, hipStream_t s, std::string *err) {
    if constexpr (MODE == MODE_STORE) {
#define H3_QK(QT, KT)                                                                        \
    if (q_dt == QT && k_dt == KT)                                                            \
        return p.n == D / 8 ? launch_one<D, IN, QT, KT, MODE, D / 8, false>(p, s, err)        \
                            : launch_one<D, IN, QT, KT, MODE, 0, false>(p, s, err);
        H3_QK(DT_F32, DT_F16) H3_QK(DT_F32, DT_BF16) H3_QK(DT_F32, DT_F32)
        H3_QK(DT_F16, DT_F16) H3_QK(DT_F16, DT_BF16) H3_QK(DT_F16, DT_F32)
        H3_QK(DT_BF16, DT_F16) H3_QK(DT_BF16, DT_BF16) H3_QK(DT_BF16, DT_F32)
#undef H3_QK
    } else if constexpr (MODE == MODE_AMAX) {
        return p.n == D / 8 ? launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, D / 8, false>(p, s, err)
                            : launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, 0, false>(p, s, err);
    } else {
        if (p.v_fp8)
            return p.n == D / 8 ? launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, D / 8, true>(p, s, err)
                                : launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, 0, true>(p, s, err);
        return p.n == D / 8 ? launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, D / 8, false>(p, s, err)
                            : launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, 0, false>(p, s, err);
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
