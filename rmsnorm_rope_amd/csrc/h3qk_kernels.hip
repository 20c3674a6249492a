// gfx950 kernels for the MiniMax-H3 QK preparation: per-head RMSNorm + partial 3-axis RoPE +
// head-major permute ([SDCPP-19] fused QKV / ggml_rope_pe_permute_rms commits, [OMNI-6607]
// Operations table), and the FP8 amax and E4M3 cast passes ([TRT-21485] Summary and
// fused_fp8_qk commits).  The numerical contract is stated in include/h3qk.h.
//
// Work decomposition (wave64):
//   * A work item is 8 consecutive tokens of one item and 2 of its heads.  Lane 8 g + l serves
//     token g of the 8 and holds, of every head row it touches, the dims
//     {8W m + W c + k : m < M, k < W} of its chunk c = chunk_of_lane(l), with W = 4, M = 2 for
//     D = 64 and W = 8, M = 2 for D = 128.  Loads are 8 W contiguous bytes per token per
//     instruction, the f32 Q store of a D = 64 row is two full 128-byte lines, V moves in 16-byte
//     lanes.  Every address is a wave-uniform base plus a 32-bit lane offset.
//   * The halving reduction tree maps onto that layout as: levels o >= 8W fold chunks inside
//     the lane, levels 4W, 2W, W are DPP butterflies across the token's 8 lanes (half-mirror,
//     then xor 2, then xor 1), levels below W fold inside the chunk.  Floating-point addition is
//     commutative, so the butterfly partner computes the same bits as the tree node, and all
//     8 lanes end with ss.
//   * Store and cast passes: one work item per wave, short-lived blocks of 1 to 4 waves (8 tokens x
//     2 to 8 heads; the geometry is chosen per pass, see store_threads).
//     Blocks are dispatched in order, so the chip writes a narrow sliding window of
//     each head plane of the [B, H, T, D] outputs; on MI355X that keeps HBM write efficiency
//     well above a persistent grid-stride sweep, which holds a window of every plane open.
//     Each wave issues its data loads first, stores V (which needs nothing from Q and K) as soon
//     as it arrives, then decodes positions and fetches weights and rotary entries.  Outputs are
//     written once and never read back, so they bypass the caches (nontemporal stores), each row
//     as whole 128-byte lines.  Resident waves per CU are capped per pass (store_waves_per_cu;
//     small D = 64 store launches: kSmallGridWavesPerCU).
//   * Amax pass: persistent waves over the work items with the next item's loads in flight
//     while the current one is reduced, one atomic max per block and tensor.  It stores nothing,
//     so it always takes W = 4 (M = D / 32), which keeps the cross-lane tree levels at 12 DPP adds
//     per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "h3qk_device.h"
#include "h3qk_internal.h"

namespace h3 {
namespace {

// ------------------------------------------------------------------ store / cast kernel

// VM: what V becomes.  0: a bit copy; 1 (cast pass): E4M3 codes with the third descale;
// 2 (store pass, sage emission): RN16(v * kv_scale), with K also multiplied by kv_scale.
template <int D, int IN, int QT, int KT, int MODE, int NN, int VM>
__global__ __launch_bounds__(256) void qk_kernel(const QkParams p) {
    constexpr bool VF8 = VM == 1;
    constexpr int W = (D == 64) ? 4 : 8;
    constexpr int M = D / (8 * W);
    constexpr int VC = D / 64;  // 16-byte V chunks per lane
    constexpr int HPW = kHeadsPerWave;
    static_assert(M >= 1 && 8 * W * M == D, "layout");
    static_assert(MODE == MODE_STORE || MODE == MODE_CAST, "store / cast kernel");
    static_assert(!VF8 || MODE == MODE_CAST, "V codes only in the cast pass");
    static_assert(VM != 2 || (MODE == MODE_STORE && KT == DT_F32), "sage: f32 K from the store pass");
    constexpr int NS = VF8 ? 3 : 2;  // scaled tensors: Q, K (and V)

    const int lane = threadIdx.x & 63;
    const int c = chunk_of_lane(lane & 7);  // chunk of the row this lane holds
    const int g = lane >> 3;
    const int64_t item0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // The cast walks the items from last to first, starting where the amax pass before it ends.
    // Measured on the FP8 long sequence: amax + cast 831 -> 820 us, the cast alone 602 -> 596 us;
    // the cast costs the same inside the pair as alone, so the gain is the order itself, not lines
    // left in the last-level cache.  The store pass runs either way alike.
    const int64_t item = MODE == MODE_CAST ? p.items - 1 - item0 : item0;

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
    if (item < 0 || item >= p.items) return;

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
            if constexpr (kF32PairStore<QT, W, M>) {
                store_f32_zero_row_pairs(p.q, o + olane, c);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_zero_chunk<QT, W>(p.q, o + (olane + 8 * W * m + W * c));
            }
            if constexpr (kF32PairStore<KT, W, M>) {
                store_f32_zero_row_pairs(p.k, o + olane, c);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_zero_chunk<KT, W>(p.k, o + (olane + 8 * W * m + W * c));
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
    // every slot loads (an absent head of an odd head count re-reads the last head; its rows are
    // never stored): no branch between the loads
    // (the head's start joins the uniform base; the chunk's place in the row is a constant offset)
    const uint32_t lo = tlane + W * c, lv = tlane + 8 * c;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const int64_t h = min(h0 + u, p.H - 1);
        const uint16_t *bq = tokb + h * D, *bk = tokb + (p.H + h) * D, *bv = tokb + (2 * p.H + h) * D;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            load_chunk<W>(at16(bq, lo) + 8 * W * m, rq[u][m]);
            load_chunk<W>(at16(bk, lo) + 8 * W * m, rk[u][m]);
        }
#pragma unroll
        for (int vc = 0; vc < VC; ++vc) rv[u][vc] = *reinterpret_cast<const u32x4 *>(at16(bv, lv) + 64 * vc);
    }
    // V needs nothing from Q and K: a bit copy (or, for the sage emission, RN16(v * kv_scale)) is
    // stored as soon as it arrives, which frees its registers before the row arithmetic (measured:
    // cast 627 -> 609 us on the FP8 long sequence, store 631 -> 623 us on the full latent)
    uint32_t nsat[3] = {0u, 0u, 0u};  // cast: quotients past the E4M3 range per tensor, this wave
    if constexpr (VM == 1) {  // V codes with the third descale
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= nh) break;
            const int64_t o = obase + u * plane;
            float xv[VC][8];
#pragma unroll
            for (int vc = 0; vc < VC; ++vc)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t wd = rv[u][vc][e >> 1];
                    xv[vc][e] = in_to_f32<IN>((e & 1) ? (wd >> 16) : (wd & 0xFFFFu));
                }
            uint32_t cv[VC][2];
            cast_e4m3_wave<VC, 8>(xv, ds[2], rcp[2], fast, p.sat_slots != nullptr, nsat[2], cv);
            if constexpr (VC == 2) {  // each token's 128-byte row in one instruction
                store_words_pairs<1, 8>(p.v, o + olane, c, cv[0], cv[1]);
            } else {  // 8 tokens' 64-byte rows: 512 contiguous bytes
                st_nt(reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(p.v) + o + (olane + 8 * c)),
                      (u32x2){cv[0][0], cv[0][1]});
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= nh) break;
            const int64_t o = obase + u * plane;
#pragma unroll
            for (int vc = 0; vc < VC; ++vc) {
                u32x4 w = rv[u][vc];
                if constexpr (VM == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = keep_f32(in_to_f32<IN>(w[e] & 0xFFFFu) * p.kv_scale);
                        const float hi = keep_f32(in_to_f32<IN>(w[e] >> 16) * p.kv_scale);
                        w[e] = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
                    }
                }
                st_nt(reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(p.v) + o + (olane + 64 * vc + 8 * c)), w);
            }
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
    // independent chains hide latency better at its few waves per SIMD (measured: shared is 7 %
    // slower on the full latent, 35 % on one tile).
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
            uint32_t cw[2][M][W / 4];
            cast_e4m3_wave<M, W>(xq, ds[0], rcp[0], fast, p.sat_slots != nullptr, nsat[0], cw[0]);
            cast_e4m3_wave<M, W>(xk, ds[1], rcp[1], fast, p.sat_slots != nullptr, nsat[1], cw[1]);
            if constexpr (W == 8 && M == 2) {
                store_words_pairs<1, W>(p.q, o + olane, c, cw[0][0], cw[0][1]);
                store_words_pairs<1, W>(p.k, o + olane, c, cw[1][0], cw[1][1]);
            } else if constexpr (W == 4 && M == 2) {
                store_word_pairs(p.q, o + olane, c, cw[0][0][0], cw[0][1][0]);
                store_word_pairs(p.k, o + olane, c, cw[1][0][0], cw[1][1][0]);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    store_code_words<W>(p.q, o + (olane + 8 * W * m + W * c), cw[0][m]);
                    store_code_words<W>(p.k, o + (olane + 8 * W * m + W * c), cw[1][m]);
                }
            }
        } else {
            if constexpr (VM == 2) {  // sage: K * kv_scale, rounded once in binary32
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; ++k) xk[m][k] = xk[m][k] * p.kv_scale;
            }
            if constexpr (kPairStore<QT, W, M>) {
                store_row_pairs<QT, W>(p.q, o + olane, c, xq);
            } else if constexpr (kF32PairStore<QT, W, M>) {
                store_f32_row_pairs<W>(p.q, o + olane, c, xq);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_chunk<QT, W>(p.q, o + (olane + 8 * W * m + W * c), xq[m]);
            }
            if constexpr (kPairStore<KT, W, M>) {
                store_row_pairs<KT, W>(p.k, o + olane, c, xk);
            } else if constexpr (kF32PairStore<KT, W, M>) {
                store_f32_row_pairs<W>(p.k, o + olane, c, xk);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_chunk<KT, W>(p.k, o + (olane + 8 * W * m + W * c), xk[m]);
            }
        }
    }
    if constexpr (MODE == MODE_CAST) {
        // partial counts spread over slots (one 128-byte line each) to keep the atomics apart
        if (p.sat_slots && (nsat[0] | nsat[1] | nsat[2]) && lane == (int)__builtin_ctzll(__builtin_amdgcn_read_exec())) {
            unsigned long long *slot = p.sat_slots + 16 * (blockIdx.x & (H3_SAT_SLOTS - 1));
            if (nsat[0]) atomicAdd(slot, (unsigned long long)nsat[0]);
            if (nsat[1]) atomicAdd(slot + 1, (unsigned long long)nsat[1]);
            if (nsat[2]) atomicAdd(slot + 2, (unsigned long long)nsat[2]);
        }
    }
}

// ------------------------------------------------------------------ amax kernel

template <int D, int W, int M, int HPW, bool VA>
struct AmaxItem {
    uint32_t rq[HPW][M][W / 2], rk[HPW][M][W / 2];
    uint32_t rv[VA ? HPW : 1][M][W / 2];  // V bits (VA: V's amax too)
    int b, i, h0, nh;
    bool live;  // a valid token of an existing item
};

template <int D, int W, int M, int HPW, bool VA>
__device__ __forceinline__ void amax_fetch(const QkParams &p, int64_t item, int g, int c,
                                           AmaxItem<D, W, M, HPW, VA> &it) {
    it.live = false;
    if (item >= p.items) return;
    const uint32_t it32 = (uint32_t)item;  // items < 2^31 (checked on the host)
    const uint32_t bgi = it32 / (uint32_t)p.head_chunks;
    const int hc = (int)(it32 - bgi * (uint32_t)p.head_chunks);
    const uint32_t b32 = bgi / (uint32_t)p.groups;
    // item is the same in every lane: so are b and the token group (made explicit for the compiler)
    const int b = __builtin_amdgcn_readfirstlane((int)b32);
    const int tg = __builtin_amdgcn_readfirstlane((int)(bgi - b32 * (uint32_t)p.groups));
    it.b = b;
    it.i = tg * 8 + g;
    it.h0 = hc * HPW;
    it.nh = min(HPW, p.H - it.h0);
    if (it.i >= p.T || it.i >= p.vlen[it.b]) return;
    it.live = true;
    // the wave's first token as a uniform base, the lane's token as a 32-bit offset
    const uint16_t *tokb = p.qkv + (int64_t)b * p.batch_stride + (int64_t)tg * 8 * p.row_stride;
    const uint32_t tlane = (uint32_t)g * (uint32_t)p.row_stride;  // < 2^26 * 8 (checked on the host)
    // every slot loads (an absent head of an odd head count re-reads the last head, and its row is
    // never reduced): no branch between the loads, so none of them waits for another.  The 8 rows
    // are one raw buffer (8 row strides < 2^30 bytes): every load takes the lane's byte offset in
    // one VGPR, the same for every item, the head's place as a scalar offset and the chunk's as an
    // immediate, so no item's addresses take registers.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)tokb, (short)0, (int)(16u * (uint32_t)p.row_stride), kRawBufferFlags);
    const uint32_t lo = (tlane + W * c) * 2u;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const int h = min(it.h0 + u, p.H - 1);
        const int sq = h * D * 2, sk = (p.H + h) * D * 2, sv = (2 * p.H + h) * D * 2;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            load_chunk_buf<W>(rs, lo + 16u * W * m, sq, it.rq[u][m]);
            load_chunk_buf<W>(rs, lo + 16u * W * m, sk, it.rk[u][m]);
            if constexpr (VA) load_chunk_buf<W>(rs, lo + 16u * W * m, sv, it.rv[u][m]);
        }
    }
}

template <int D, int IN, int NN, bool VA>
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
    MagMax mx0, mx1;  // largest |y'| of Q and of K
    uint32_t mv = 0u;  // VA: max of |v| 16-bit bits (NaN above +inf above every finite value)

    using Item = AmaxItem<D, W, M, HPW, VA>;
    struct Rot { float cs[M][W / 2], sn[M][W / 2]; bool rot[M][W / 2]; };
    auto rotary = [&](const Item &it, Rot &r) {
        if (it.live) rotary_entries<W, M, NN>(p, it.b, it.i, c, r.cs, r.sn, r.rot);
    };
    auto reduce = [&](const Item &it, const Rot &r) {
        if (!it.live) return;
        const auto &cs = r.cs;
        const auto &sn = r.sn;
        const auto &rot = r.rot;
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= it.nh) break;
            float xq[M][W], xk[M][W];
            unpack_row<W, M, IN>(it.rq[u], xq);
            unpack_row<W, M, IN>(it.rk[u], xk);
            const float rq_ = row_rstd(row_sumsq<W, M>(xq), inv_d, p.eps);
            const float rk_ = row_rstd(row_sumsq<W, M>(xk), inv_d, p.eps);
            row_scale_rotate<W, M>(xq, rq_, wq, cs, sn, rot);
            row_scale_rotate<W, M>(xk, rk_, wk, cs, sn, rot);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int k = 0; k < W; k += 2) {
                    mx0.add2(xq[m][k], xq[m][k + 1]);
                    mx1.add2(xk[m][k], xk[m][k + 1]);
                }
            if constexpr (VA) {
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W / 2; ++k)
                        mv = max(mv, max(it.rv[u][m][k] & 0x7FFFu, (it.rv[u][m][k] >> 16) & 0x7FFFu));
            }
        }
    };
    // Two item buffers that take turns (the loop is unrolled by two rather than copying the
    // prefetched item into the current one): each item is reduced while the next one's loads are in
    // flight.
    // The rotary entries of the item about to be reduced are fetched before the next item's loads
    // are issued: loads complete in issue order, so entries fetched after them would make the
    // reduction wait for the whole next item.
    Item a, b;
    Rot r;
    amax_fetch(p, wave0, g, c, a);
    for (int64_t item = wave0; item < p.items; item += 2 * nwaves) {
        rotary(a, r);
        amax_fetch(p, item + nwaves, g, c, b);
        reduce(a, r);
        if (item + nwaves >= p.items) break;
        rotary(b, r);
        amax_fetch(p, item + 2 * nwaves, g, c, a);
        reduce(b, r);
    }
    constexpr int NT = VA ? 3 : 2;
    __shared__ uint32_t red[3][4];
    const uint32_t m0 = wave_max_u32(mx0.bits());
    const uint32_t m1 = wave_max_u32(mx1.bits());
    if (lane == 0) {
        red[0][wv] = m0;
        red[1][wv] = m1;
    }
    if constexpr (VA) {
        // a 16-bit magnitude maps monotonically (NaN above +inf) to the binary32 bits of its value
        mv = wave_max_u32(mv);
        if (lane == 0) red[2][wv] = __float_as_uint(in_to_f32<IN>(mv));
    }
    __syncthreads();
    if (threadIdx.x < NT) {
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

}  // namespace

int clear_words(uint32_t *a, int n, hipStream_t stream, const char *what, std::string *err) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, a, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string(what) + " clear launch failed: " + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

namespace {

// Totals of the clip-counter slots: sat[t] = sum over slots of slots[16 slot + t], one wave.
__global__ __launch_bounds__(64) void sat_total_kernel(const unsigned long long *slots, unsigned long long *sat) {
    const int l = threadIdx.x;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        unsigned long long v = 0;
        for (int s = l; s < H3_SAT_SLOTS; s += 64) v += slots[16 * s + t];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (l == 0) sat[t] = v;
    }
}

}  // namespace

// Partial clip counts of the allocation-free static cast: H3_SAT_SLOTS slots of 16 words, 16 KiB.
// One copy per GPU, held until the process ends; host code reaches it only through the device
// address hipGetSymbolAddress returns (scratch_slots), never through its name.
static __device__ __align__(256) unsigned long long scratch[H3_SAT_SLOTS * 16];

int clear_sat_slots(unsigned long long *slots, hipStream_t stream, std::string *err) {
    return clear_words(reinterpret_cast<uint32_t *>(slots), 2 * 16 * H3_SAT_SLOTS, stream, "clip counter", err);
}

int sat_total(const unsigned long long *slots, unsigned long long *sat, hipStream_t stream, std::string *err) {
    hipLaunchKernelGGL(sat_total_kernel, dim3(1), dim3(64), 0, stream, slots, sat);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("clip counter total launch failed: ") + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

bool scratch_slots(unsigned long long **slots, std::string *err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static unsigned long long *addr[kMaxDevices];  // per device; null: not looked up yet
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = "no current HIP device (or a device index past 63)";
        return false;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = std::string("scratch address lookup failed: ") + hipGetErrorString(e);
            return false;
        }
        addr[dev] = static_cast<unsigned long long *>(p);
    }
    *slots = addr[dev];
    return true;
}

// ------------------------------------------------------------------ dispatch

bool device_facts(DeviceFacts *f, std::string *err) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        *err = "no current HIP device";
        return false;
    }
    static std::mutex mu;
    static std::vector<DeviceFacts> cache;  // by device id; cus == 0: not queried yet
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= cache.size()) cache.resize((size_t)dev + 1);
    DeviceFacts &c = cache[(size_t)dev];
    if (c.cus == 0) {
        DeviceFacts t;
        t.device = dev;
        if (hipDeviceGetAttribute(&t.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&t.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            t.cus <= 0 || t.lds_per_cu <= 0) {
            *err = "device query failed";
            return false;
        }
        c = t;
    }
    *f = c;
    return true;
}

bool resident_blocks(const void *kern, const DeviceFacts &f, int *blocks, std::string *err) {
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(kern, f.device);
    auto it = cache.find(key);
    if (it == cache.end()) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n <= 0) {
            *err = "occupancy query failed";
            return false;
        }
        it = cache.emplace(key, n).first;
    }
    *blocks = it->second;
    return true;
}

int launch_kernel(const void *kern, int64_t blocks, size_t lds, QkParams &p, hipStream_t stream, std::string *err,
                  int threads) {
    if (blocks <= 0) return H3_OK;
    // the dispatch's grid is a 32-bit count of work-items
    if ((uint64_t)blocks * (uint64_t)threads > 0xFFFFFFFFull) {
        *err = "problem too large for one launch";
        return H3_EUNSUPPORTED;
    }
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3((unsigned)threads), args, lds, stream);
    if (e != hipSuccess) {
        *err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return H3_ELAUNCH;
    }
    return H3_OK;
}

namespace {

// Launch geometry of the store / cast kernels (store_threads, store_waves_per_cu).  They stream
// with no reuse, and on MI355X fewer and smaller concurrent blocks keep a narrower window of every
// output plane open in HBM; the casts, which do more arithmetic per byte, want more waves in flight
// where their registers allow.  The cap is imposed by reserving the matching share of the CU's LDS
// per block (the kernels use none).

template <int D, int IN, int QT, int KT, int MODE, int NN, int VM>
int launch_one(QkParams &p, hipStream_t stream, std::string *err) {
    constexpr bool VF8 = VM == 1;
    DeviceFacts f;
    if (!device_facts(&f, err)) return H3_ELAUNCH;
    if constexpr (MODE == MODE_AMAX) {
        auto kern = qk_amax_kernel<D, IN, NN, VF8>;
        int max_blocks = 0;  // resident blocks per CU of this kernel
        if (!resident_blocks(reinterpret_cast<const void *>(kern), f, &max_blocks, err)) return H3_ELAUNCH;
        const int rc = clear_words(reinterpret_cast<uint32_t *>(p.amax), VF8 ? 3 : 2, stream, "amax", err);
        if (rc != H3_OK) return rc;
        // persistent waves, two rounds of resident blocks: one atomic per block and tensor
        int64_t blocks = (p.items + 3) / 4;
        const int64_t cap = 2 * (int64_t)max_blocks * f.cus;
        if (blocks > cap) blocks = cap;
        return launch_kernel(reinterpret_cast<const void *>(kern), blocks, 0, p, stream, err);
    } else {
        auto kern = qk_kernel<D, IN, QT, KT, MODE, NN, VM>;
        if (MODE == MODE_CAST && p.sat_slots) {
            const int rc = clear_sat_slots(p.sat_slots, stream, err);
            if (rc != H3_OK) return rc;
        }
        constexpr bool cast = MODE == MODE_CAST, f32out = QT == DT_F32 || KT == DT_F32;
        constexpr int threads = store_threads<D, cast, f32out>(), wpb = threads / 64;  // waves (items) per block
        constexpr int blocks_per_cu = store_waves_per_cu<D, cast>() / wpb;
        static_assert(blocks_per_cu >= 3, "at most a third of the CU's LDS per block");
        const int64_t blocks = (p.items + wpb - 1) / wpb;
        int per_cu = blocks_per_cu;
        if (D == 64 && !cast && blocks <= (int64_t)kSmallGridRounds * blocks_per_cu * f.cus)
            per_cu = kSmallGridWavesPerCU / wpb;
        const size_t lds = (size_t)(f.lds_per_cu / per_cu);
        const int rc = launch_kernel(reinterpret_cast<const void *>(kern), blocks, lds, p, stream, err, threads);
        if (rc != H3_OK || MODE != MODE_CAST || !p.sat_slots) return rc;
        return sat_total(p.sat_slots, p.sat, stream, err);
    }
}

template <int D, int IN, int MODE>
int dispatch_out(int q_dt, int k_dt, QkParams &p, hipStream_t s, std::string *err) {
    if constexpr (MODE == MODE_STORE) {
        if (p.sage)  // F32 Q, F32 K * kv_scale, F16 V * kv_scale
            return p.n == D / 8 ? launch_one<D, IN, DT_F32, DT_F32, MODE, D / 8, 2>(p, s, err)
                                : launch_one<D, IN, DT_F32, DT_F32, MODE, 0, 2>(p, s, err);
#define H3_QK(QT, KT)                                                                        \
    if (q_dt == QT && k_dt == KT)                                                            \
        return p.n == D / 8 ? launch_one<D, IN, QT, KT, MODE, D / 8, 0>(p, s, err)            \
                            : launch_one<D, IN, QT, KT, MODE, 0, 0>(p, s, err);
        H3_QK(DT_F32, DT_F16) H3_QK(DT_F32, DT_BF16) H3_QK(DT_F32, DT_F32)
        H3_QK(DT_F16, DT_F16) H3_QK(DT_F16, DT_BF16) H3_QK(DT_F16, DT_F32)
        H3_QK(DT_BF16, DT_F16) H3_QK(DT_BF16, DT_BF16) H3_QK(DT_BF16, DT_F32)
#undef H3_QK
    } else {
        if (p.v_fp8)
            return p.n == D / 8 ? launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, D / 8, 1>(p, s, err)
                                : launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, 0, 1>(p, s, err);
        return p.n == D / 8 ? launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, D / 8, 0>(p, s, err)
                            : launch_one<D, IN, DT_E4M3, DT_E4M3, MODE, 0, 0>(p, s, err);
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
