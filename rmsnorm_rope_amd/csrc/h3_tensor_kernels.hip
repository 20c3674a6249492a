// gfx950 kernels for one separately projected tensor [B, T, H, D] (the per-tensor form of the
// QK preparation: [TRT-21485] norm_rope_tensor commit, for the asynchronous Ulysses path, where Q,
// K and V come out of three projections, and the split launch mode that runs a packed QKV through
// per-tensor passes with the packed row stride).  Q and K rows are RMS-normalised with the
// tensor's weight and rotated; without a weight (V) the values pass through unchanged.  The
// output is a 16-bit or f32 tensor, or E4M3 codes with a per-tensor descale, written [B, H, T, D]
// or [B, T, H, D].  The numerical contract is stated in include/h3qk.h.
//
// The lane layout and the reduction tree are those of the fused kernels (h3qk_kernels.hip): a
// wave serves 8 consecutive tokens, lane 8 g + l holds chunk chunk_of_lane(l) of token g's rows.
// With one tensor instead of three, a wave takes 4 heads (kTensorHeads) so that it handles as
// many rows as a fused wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3qk_device.h"
#include "h3qk_internal.h"

namespace h3 {
namespace {

// ------------------------------------------------------------------ store / cast kernel

template <int D, int IN, int OT, int MODE, int NN, bool NORM>
__global__ __launch_bounds__(256) void tensor_kernel(const QkParams p) {
    constexpr int W = (D == 64) ? 4 : 8;
    constexpr int M = D / (8 * W);
    constexpr int HPW = kTensorHeads;
    static_assert(M >= 1 && 8 * W * M == D, "layout");
    static_assert(MODE == MODE_STORE || MODE == MODE_CAST, "store / cast kernel");
    static_assert((MODE == MODE_CAST) == (OT == DT_E4M3), "codes come from the cast pass only");

    const int lane = threadIdx.x & 63;
    const int c = chunk_of_lane(lane & 7);
    const int g = lane >> 3;
    const int64_t item0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the cast walks the items from last to first, where the amax pass before it ended
    const int64_t item = MODE == MODE_CAST ? p.items - 1 - item0 : item0;

    float ds = 1.0f, rcp = 1.0f;
    bool fast = true;
    if constexpr (MODE == MODE_CAST) {
        const float a = p.amax[0];
        ds = a > 0.0f ? (p.static_scale ? a : a / 448.0f) : 1.0f;
        rcp = 1.0f / ds;
        fast = ds >= 0x1p-60f && ds <= 0x1p60f;
        if (p.descale && item == 0 && lane == 0) p.descale[0] = ds;
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
    // output row (b, h, i) starts at b H T D + h out_hstride + i out_tstride
    const int64_t obase = (int64_t)b * p.H * p.T * D + (int64_t)h0 * p.out_hstride + (int64_t)tg * 8 * p.out_tstride;
    const uint32_t olane = (uint32_t)g * (uint32_t)p.out_tstride;  // 8 out_tstride < 2^31 (checked on the host)

    if (i >= p.vlen[b]) {  // padding token: zeros
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= nh) break;
            const int64_t o = obase + u * p.out_hstride;
            if constexpr (kF32PairStore<OT, W, M>) {
                store_f32_zero_row_pairs(p.q, o + olane, c);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_zero_chunk<OT, W>(p.q, o + (olane + 8 * W * m + W * c));
            }
        }
        return;
    }

    // 1. every data load of the item first
    const uint16_t *tokb = p.qkv + (int64_t)b * p.batch_stride + (int64_t)tg * 8 * p.row_stride;
    const uint32_t tlane = (uint32_t)g * (uint32_t)p.row_stride;  // < 2^26 * 8 (checked on the host)
    uint32_t r[HPW][M][W / 2];
    // every slot loads (an absent head of a head count that is not a multiple of 4 re-reads the last
    // head; its rows are never stored): no branch between the loads
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const uint32_t hd = (uint32_t)min(h0 + u, p.H - 1) * D;
#pragma unroll
        for (int m = 0; m < M; ++m) load_chunk<W>(at16(tokb, tlane + hd + 8 * W * m + W * c), r[u][m]);
    }

    // 2. normalise and rotate (Q, K) or take the values as they are (V)
    float x[HPW][M][W];
#pragma unroll
    for (int u = 0; u < HPW; ++u) unpack_row<W, M, IN>(r[u], x[u]);
    if constexpr (NORM) {
        float w[M][W];
        load_weights<W, M>(p.wq, c, w);
        float cs[M][W / 2], sn[M][W / 2];
        bool rot[M][W / 2];
        rotary_entries<W, M, NN>(p, b, i, c, cs, sn, rot);
        const float inv_d = 1.0f / (float)D;
        float ss[HPW], rr[HPW];
#pragma unroll
        for (int u = 0; u < HPW; ++u) ss[u] = row_sumsq<W, M>(x[u]);
        if constexpr (MODE == MODE_CAST) {
            rows_rstd<HPW>(ss, lane, inv_d, p.eps, rr);
        } else {
#pragma unroll
            for (int u = 0; u < HPW; ++u) rr[u] = row_rstd(ss[u], inv_d, p.eps);
        }
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            if (u >= nh) break;
            row_scale_rotate<W, M>(x[u], rr[u], w, cs, sn, rot);
        }
    }

    // 3. store, or cast and store
    uint32_t nsat = 0;  // cast: quotients past the E4M3 range in this wave
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        if (u >= nh) break;
        const int64_t o = obase + u * p.out_hstride;
        if constexpr (MODE == MODE_CAST) {
            uint32_t cw[M][W / 4];
            cast_e4m3_wave<M, W>(x[u], ds, rcp, fast, p.sat_slots != nullptr, nsat, cw);
            if constexpr (W == 8 && M == 2) {
                store_words_pairs<1, W>(p.q, o + olane, c, cw[0], cw[1]);
            } else if constexpr (W == 4 && M == 2) {
                store_word_pairs(p.q, o + olane, c, cw[0][0], cw[1][0]);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_code_words<W>(p.q, o + (olane + 8 * W * m + W * c), cw[m]);
            }
        } else {
            if constexpr (kPairStore<OT, W, M>) {
                store_row_pairs<OT, W>(p.q, o + olane, c, x[u]);
            } else if constexpr (kF32PairStore<OT, W, M>) {
                store_f32_row_pairs<W>(p.q, o + olane, c, x[u]);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) store_chunk<OT, W>(p.q, o + (olane + 8 * W * m + W * c), x[u][m]);
            }
        }
    }
    if constexpr (MODE == MODE_CAST) {
        if (nsat && lane == (int)__builtin_ctzll(__builtin_amdgcn_read_exec()))
            atomicAdd(p.sat_slots + 16 * (blockIdx.x & (H3_SAT_SLOTS - 1)), (unsigned long long)nsat);
    }
}

// ------------------------------------------------------------------ amax kernel

template <int D, int W, int M, int HPW>
struct TensorAmaxItem {
    uint32_t r[HPW][M][W / 2];
    int b, i, h0, nh;
    bool live;  // a valid token of an existing item
};

template <int D, int W, int M, int HPW>
__device__ __forceinline__ void tensor_amax_fetch(const QkParams &p, int64_t item, int g, int c,
                                                  TensorAmaxItem<D, W, M, HPW> &it) {
    it.live = false;
    if (item >= p.items) return;
    const uint32_t it32 = (uint32_t)item;
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
    const uint16_t *tokb = p.qkv + (int64_t)b * p.batch_stride + (int64_t)tg * 8 * p.row_stride;
    const uint32_t tlane = (uint32_t)g * (uint32_t)p.row_stride;  // < 2^26 * 8 (checked on the host)
    // every slot loads (an absent head re-reads the last head): no branch between the loads; the
    // head's start joins the uniform base, the chunk's place in the row is a constant offset
    const uint32_t lo = tlane + W * c;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const uint16_t *bh = tokb + (int64_t)min(it.h0 + u, p.H - 1) * D;
#pragma unroll
        for (int m = 0; m < M; ++m) load_chunk<W>(at16(bh, lo) + 8 * W * m, it.r[u][m]);
    }
}

template <int D, int IN, int NN, bool NORM>
__global__ __launch_bounds__(256) void tensor_amax_kernel(const QkParams p) {
    constexpr int W = 4;
    constexpr int M = D / (8 * W);
    constexpr int HPW = kTensorHeads;
    const int lane = threadIdx.x & 63;
    const int c = chunk_of_lane(lane & 7);
    const int g = lane >> 3;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
    const float inv_d = 1.0f / (float)D;

    float w[M][W];
    if constexpr (NORM) load_weights<W, M>(p.wq, c, w);
    uint32_t mx = 0u;  // identity: max of |x| 16-bit bits (NaN above +inf above every finite value)
    MagMax mxn;        // normalised: largest |y'|

    using Item = TensorAmaxItem<D, W, M, HPW>;
    auto reduce = [&](const Item &it) {
        if (!it.live) return;
        if constexpr (NORM) {
            float cs[M][W / 2], sn[M][W / 2];
            bool rot[M][W / 2];
            // D = 128: one load per entry (pair loads took 4 more VGPRs, a fourth wave per SIMD
            // fewer: 115 -> 126 us on the long sequence's K heads)
            rotary_entries<W, M, NN, D == 64>(p, it.b, it.i, c, cs, sn, rot);
#pragma unroll
            for (int u = 0; u < HPW; ++u) {
                if (u >= it.nh) break;
                float x[M][W];
                unpack_row<W, M, IN>(it.r[u], x);
                const float rr = row_rstd(row_sumsq<W, M>(x), inv_d, p.eps);
                row_scale_rotate<W, M>(x, rr, w, cs, sn, rot);
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W; k += 2) mxn.add2(x[m][k], x[m][k + 1]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < HPW; ++u) {
                if (u >= it.nh) break;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int k = 0; k < W / 2; ++k)
                        mx = max(mx, max(it.r[u][m][k] & 0x7FFFu, (it.r[u][m][k] >> 16) & 0x7FFFu));
            }
        }
    };
    // two item buffers taking turns (unrolled by two): each item is reduced while the next one's
    // loads are in flight
    Item a, b;
    tensor_amax_fetch(p, wave0, g, c, a);
    for (int64_t item = wave0; item < p.items; item += 2 * nwaves) {
        tensor_amax_fetch(p, item + nwaves, g, c, b);
        reduce(a);
        if (item + nwaves >= p.items) break;
        tensor_amax_fetch(p, item + 2 * nwaves, g, c, a);
        reduce(b);
    }
    if constexpr (NORM) mx = mxn.bits();
    mx = wave_max_u32(mx);
    if constexpr (!NORM) mx = __float_as_uint(in_to_f32<IN>(mx));
    __shared__ uint32_t red[4];
    if (lane == 0) red[wv] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = blockDim.x >> 6;
        uint32_t m = 0u;
        for (int k = 0; k < nw; ++k) m = max(m, red[k]);
        if (m) atomicMax(reinterpret_cast<unsigned int *>(p.amax), m);
    }
}

// ------------------------------------------------------------------ dispatch

template <int D, int IN, int OT, int MODE, int NN, bool NORM>
int launch_one(QkParams &p, hipStream_t stream, std::string *err) {
    DeviceFacts f;
    if (!device_facts(&f, err)) return H3_ELAUNCH;
    if constexpr (MODE == MODE_AMAX) {
        auto kern = tensor_amax_kernel<D, IN, NN, NORM>;
        int max_blocks = 0;  // resident blocks per CU of this kernel
        if (!resident_blocks(reinterpret_cast<const void *>(kern), f, &max_blocks, err)) return H3_ELAUNCH;
        const int rc = clear_words(reinterpret_cast<uint32_t *>(p.amax), 1, stream, "amax", err);
        if (rc != H3_OK) return rc;
        int64_t blocks = (p.items + 3) / 4;
        const int64_t cap = 2 * (int64_t)max_blocks * f.cus;
        if (blocks > cap) blocks = cap;
        return launch_kernel(reinterpret_cast<const void *>(kern), blocks, 0, p, stream, err);
    } else {
        auto kern = tensor_kernel<D, IN, OT, MODE, NN, NORM>;
        if (MODE == MODE_CAST && p.sat_slots) {
            const int rc = clear_sat_slots(p.sat_slots, stream, err);
            if (rc != H3_OK) return rc;
        }
        const size_t lds = (size_t)(f.lds_per_cu / kTensorBlocksPerCU);
        const int rc = launch_kernel(reinterpret_cast<const void *>(kern), (p.items + 3) / 4, lds, p, stream, err);
        if (rc != H3_OK || MODE != MODE_CAST || !p.sat_slots) return rc;
        return sat_total(p.sat_slots, p.sat, stream, err);
    }
}

template <int D, int IN, int OT, int MODE>
int dispatch_norm(bool norm, QkParams &p, hipStream_t s, std::string *err) {
    if (!norm) return launch_one<D, IN, OT, MODE, 0, false>(p, s, err);
    return p.n == D / 8 ? launch_one<D, IN, OT, MODE, D / 8, true>(p, s, err)
                        : launch_one<D, IN, OT, MODE, 0, true>(p, s, err);
}

template <int D, int IN>
int dispatch_out(int mode, int out_dt, bool norm, QkParams &p, hipStream_t s, std::string *err) {
    if (mode == MODE_AMAX) return dispatch_norm<D, IN, DT_E4M3, MODE_AMAX>(norm, p, s, err);
    if (mode == MODE_CAST) return dispatch_norm<D, IN, DT_E4M3, MODE_CAST>(norm, p, s, err);
    if (out_dt == DT_F32) return dispatch_norm<D, IN, DT_F32, MODE_STORE>(norm, p, s, err);
    if (out_dt == DT_F16) return dispatch_norm<D, IN, DT_F16, MODE_STORE>(norm, p, s, err);
    if (out_dt == DT_BF16) return dispatch_norm<D, IN, DT_BF16, MODE_STORE>(norm, p, s, err);
    *err = "unsupported output dtype";
    return H3_EUNSUPPORTED;
}

template <int D>
int dispatch_in(int mode, int in_dt, int out_dt, bool norm, QkParams &p, hipStream_t s, std::string *err) {
    if (in_dt == DT_F16) return dispatch_out<D, DT_F16>(mode, out_dt, norm, p, s, err);
    if (in_dt == DT_BF16) return dispatch_out<D, DT_BF16>(mode, out_dt, norm, p, s, err);
    *err = "unsupported input dtype";
    return H3_EUNSUPPORTED;
}

}  // namespace

int launch_tensor(int mode, int D, int in_dt, int out_dt, bool norm, QkParams &p, hipStream_t stream,
                  std::string *err) {
    if (D == 64) return dispatch_in<64>(mode, in_dt, out_dt, norm, p, stream, err);
    if (D == 128) return dispatch_in<128>(mode, in_dt, out_dt, norm, p, stream, err);
    *err = "unsupported head dim";
    return H3_EUNSUPPORTED;
}

}  // namespace h3
