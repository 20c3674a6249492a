// Internal launch interface between the host-side validation (h3qk_api.cpp) and the gfx950
// kernels (h3qk_kernels.hip).  Not installed; the public interface is include/h3qk.h.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define H3_HD __host__ __device__
#else
#define H3_HD
#endif

#ifndef H3QK_NO_HIP
#include <string>

#include "h3qk.h"
#endif

namespace h3 {

// Unsigned division of any 32-bit n by an invariant divisor d >= 1 with one multiply-high
// (Granlund and Montgomery, "Division by invariant integers using multiplication", PLDI 1994,
// unsigned case): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//   t = mulhi(m, n),  n / d = (t + ((n - t) >> s1)) >> s2,  s1 = min(l, 1), s2 = max(l - 1, 0).
struct DivMagic {
    uint32_t m, s1, s2, d;
};

inline DivMagic div_magic(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    DivMagic r;
    r.m = (uint32_t)m;
    r.s1 = l ? 1u : 0u;
    r.s2 = l ? l - 1u : 0u;
    r.d = d;
    return r;
}

H3_HD inline uint32_t div_apply(uint32_t n, const DivMagic &g) {
    const uint32_t t = (uint32_t)(((uint64_t)g.m * n) >> 32);
    return (t + ((n - t) >> g.s1)) >> g.s2;
}

// Blocks of a one-dimensional launch covering `units` work units, `per_block` per block, counted in
// 64 bits: the elementwise ops accept up to 2^32 - 1 units, where a 32-bit sum would wrap to zero.
H3_HD constexpr uint64_t blocks_for(uint64_t units, uint64_t per_block) {
    return (units + per_block - 1) / per_block;
}

#ifndef H3QK_NO_HIP
enum Mode : int { MODE_STORE = 0, MODE_AMAX = 1, MODE_CAST = 2 };

constexpr int kHeadsPerWave = 2;  // heads of one 8-token group served by one wave (fused Q, K, V)
constexpr int kTensorHeads = 4;   // the same for one separately projected tensor

// Launch geometry of the fused store / cast kernels: threads per block (one 8-token work item per
// wave) and the most resident waves per CU (a cap imposed through LDS).  Measured per pass:
//   * D = 64 store: 4-wave blocks (8 tokens x 8 heads), 12 waves per CU (the full latent: 616 us;
//     8 waves 630, 16-20 waves 636-651, 2-wave blocks 629-632).
//   * D = 64 cast: 4-wave blocks, 24 waves per CU (every wave its VGPRs allow): its arithmetic
//     wants more waves in flight (the full latent, V copied: 12 waves 530 us, 16 474, 20-24 460;
//     V codes: 632, 479 and 458-467).
//   * D = 128 store: 6 waves per CU, in 2-wave blocks (8 tokens x 4 heads) for 16-bit Q and K and in
//     1-wave blocks when Q or K is binary32 (the FP8 long-sequence shape: bf16 / bf16 at 12 waves
//     691-695 us, at 4-6 waves 669-676; f32 / f32 in 2-wave blocks 973-981, in 1-wave blocks 930-935;
//     f32 / bf16 840-849 and 812-817).
//   * D = 128 cast: 2-wave blocks, 12 waves per CU (8 waves 624 us, 12 580-584, 16 587; 1-wave
//     blocks 600).
template <int D, bool CAST, bool F32OUT>
constexpr int store_threads() { return D == 64 ? 256 : (!CAST && F32OUT) ? 64 : 128; }
template <int D, bool CAST>
constexpr int store_waves_per_cu() { return D == 64 ? (CAST ? 24 : 12) : (CAST ? 12 : 6); }
// A D = 64 store launch of at most kSmallGridRounds rounds of resident blocks (at 12 waves per CU)
// runs 16 waves per CU instead: with so few rounds the last, partial one weighs more than the
// narrower write window gains.  Measured (8 buffer sets rotated): one 31x16x16 tile, 2.6 rounds,
// 25.3 -> 24.1 us; 4 rounds 37.3 -> 36.2; 8 rounds 67.9 -> 66.8; 12 rounds 98.0 either way;
// 16 rounds 129.1 -> 130.5, 24 rounds 189.9 -> 193.9.
constexpr int kSmallGridRounds = 8;
constexpr int kSmallGridWavesPerCU = 16;
// Resident blocks per CU of the one-tensor kernels: 4, their waves moving fewer bytes each
// (measured on the full latent's K heads: 3 blocks 234 us, 4 blocks 175 us, 6-8 within 1 % of 4).
constexpr int kTensorBlocksPerCU = 4;

// Everything a QK kernel reads, passed by value in the kernel arguments (< 1.5 KiB).
struct QkParams {
    const uint16_t *qkv;
    void *q;
    void *k;
    void *v;
    const float *wq;
    const float *wk;
    const float *cos_tab;
    const float *sin_tab;
    float *amax;        // MODE_AMAX: reduced into (cleared first); MODE_CAST: read (amaxes, or
                        // descales when static_scale)
    float *descale;     // MODE_CAST: written by the first wave, or null
    unsigned long long *sat;  // MODE_CAST: the per-tensor counts of |quotient| > 448 (3 words), or null
    unsigned long long *sat_slots;  // MODE_CAST with sat: H3_SAT_SLOTS slots of 16 words (one 128-byte
                                    // line each) where waves add partial counts; cleared first
    int64_t row_stride;
    int64_t batch_stride;
    int64_t items;               // B * groups * head_chunks
    int32_t B, T, H, n;
    int32_t Gh, Gw;
    int32_t base_h, base_w;      // first table row of the h and w parts
    int32_t groups;              // token groups of 8 per item: ceil(T / 8)
    int32_t head_chunks;         // ceil(H / kHeadsPerWave)
    DivMagic div_gw, div_gh;     // token -> (t, h, w) decode
    float eps;
    float inv_n;                 // 1 / n (pair -> axis decode), 0 when n = 0
    int32_t tab_pairs;           // both rotary tables 8-byte aligned: even entry pairs load as one
    int32_t static_scale;        // MODE_CAST: amax[] holds the caller's descales
    int32_t v_fp8;               // MODE_CAST: V written as E4M3 codes with the third scale;
                                 // MODE_AMAX: V's amax reduced into amax[2]
    int32_t sage;                // MODE_STORE: sage emission (F32 Q, F32 K * kv_scale, F16 V * kv_scale)
    float kv_scale;
    int64_t out_hstride;         // one tensor: output elements between heads
    int64_t out_tstride;         // one tensor: output elements between tokens
    int32_t off[H3_MAX_BATCH][3];
    int32_t vlen[H3_MAX_BATCH];
};

// Facts of the calling thread's current device, queried on its first use and cached per device
// (thread-safe).
struct DeviceFacts {
    int device = -1;
    int cus = 0;
    int lds_per_cu = 0;
};
bool device_facts(DeviceFacts *f, std::string *err);

// Resident 256-thread blocks per CU of `kern` on the device of `f` (hipOccupancy query, cached per
// kernel and device, thread-safe); false with *err set when the query fails.
bool resident_blocks(const void *kern, const DeviceFacts &f, int *blocks, std::string *err);

// One launch of `kern` with 256-thread blocks and the parameters by value.
int launch_kernel(const void *kern, int64_t blocks, size_t lds, QkParams &p, hipStream_t stream, std::string *err,
                  int threads = 256);

// Zero n words on the stream (one block).
int clear_words(uint32_t *a, int n, hipStream_t stream, const char *what, std::string *err);

// Zero the H3_SAT_SLOTS partial-count slots (one block, on the stream).
int clear_sat_slots(unsigned long long *slots, hipStream_t stream, std::string *err);

// sat[0..2] = sums of the clip-counter slots (one wave, on the stream).
int sat_total(const unsigned long long *slots, unsigned long long *sat, hipStream_t stream, std::string *err);

// Device address of this GPU's copy of the library's static partial-count slots (the scratch of
// the allocation-free static cast), looked up on the first call on each device and kept.
bool scratch_slots(unsigned long long **slots, std::string *err);

// Launch one QK pass.  Returns H3_OK or H3_ELAUNCH / H3_EUNSUPPORTED with *err filled.
int launch_qk(int mode, int D, int in_dt, int q_dt, int k_dt, QkParams &p, hipStream_t stream,
              std::string *err);

// Launch one pass over a single separately projected tensor (mode as above; norm: with weight
// p.wq, else the identity).  The output pointer is p.q.
int launch_tensor(int mode, int D, int in_dt, int out_dt, bool norm, QkParams &p, hipStream_t stream,
                  std::string *err);

// Decoder-block elementwise ops (arguments already validated).
int launch_swiglu(int dt, const void *x, void *y, int64_t N, int64_t F, hipStream_t stream, std::string *err);
int launch_scaled_residual(int dt, const float *res, const void *branch, const float *scale, int64_t scale_len,
                           float *out, int64_t N, int64_t C, hipStream_t stream, std::string *err);
#endif

}  // namespace h3
