/*
 * libh3qk — MiniMax-H3 attention input preparation on AMD MI355X (gfx950).
 *
 * One memory-bound pass over the fused QKV projection of a MiniMax-H3 attention block:
 * per-head RMS normalisation of every Q and K head row with a learned per-dim weight, partial
 * 3-axis (t, h, w) rotary embedding, and a head-major store of Q, K and V; plus an FP8 variant
 * (per-tensor amax pass, then a cast pass to OCP E4M3FN codes with descales).
 *
 * Pages the operations follow:
 *   [SDCPP-19]  stable-diffusion.cpp PR #19 "MiniMax-H3: sage takes the fused RoPE op, faster
 *               video and audio VAE decode": commit messages on the fused QKV decoder path
 *               (q/k normalised on the fused projection, partial RoPE, Q in binary32 and K, V in binary16 written
 *               head-major) and on ggml_rope_pe_permute_rms (norm fused into the RoPE/permute op).
 *   [OMNI-6607] vllm-omni PR #6607 (MiniMax-H3 video VAE decoder eager ops), "Operations" table:
 *               one fused reduction + RoPE per Q/K tensor with a fixed RMS reduction tree and
 *               explicit rounding, bitwise equal to its reference; scaled residual and SwiGLU rows.
 *   [TRT-21485] TensorRT-LLM PR #21485 "cuDNN FP8 attention path for MiniMax-H3 on SM107 under
 *               Ulysses": Summary (the QK norm, the RoPE and the per-tensor FP8 cast done as an
 *               amax pass, then a cast pass), commit messages on norm_rope_tensor(x, weight, cos, sin,
 *               eps), the packed-QKV row stride, outputs that may not alias inputs, and the
 *               per-item valid length that keeps padded rows out of the amax.
 *
 * Numerical contract (identical on every call, bitwise reproducible):
 *   x_d  = the 16-bit input value, exactly, as binary32
 *   a_d  = x_d * x_d                                  (binary32, round to nearest even)
 *   fixed halving tree: for o = D/2, D/4, ..., 1 and d < o: a_d = a_d + a_{d+o}; ss = a_0
 *   r    = 1 / sqrt(ss * (1/D) + eps)                 (correctly rounded sqrt, then division)
 *   y_d  = (x_d * r) * w_d
 *   pair p < 3n (n = pairs_per_axis): axis = p / n (0 = t, 1 = h, 2 = w), j = p mod n,
 *     (c, s) = (cos_tab, sin_tab)[base_axis + pos_axis][j], base = (0, P_t, P_t + P_h);
 *     y'_{2p} = e*c - f*s,  y'_{2p+1} = e*s + f*c      (e = y_{2p}, f = y_{2p+1}; each product
 *     rounded, then the sum); dims >= 6n pass through.
 * No fused multiply-add anywhere in this chain, IEEE denormals, round to nearest even at every
 * store.  Token i of item b sits at grid position (i / (Gh*Gw), (i / Gw) mod Gh, i mod Gw) plus
 * pos_offset[b]; tokens i >= valid_len[b] are padding: all their outputs are +0 (code 0x00) and
 * they never enter the amax.
 *
 * Conventions for every entry point:
 *   - data pointers are DEVICE pointers (HIP global memory) unless marked HOST; the descriptor
 *     itself is a HOST struct read during the call only;
 *   - work is enqueued on `stream` (0 = the null stream) and is asynchronous: no host sync;
 *   - the caller owns every buffer; the library allocates no device or host memory and keeps no
 *     pointer after it returns (h3_qk_cast_e4m3_static_noalloc's scratch is a static array of
 *     the library's device code, not an allocation);
 *   - arguments are validated on the host before anything is enqueued: a call that returns an
 *     error has enqueued nothing (all or nothing), and h3_last_error() describes the failure;
 *   - the unsupported cases return H3_EUNSUPPORTED so a caller can keep its own path;
 *   - outputs must not overlap any input or any other output (H3_EALIAS);
 *   - calls may come from several host threads at once (the per-device caches of device
 *     attributes and kernel occupancy are lock-protected; the error text is per thread);
 *   - every pass is a sequence of kernel launches on `stream` (buffers that must start at zero
 *     are cleared by a kernel, not a memset), so a caller may capture the calls in a HIP graph.
 */
#ifndef H3QK_H
#define H3QK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3_ABI_VERSION 1
#define H3_MAX_BATCH 64
#define H3_SAT_SLOTS 128                       /* partial-count slots of a clip-counter buffer */
#define H3_SAT_WORDS (16 * (H3_SAT_SLOTS + 1)) /* uint64 words of a clip-counter buffer */

typedef enum { H3_F32 = 0, H3_F16 = 1, H3_BF16 = 2, H3_E4M3FN = 3 } h3_dtype;

/* Output layout of the one-tensor entry points. */
typedef enum { H3_LAYOUT_BHTD = 0, H3_LAYOUT_BTHD = 1 } h3_layout;

enum {
    H3_OK = 0,
    H3_EINVAL = -1,       /* null pointer, non-positive size, bad stride or eps */
    H3_EUNSUPPORTED = -2, /* head dim, dtype combination or rotary split not provided */
    H3_EALIGN = -3,       /* a pointer or stride is not 16-byte aligned */
    H3_ERANGE = -4,       /* valid_len or a position falls outside the grid or the tables */
    H3_EALIAS = -5,       /* an output overlaps an input or another output */
    H3_ELAUNCH = -6       /* the HIP runtime refused the launch (message in h3_last_error) */
};

/* Problem description shared by the QK entry points (a HOST struct).  The one-tensor entry points
   read it for a single [B, T, H, D] tensor: H is that tensor's head count and row_stride, >= H*D,
   the elements between its consecutive tokens. */
typedef struct {
    int32_t B;                 /* items in the batch, 1..H3_MAX_BATCH */
    int32_t T;                 /* padded tokens per item (>= 1) */
    int32_t H;                 /* heads (>= 1) */
    int32_t D;                 /* head dim: 64 or 128 */
    int64_t row_stride;        /* elements between consecutive tokens of the fused projection,
                                  >= 3*H*D, <= 2^26, multiple of 8 (16 bytes) */
    int64_t batch_stride;      /* elements between consecutive items, multiple of 8,
                                  >= T*row_stride when B > 1 */
    int32_t grid[3];           /* Gt, Gh, Gw: token i -> (i/(Gh*Gw), (i/Gw)%Gh, i%Gw) */
    int32_t pos_offset[H3_MAX_BATCH][3]; /* per-item (t, h, w) position offsets, >= 0 */
    int32_t valid_len[H3_MAX_BATCH];     /* per-item valid tokens, 0..min(T, Gt*Gh*Gw) */
    int32_t pairs_per_axis;    /* n: rotated pairs per axis, 0 <= 6n <= D */
    int32_t table_len[3];      /* P_t, P_h, P_w: rows of the t, h, w parts of the tables;
                                  pos_offset[b][a] + grid[a] <= table_len[a] for every item;
                                  (P_t + P_h + P_w) * n <= 2^30 (else H3_EINVAL) */
    const float *cos_tab;      /* DEVICE fp32 [(P_t + P_h + P_w)][n], axis-major t, h, w;
                                  4-byte aligned (else H3_EALIGN); with both tables 8-byte
                                  aligned the kernels read neighbouring entries together;
                                  never read (may be NULL) when n = 0 */
    const float *sin_tab;      /* DEVICE fp32, same layout */
    float eps;                 /* finite, >= 0 */
} h3_qk_desc;

/*
 * Fused RMSNorm + partial 3-axis RoPE + head-major permute, one pass.
 *   qkv    DEVICE, in_dt (H3_F16 or H3_BF16), item b token i at qkv + b*batch_stride +
 *          i*row_stride, laid out [Q heads | K heads | V heads], each head's D values contiguous
 *   w_q, w_k  DEVICE fp32 [D] norm weights (shared by all heads)
 *   q_out  DEVICE [B, H, T, D] contiguous, q_dt in {H3_F32, H3_F16, H3_BF16}
 *   k_out  DEVICE [B, H, T, D] contiguous, k_dt in {H3_F32, H3_F16, H3_BF16}
 *   v_out  DEVICE [B, H, T, D] contiguous, dtype in_dt: a bit copy of the V heads
 * Q and K take y' rounded (RNE) to their dtypes; padding tokens are written as +0.
 * Follows [SDCPP-19] (fused QKV path, ggml_rope_pe_permute_rms) and [OMNI-6607] (Q/K
 * normalization + RoPE row).
 */
int h3_qk_rmsnorm_rope_permute(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                               const float *w_q, const float *w_k,
                               void *q_out, h3_dtype q_dt, void *k_out, h3_dtype k_dt,
                               void *v_out, hipStream_t stream);

/*
 * Sage emission ([SDCPP-19] sage commit: the fused RoPE/permute op writes the head-major tensors
 * the sage attention reads, with the rounding points of the unfused scale-then-cast chain):
 *   q_out  DEVICE fp32 [B, H, T, D]: y'_Q
 *   k_out  DEVICE fp32 [B, H, T, D]: RN32(y'_K * kv_scale)
 *   v_out  DEVICE fp16 [B, H, T, D]: RN16(RN32(v * kv_scale)), v the V input value (f16 or bf16)
 *   kv_scale  HOST fp32, finite.  Padding tokens are +0.
 */
int h3_qk_rmsnorm_rope_permute_sage(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                                    const float *w_q, const float *w_k, float kv_scale,
                                    float *q_out, float *k_out, uint16_t *v_out, hipStream_t stream);

/*
 * FP8 amax pass: amax_qk[0] = max |y'| over the valid Q rows of all items, amax_qk[1] the same
 * over the valid K rows ([TRT-21485] Summary and valid-length commit).
 *   amax_qk  DEVICE fp32 [2], overwritten (cleared on the stream, then reduced into).
 * Max is exact, so the result does not depend on the reduction order.  A NaN y' makes the
 * result NaN.  A multi-GPU caller all-reduces (MAX) amax_qk between this call and the cast.
 */
int h3_qk_amax(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
               const float *w_q, const float *w_k, float *amax_qk, hipStream_t stream);

/*
 * FP8 cast pass ([TRT-21485] Summary and fused_fp8_qk commit):
 *   descale_s = amax_qk[s] / 448 if amax_qk[s] > 0, else 1   (read on the device, no host sync)
 *   q_codes / k_codes  DEVICE uint8 [B, H, T, D]: E4M3FN(RN(y' / descale_s)), round to nearest
 *                      even, saturating to +-448 (also +-inf); a NaN gives a NaN code (0x7F or
 *                      0xFF, sign not specified); 0x00 for padding tokens
 *   v_out              DEVICE [B, H, T, D], dtype in_dt: bit copy of the V heads (+0 for padding)
 *   descale_qk         DEVICE fp32 [2] out: the two descales for the attention consumer
 *   amax_qk            DEVICE fp32 [2] in, from h3_qk_amax (static descales: see below)
 */
int h3_qk_cast_e4m3(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                    const float *w_q, const float *w_k, const float *amax_qk,
                    uint8_t *q_codes, uint8_t *k_codes, void *v_out, float *descale_qk,
                    hipStream_t stream);

/*
 * FP8 cast with static descales, no amax pass ([TRT-21485]: the static scale table offered as the
 * alternative to dynamic scales, the per-tensor cast of Q, K and V, and the saturation log, a
 * per-tensor count of the elements that saturate at the E4M3 range):
 *   descale_qkv  DEVICE fp32 [2] (Q, K), or [3] (Q, K, V) when v_dt is H3_E4M3FN: the caller's
 *                descales, read on the device; a value that is not > 0 (zero, negative, NaN) is
 *                read as 1.  Any calibration margin is the caller's to apply.
 *   q_codes / k_codes  DEVICE uint8 [B, H, T, D]: E4M3FN(RN(y' / descale_s)) as in h3_qk_cast_e4m3
 *   v_out        DEVICE [B, H, T, D]: v_dt == in_dt: a bit copy of the V heads; v_dt == H3_E4M3FN:
 *                uint8 codes E4M3FN(RN(v / descale_qkv[2])) of the V input values.  Padding: 0.
 *   sat_qkv      DEVICE uint64 [H3_SAT_WORDS], or NULL: a clip-counter buffer, overwritten.
 *                sat_qkv[0..2] receive the number of valid elements of Q, K, V whose binary32
 *                quotient exceeds 448 in magnitude (saturated codes; a NaN quotient is not counted;
 *                sat_qkv[2] = 0 when V is copied).  Words 16 on hold H3_SAT_SLOTS per-slot partial
 *                counts (cleared, added to, then summed, all on the stream); words 3..15 are not
 *                used.  8-byte aligned, not overlapping any other argument.
 * With descale_s = amax_s / 448 this writes the codes h3_qk_cast_e4m3 writes.
 */
int h3_qk_cast_e4m3_static(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                           const float *w_q, const float *w_k, const float *descale_qkv,
                           uint8_t *q_codes, uint8_t *k_codes, void *v_out, h3_dtype v_dt,
                           uint64_t *sat_qkv, hipStream_t stream);

/*
 * h3_qk_cast_e4m3_static for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and outputs,
 * except that no counter buffer is passed in:
 *   sat_counts   DEVICE uint64 [3], or NULL: receives the three clip counts (Q, K, V) that
 *                h3_qk_cast_e4m3_static writes to sat_qkv[0..2].  8-byte aligned.
 * The partial counts live in a static device array of the library, H3_SAT_SLOTS slots of 128
 * bytes (16 KiB), one copy per GPU held until the process ends, cleared by a kernel at the start
 * of each call.  Its size does not depend on the problem (a block adds into slot blockIdx mod
 * H3_SAT_SLOTS), so every problem h3_qk_cast_e4m3_static accepts fits it and the size limits are
 * those of that call.  Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race on it and their counts may be wrong; their
 * codes are not affected.  No hipMalloc, hipFree or other allocation is made (the array's device
 * address is looked up once per GPU, on the first call there).
 */
int h3_qk_cast_e4m3_static_noalloc(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                                   const float *w_q, const float *w_k, const float *descale_qkv,
                                   uint8_t *q_codes, uint8_t *k_codes, void *v_out, h3_dtype v_dt,
                                   uint64_t *sat_counts, hipStream_t stream);

/*
 * FP8 recipe with V cast too ([TRT-21485]: Q, K and V cast to E4M3 with per-tensor scales, a
 * dynamic amax pass then a cast pass).  Amax pass over the fused projection:
 *   amax_qkv  DEVICE fp32 [3], overwritten: [0], [1] as h3_qk_amax; [2] = max |v| over the valid
 *             V rows (V is not normalised).  A NaN makes its entry NaN.
 */
int h3_qkv_amax(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                const float *w_q, const float *w_k, float *amax_qkv, hipStream_t stream);

/*
 * Cast pass of the same recipe: descale_s = amax_qkv[s] / 448 if amax_qkv[s] > 0, else 1;
 *   q_codes, k_codes  DEVICE uint8 [B, H, T, D]: as h3_qk_cast_e4m3
 *   v_codes           DEVICE uint8 [B, H, T, D]: E4M3FN(RN(v / descale_2)); 0x00 for padding
 *   descale_qkv       DEVICE fp32 [3] out
 */
int h3_qkv_cast_e4m3(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                     const float *w_q, const float *w_k, const float *amax_qkv,
                     uint8_t *q_codes, uint8_t *k_codes, uint8_t *v_codes, float *descale_qkv,
                     hipStream_t stream);

/*
 * One separately projected tensor ([TRT-21485] norm_rope_tensor commit: a single [B, S, H, D] tensor
 * of the asynchronous Ulysses path, norm + RoPE for Q or K, the identity for V, to a 16-bit dtype
 * or to E4M3 codes with a descale per tensor; and the split mode, where a packed QKV goes through
 * these single-tensor passes with its packed row stride).
 *   x    DEVICE in_dt: head h of token i of item b at x + b*batch_stride + i*row_stride + h*D
 *        (a compact [B, T, H, D] tensor has row_stride = H*D; the K part of a fused projection is
 *        x = qkv + H*D with row_stride = 3*H*D)
 *   w    DEVICE fp32 [D]: the tensor's norm weight (y' as in the contract above), or NULL: the
 *        identity (y' = x, neither normalised nor rotated)
 *   out  DEVICE out_dt in {H3_F32, H3_F16, H3_BF16}: RN(y'), laid out [B, H, T, D]
 *        (H3_LAYOUT_BHTD) or [B, T, H, D] (H3_LAYOUT_BTHD); padding tokens +0
 */
int h3_tensor_norm_rope(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w,
                        void *out, h3_dtype out_dt, h3_layout out_layout, hipStream_t stream);

/*
 * Per-tensor amax of the same y': *amax = max |y'| over the valid rows (DEVICE fp32 [1],
 * overwritten; NaN propagates; +0 when nothing is valid).
 */
int h3_tensor_amax(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w,
                   float *amax, hipStream_t stream);

/*
 * Per-tensor E4M3 cast of the same y':
 *   scale       DEVICE fp32 [1]: an amax (scale_is_descale = 0: descale = amax / 448 if > 0, else 1)
 *               or a caller's descale (scale_is_descale = 1: used when > 0, else 1)
 *   codes       DEVICE uint8, layout out_layout: E4M3FN(RN(y' / descale)), as h3_qk_cast_e4m3
 *   descale     DEVICE fp32 [1] out, or NULL
 *   sat         DEVICE uint64 [H3_SAT_WORDS], or NULL: a clip-counter buffer as in
 *               h3_qk_cast_e4m3_static; sat[0] receives the count of valid elements whose quotient
 *               exceeds 448 in magnitude (sat[1], sat[2] = 0)
 */
int h3_tensor_cast_e4m3(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w,
                        const float *scale, int scale_is_descale, uint8_t *codes,
                        h3_layout out_layout, float *descale, uint64_t *sat, hipStream_t stream);

/*
 * SwiGLU on the 16-bit output of a decoder block's w1 projection ([OMNI-6607] Operations table,
 * SwiGLU row: silu of the gate half times the up half of the FP16 w1 projection output):
 *   x  DEVICE dt [N][2F] row-major: gate g = x[:, :F], up u = x[:, F:]
 *   y  DEVICE dt [N][F]:  y = RN_dt(v), v = RN64(RN64(g / RN64(1 + exp(-g))) * u), the silu
 *      product evaluated in binary64 and rounded once to dt (round to nearest even; NaN stays NaN,
 *      its payload and sign not specified).
 * dt is H3_F16 or H3_BF16; F a multiple of 8; N * F / 8 < 2^32; x, y 16-byte aligned, not
 * overlapping.  Each element takes a binary32 evaluation when its rounding to dt is certain to be
 * v's, and the binary64 evaluation otherwise (about one element in a thousand for data near zero,
 * every element with |g| > 64).
 */
int h3_swiglu(const void *x, h3_dtype dt, void *y, int64_t N, int64_t F, hipStream_t stream);

/*
 * Scaled residual ([OMNI-6607] Operations table, scaled-residual row: a binary32 residual plus a
 * binary16 branch multiplied by a binary32 scale, no fused multiply-add):
 *   out[n][c] = res[n][c] + (branch[n][c] * scale[scale_len == 1 ? 0 : c])
 * in binary32, the product rounded before the sum.  res, out DEVICE fp32 [N][C]; branch DEVICE
 * branch_dt (H3_F16 or H3_BF16) [N][C]; scale DEVICE fp32 [scale_len], scale_len 1 or C.  C a
 * multiple of 4; N * C / 4 < 2^32; res, out, scale 16-byte and branch 8-byte aligned; out overlaps
 * no input.
 */
int h3_scaled_residual(const float *res, const void *branch, h3_dtype branch_dt, const float *scale,
                       int64_t scale_len, float *out, int64_t N, int64_t C, hipStream_t stream);

/* Thread-local text of the last error of an h3_* call on this thread ("" after success);
   valid until the next h3_* call on the same thread. */
const char *h3_last_error(void);

/* H3_ABI_VERSION of the built library. */
int h3_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3QK_H */
