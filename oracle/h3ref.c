/*
 * h3ref — CPU oracle for the MiniMax-H3 attention input preparation:
 *   per-head RMS normalisation of every Q and K head row with a learned per-dim weight,
 *   partial 3-axis (t, h, w) rotary embedding, and a head-major [B, H, T, D] store of Q, K, V;
 *   plus the FP8 variant (per-tensor amax over the valid rows, then an OCP E4M3FN cast).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline
 * leg may load this library.  It shares no code, header or table with the GPU library.
 *
 * What is computed follows the pages:
 *   - vllm-omni PR #6607 (MiniMax-H3 VAE decoder eager ops), "Operations" table, Q/K
 *     normalization + RoPE row: one fused reduction + RoPE per Q/K tensor with a fixed RMS
 *     reduction tree and explicit rounding; scaled-residual row: the product rounded before the sum.
 *   - stable-diffusion.cpp PR #19, commit messages on the fused QKV path and on
 *     ggml_rope_pe_permute_rms: q/k read from the fused projection, per-head norm, partial RoPE,
 *     Q in binary32 and K, V in binary16 written head-major with the same products, sums and casts.
 *   - TensorRT-LLM PR #21485, Summary and the fused_fp8_qk commit messages: the FP8 path as two
 *     passes over the normalised, rotated Q and K (a per-tensor amax, then the cast with the
 *     scales it gives); padded rows (from the
 *     key-padding mask) left out of the amax; the packed QKV row stride; the static scale table
 *     and the saturation log; the cast of V; norm_rope_tensor for separately projected tensors.
 *   - stable-diffusion.cpp PR #19, the sage commit: F32 Q, F32 K * kv_scale, F16 V * kv_scale.
 *   - vllm-omni PR #6607, "Operations" table, SwiGLU and scaled-residual rows.
 * Where the pages leave a step open, the reading taken is written next to the step.  Every public
 * function here is pinned by the tests (closed forms, brute force, library routines, the numpy
 * twin in twin.py).
 *
 * Entry points keep their per-call row buffers in thread-local storage, so several host threads may
 * call them at once on disjoint outputs (the bench times the oracle on one core and on all cores).
 *
 * Arithmetic: IEEE binary32, one rounding per written operation, in the order written.
 * Build with -O2 -ffp-contract=off and without fast-math: no fused multiply-add, no
 * reassociation, no flush-to-zero.  sqrtf and '/' are correctly rounded on x86-64 SSE.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* dtype codes (match the Python wrapper) */
enum { REF_F32 = 0, REF_F16 = 1, REF_BF16 = 2, REF_E4M3 = 3 };

typedef struct {
    int32_t B, T, H, D;
    int64_t row_stride;         /* elements between consecutive tokens of one item */
    int64_t batch_stride;       /* elements between consecutive items */
    int32_t grid[3];            /* Gt, Gh, Gw */
    const int32_t *pos_offset;  /* [B][3] */
    const int32_t *valid_len;   /* [B] */
    int32_t n;                  /* rotated pairs per axis */
    int32_t table_len[3];       /* rows of the t, h, w parts of the tables */
    const float *cos_tab;       /* [(P_t + P_h + P_w)][n] */
    const float *sin_tab;
    float eps;
} h3ref_problem;

/* ------------------------------------------------------------------ scalar encodings */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Round-to-nearest-even of m / 2^s for a non-negative integer m. */
static uint64_t rne_shift(uint64_t m, int s) {
    if (s <= 0) return m;
    if (s >= 64) return 0;
    uint64_t q = m >> s;
    uint64_t rem = m & ((1ull << s) - 1);
    uint64_t half = 1ull << (s - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
    return q;
}

/* Split a finite non-zero binary32 into integer significand and unbiased exponent of its
   leading significand bit: |f| = sig * 2^(e - 23). */
static void split_f32(uint32_t a, uint64_t *sig, int *e) {
    uint32_t E = a >> 23, m = a & 0x7FFFFF;
    if (E == 0) { *sig = m; *e = -126; }          /* subnormal: no implicit bit */
    else        { *sig = m | 0x800000; *e = (int)E - 127; }
}

float h3ref_f16_decode(uint16_t h) {
    uint32_t s = (uint32_t)(h & 0x8000) << 16, E = (h >> 10) & 0x1F, m = h & 0x3FF;
    float v;
    if (E == 0)       v = ldexpf((float)m, -24);                 /* exact */
    else if (E == 31) return bits_to_f32(s | 0x7F800000 | (m << 13));
    else              v = ldexpf((float)(m | 0x400), (int)E - 25);
    return bits_to_f32(s | f32_to_bits(v));
}

/* binary32 -> binary16, round to nearest even, overflow to infinity, NaN stays NaN (quiet). */
uint16_t h3ref_f16_encode(float f) {
    uint32_t x = f32_to_bits(f), sign = (x >> 16) & 0x8000, a = x & 0x7FFFFFFF;
    if (a > 0x7F800000) return (uint16_t)(sign | 0x7E00 | ((a >> 13) & 0x3FF));
    if (a >= 0x477FF000) return (uint16_t)(sign | 0x7C00);      /* >= 65520 rounds past 65504 */
    if (a == 0) return (uint16_t)sign;
    uint64_t sig; int e; split_f32(a, &sig, &e);
    /* normal results (e >= -14): drop 13 bits; the carry may bump the exponent.
       subnormal results: k = |f| * 2^24 rounded, stored as the code itself. */
    if (e >= -14) return (uint16_t)(sign | (((uint32_t)(e + 14) << 10) + (uint32_t)rne_shift(sig, 13)));
    return (uint16_t)(sign | (uint32_t)rne_shift(sig, 13 + (-14 - e)));
}

float h3ref_bf16_decode(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest even, NaN stays NaN (quiet). */
uint16_t h3ref_bf16_encode(float f) {
    uint32_t x = f32_to_bits(f);
    if ((x & 0x7FFFFFFF) > 0x7F800000) return (uint16_t)((x >> 16) | 0x40);
    uint32_t lo = x & 0xFFFF, hi = x >> 16;
    if (lo > 0x8000 || (lo == 0x8000 && (hi & 1))) hi += 1;
    return (uint16_t)hi;
}

/* binary32 -> OCP FP8 E4M3FN (bias 7, no infinities, S.1111.111 = NaN, max finite 448,
   subnormal step 2^-9), round to nearest even, saturating: |f| > 448 and +-inf give +-448;
   NaN gives 0x7F with the sign. */
uint8_t h3ref_e4m3_encode(float f) {
    uint32_t x = f32_to_bits(f), sign = (x >> 24) & 0x80, a = x & 0x7FFFFFFF;
    if (a > 0x7F800000) return (uint8_t)(sign | 0x7F);
    if (a > 0x43E00000) return (uint8_t)(sign | 0x7E);          /* > 448 */
    if (a == 0) return (uint8_t)sign;
    uint64_t sig; int e; split_f32(a, &sig, &e);
    if (e >= -6) return (uint8_t)(sign | (((uint32_t)(e + 6) << 3) + (uint32_t)rne_shift(sig, 20)));
    return (uint8_t)(sign | (uint32_t)rne_shift(sig, 20 + (-6 - e)));
}

float h3ref_e4m3_decode(uint8_t c) {
    uint32_t s = (uint32_t)(c & 0x80) << 24, E = (c >> 3) & 0xF, m = c & 7;
    if (E == 15 && m == 7) return bits_to_f32(s | 0x7FC00000);
    float v = (E == 0) ? ldexpf((float)m, -9) : ldexpf((float)(m | 8), (int)E - 10);
    return bits_to_f32(s | f32_to_bits(v));
}

void h3ref_f16_encode_array(const float *x, uint16_t *y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = h3ref_f16_encode(x[i]); }
void h3ref_bf16_encode_array(const float *x, uint16_t *y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = h3ref_bf16_encode(x[i]); }
void h3ref_e4m3_encode_array(const float *x, uint8_t *y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = h3ref_e4m3_encode(x[i]); }

/* ------------------------------------------------------------------ the row */

static float load_in(const void *base, int dt, int64_t idx) {
    const uint16_t *p = (const uint16_t *)base;
    return dt == REF_BF16 ? h3ref_bf16_decode(p[idx]) : h3ref_f16_decode(p[idx]);
}

/*
 * One Q or K head row: RMS normalisation with weight w, then the partial 3-axis rotation.
 *   a_d = x_d * x_d
 *   fixed halving tree: for o = D/2, D/4, ..., 1 and d < o:  a_d = a_d + a_{d+o};  ss = a_0
 *     (reading of the pages' "reference RMS reduction order/tree", which they never print:
 *      the balanced tree a 64-lane wavefront computes with one dimension per lane)
 *   ms = ss * (1/D)   (exact scaling for power-of-two D)
 *   r  = 1 / sqrt(ms + eps)   (correctly rounded sqrt, then correctly rounded division)
 *   y_d = (x_d * r) * w_d
 *   pair p < 3n rotates (y_2p, y_2p+1) by the table entry of axis p / n, frequency p mod n:
 *     y'_2p = e c - f s,  y'_2p+1 = e s + f c   (each product rounded, then the sum)
 *   dimensions >= 6n pass through.
 * crow[a], srow[a] point at the n entries of the table row for axis a at this token.
 */
void h3ref_norm_rope_row(const float *x, int D, const float *w, float eps, int n,
                         const float *const crow[3], const float *const srow[3], float *y) {
    float a[256];
    for (int d = 0; d < D; ++d) a[d] = x[d] * x[d];
    for (int o = D / 2; o >= 1; o /= 2)
        for (int d = 0; d < o; ++d) a[d] = a[d] + a[d + o];
    float ms = a[0] * (1.0f / (float)D);
    float v = ms + eps;
    float sq = sqrtf(v);
    float r = 1.0f / sq;
    for (int d = 0; d < D; ++d) {
        float t = x[d] * r;
        y[d] = t * w[d];
    }
    for (int p = 0; p < 3 * n; ++p) {
        int axis = p / n, j = p % n;
        float c = crow[axis][j], s = srow[axis][j];
        float e = y[2 * p], f = y[2 * p + 1];
        float ec = e * c, fs = f * s, es = e * s, fc = f * c;
        y[2 * p] = ec - fs;
        y[2 * p + 1] = es + fc;
    }
}

/* Token i of item b -> table rows of its t, h, w positions (flattened t-major grid, w fastest,
   plus the item's offsets).  Returns 0, or -1 when a position falls outside its table part. */
int h3ref_token_rows(const h3ref_problem *P, int b, int64_t i, int rows[3]) {
    int64_t gh = P->grid[1], gw = P->grid[2];
    int64_t pos[3];
    pos[0] = i / (gh * gw) + P->pos_offset[3 * b + 0];
    pos[1] = (i / gw) % gh + P->pos_offset[3 * b + 1];
    pos[2] = i % gw + P->pos_offset[3 * b + 2];
    int64_t base = 0;
    for (int a = 0; a < 3; ++a) {
        if (pos[a] < 0 || pos[a] >= P->table_len[a]) return -1;
        rows[a] = (int)(base + pos[a]);
        base += P->table_len[a];
    }
    return 0;
}

static void store_out(void *dst, int dt, int64_t idx, float v) {
    switch (dt) {
    case REF_F32: ((float *)dst)[idx] = v; break;
    case REF_F16: ((uint16_t *)dst)[idx] = h3ref_f16_encode(v); break;
    case REF_BF16: ((uint16_t *)dst)[idx] = h3ref_bf16_encode(v); break;
    default: ((uint8_t *)dst)[idx] = h3ref_e4m3_encode(v); break;
    }
}

static int dt_size(int dt) { return dt == REF_F32 ? 4 : (dt == REF_E4M3 ? 1 : 2); }

/*
 * y' of every Q row (slot 0, weight w_q) and K row (slot 1, weight w_k) of token i of item b:
 * yqk[s][h][d].  `row` points at the token's first element of the fused projection, laid out
 * [Q heads | K heads | V heads] with each head's D values contiguous.
 * Returns 1 for a padded token (i >= valid_len[b]; nothing computed), 0 otherwise, and -1 when a
 * position falls outside the tables.
 */
static int token_qk(const h3ref_problem *P, const uint16_t *row, int in_dt, const float *w_q,
                    const float *w_k, int b, int64_t i, float *yqk) {
    if (i >= P->valid_len[b]) return 1;
    int rows[3];
    if (h3ref_token_rows(P, b, i, rows) != 0) return -1;
    const float *crow[3], *srow[3];
    for (int a = 0; a < 3; ++a) {
        crow[a] = P->cos_tab + (int64_t)rows[a] * P->n;
        srow[a] = P->sin_tab + (int64_t)rows[a] * P->n;
    }
    float x[256];
    int H = P->H, D = P->D;
    for (int s = 0; s < 2; ++s)
        for (int h = 0; h < H; ++h) {
            for (int d = 0; d < D; ++d) x[d] = load_in(row, in_dt, ((int64_t)s * H + h) * D + d);
            h3ref_norm_rope_row(x, D, s == 0 ? w_q : w_k, P->eps, P->n, crow, srow,
                                yqk + ((int64_t)s * H + h) * D);
        }
    return 0;
}

/*
 * What one store writes.  fp8 == 0: Q and K take y' rounded to q_dt / k_dt, V is a bit copy.
 * fp8 == 1: Q and K take E4M3(y' / ds[s]); V takes E4M3(v / ds[2]) when v_fp8, else a bit copy.
 * sat (optional) counts, per tensor (Q, K, V), the cast elements whose quotient lies outside the
 * E4M3 range, |y' / ds| > 448 (TensorRT-LLM PR #21485, the saturation-log commit: a per-tensor
 * count of what saturates).  A NaN quotient is not counted; padded tokens are not counted.
 */
typedef struct {
    int fp8, v_fp8;
    float ds[3];
    uint64_t *sat;
} store_opts;

static uint8_t cast_one(float t, float ds, uint64_t *sat) {
    float q = t / ds;
    if (sat && fabsf(q) > 448.0f) *sat += 1;
    return h3ref_e4m3_encode(q);
}

/*
 * Store one token.  A padded token is +0 everywhere.  Output element (h, d) of this token goes
 * to index o0 + h * head_stride + d.
 */
static void store_token(const h3ref_problem *P, const uint16_t *row, int in_dt, int padded,
                        const float *yqk, const store_opts *so, void *q, int q_dt, void *k, int k_dt,
                        void *v, int64_t o0, int64_t head_stride) {
    int H = P->H, D = P->D;
    for (int h = 0; h < H; ++h) {
        int64_t o = o0 + (int64_t)h * head_stride;
        for (int s = 0; s < 2; ++s) {
            void *dst = s == 0 ? q : k;
            int dt = so->fp8 ? REF_E4M3 : (s == 0 ? q_dt : k_dt);
            const float *y = yqk + ((int64_t)s * H + h) * D;
            for (int d = 0; d < D; ++d) {
                if (padded) { memset((char *)dst + (o + d) * dt_size(dt), 0, (size_t)dt_size(dt)); continue; }
                if (so->fp8) ((uint8_t *)dst)[o + d] = cast_one(y[d], so->ds[s], so->sat ? so->sat + s : 0);
                else store_out(dst, dt, o + d, y[d]);
            }
        }
        int64_t vi = ((int64_t)2 * H + h) * D;
        for (int d = 0; d < D; ++d) {
            if (so->fp8 && so->v_fp8)
                ((uint8_t *)v)[o + d] = padded ? 0 : cast_one(load_in(row, in_dt, vi + d), so->ds[2],
                                                              so->sat ? so->sat + 2 : 0);
            else
                ((uint16_t *)v)[o + d] = padded ? 0 : row[vi + d];
        }
    }
}

/* descale = amax / 448 when amax > 0, else 1 (an all-zero or empty tensor). */
float h3ref_descale(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

/* A descale from a caller's table: used as given when > 0, else 1 (zero, negative or NaN), the
   same guard as the dynamic descale. */
float h3ref_static_descale(float d) { return d > 0.0f ? d : 1.0f; }

static int run_items(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                     const float *w_k, const store_opts *so, void *q, int q_dt, void *k, int k_dt,
                     void *v) {
    int H = P->H, D = P->D;
    int64_t plane = (int64_t)H * P->T * D;
    static __thread float yqk[2 * 64 * 256];
    if (H > 64 || D > 256) return -2;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->T; ++i) {
            const uint16_t *row = (const uint16_t *)qkv + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_qk(P, row, in_dt, w_q, w_k, b, i, yqk);
            if (rc < 0) return rc;
            store_token(P, row, in_dt, rc == 1, yqk, so, q, q_dt, k, k_dt, v, b * plane + i * D,
                        (int64_t)P->T * D);
        }
    return 0;
}

/*
 * Non-FP8 pass over the whole problem.  q, k, v are head-major [B, H, T, D]: Q and K take y'
 * rounded to q_dt / k_dt, V is a bit copy of the input, padded tokens are +0.
 */
int h3ref_qk_rmsnorm_rope_permute(const h3ref_problem *P, const void *qkv, int in_dt,
                                  const float *w_q, const float *w_k,
                                  void *q, int q_dt, void *k, int k_dt, void *v) {
    store_opts so = {0, 0, {1.0f, 1.0f, 1.0f}, 0};
    return run_items(P, qkv, in_dt, w_q, w_k, &so, q, q_dt, k, k_dt, v);
}

/*
 * Per-tensor amax: amax[0] = max |y'| over the valid Q rows of every item, amax[1] the same for
 * K.  Padded rows do not enter; an empty set gives +0.  A NaN |y'| makes the maximum NaN.
 */
int h3ref_qk_amax(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                  const float *w_k, float amax[2]) {
    static __thread float yqk[2 * 64 * 256];
    int H = P->H, D = P->D;
    if (H > 64 || D > 256) return -2;
    amax[0] = 0.0f; amax[1] = 0.0f;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->valid_len[b]; ++i) {
            const uint16_t *row = (const uint16_t *)qkv + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_qk(P, row, in_dt, w_q, w_k, b, i, yqk);
            if (rc < 0) return rc;
            for (int s = 0; s < 2; ++s)
                for (int64_t e = 0; e < (int64_t)H * D; ++e) {
                    float m = fabsf(yqk[(int64_t)s * H * D + e]);
                    if (isnan(m) || isnan(amax[s])) amax[s] = NAN;
                    else if (m > amax[s]) amax[s] = m;
                }
        }
    return 0;
}

/*
 * FP8 cast pass: descale_s = amax_s / 448 (1 when amax_s is not > 0), Q and K codes
 * E4M3(y' / descale_s) head-major [B, H, T, D], V a bit copy of the 16-bit input, padded tokens
 * +0 (code 0x00).  descale[2] receives the two descales.
 */
int h3ref_qk_cast_e4m3(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                       const float *w_k, const float amax[2], uint8_t *q, uint8_t *k, void *v,
                       float descale[2]) {
    store_opts so = {1, 0, {h3ref_descale(amax[0]), h3ref_descale(amax[1]), 1.0f}, 0};
    if (descale) { descale[0] = so.ds[0]; descale[1] = so.ds[1]; }
    return run_items(P, qkv, in_dt, w_q, w_k, &so, q, REF_E4M3, k, REF_E4M3, v);
}

/*
 * FP8 cast with static descales (TensorRT-LLM PR #21485: a static scale table as the opt-in
 * alternative to the dynamic amax pass; the saturation-log commit).  descale[0], [1] (and [2]
 * when v_fp8) come from the caller, each guarded by h3ref_static_descale.  Q and K codes are
 * E4M3(y' / descale_s); V is E4M3(v / descale_2) when v_fp8, else a bit copy.  sat[3] (optional)
 * is overwritten with the per-tensor counts of |quotient| > 448 (sat[2] = 0 when V is copied).
 */
int h3ref_qk_cast_e4m3_static(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                              const float *w_k, const float *descale, int v_fp8, uint8_t *q,
                              uint8_t *k, void *v, uint64_t *sat) {
    store_opts so = {1, v_fp8 ? 1 : 0,
                     {h3ref_static_descale(descale[0]), h3ref_static_descale(descale[1]),
                      v_fp8 ? h3ref_static_descale(descale[2]) : 1.0f},
                     sat};
    if (sat) { sat[0] = 0; sat[1] = 0; sat[2] = 0; }
    return run_items(P, qkv, in_dt, w_q, w_k, &so, q, REF_E4M3, k, REF_E4M3, v);
}

/*
 * The same outputs for a list of tokens only (flat ids b * T + i), reading a compact input
 * qkv_rows [n_tok][row_stride] whose row t is token tokens[t].  Outputs are [n_tok][H][D].
 * fp8 == 0: Q, K in q_dt, k_dt (descale ignored).  fp8 == 1: E4M3 codes with the final descales
 * descale[3] (V codes with descale[2] when v_fp8).  yf32 (optional) receives y' as f32
 * [n_tok][2][H][D] (zeros for padded tokens); sat[3] (optional) is added to.
 */
int h3ref_qk_tokens_ex(const h3ref_problem *P, const void *qkv_rows, int in_dt, const float *w_q,
                       const float *w_k, const int64_t *tokens, int64_t n_tok, int fp8,
                       const float *descale, int v_fp8, void *q, int q_dt, void *k, int k_dt, void *v,
                       float *yf32, uint64_t *sat) {
    static __thread float yqk[2 * 64 * 256];
    int H = P->H, D = P->D;
    if (H > 64 || D > 256) return -2;
    store_opts so = {fp8 ? 1 : 0, fp8 && v_fp8 ? 1 : 0, {1.0f, 1.0f, 1.0f}, sat};
    if (fp8) { so.ds[0] = descale[0]; so.ds[1] = descale[1]; if (v_fp8) so.ds[2] = descale[2]; }
    for (int64_t t = 0; t < n_tok; ++t) {
        int b = (int)(tokens[t] / P->T);
        int64_t i = tokens[t] % P->T;
        const uint16_t *row = (const uint16_t *)qkv_rows + t * P->row_stride;
        int rc = token_qk(P, row, in_dt, w_q, w_k, b, i, yqk);
        if (rc < 0) return rc;
        if (rc == 1) memset(yqk, 0, sizeof(float) * 2 * H * D);
        if (yf32) memcpy(yf32 + t * 2 * H * D, yqk, sizeof(float) * 2 * H * D);
        store_token(P, row, in_dt, rc == 1, yqk, &so, q, fp8 ? REF_E4M3 : q_dt, k,
                    fp8 ? REF_E4M3 : k_dt, v, t * H * D, D);
    }
    return 0;
}

/* h3ref_qk_tokens_ex with descales from amax (fp8 == 1) and V copied. */
int h3ref_qk_tokens(const h3ref_problem *P, const void *qkv_rows, int in_dt, const float *w_q,
                    const float *w_k, const int64_t *tokens, int64_t n_tok, int fp8,
                    const float *amax, void *q, int q_dt, void *k, int k_dt, void *v, float *yf32) {
    float ds[3] = {1.0f, 1.0f, 1.0f};
    if (fp8) { ds[0] = h3ref_descale(amax[0]); ds[1] = h3ref_descale(amax[1]); }
    return h3ref_qk_tokens_ex(P, qkv_rows, in_dt, w_q, w_k, tokens, n_tok, fp8, ds, 0, q, q_dt, k, k_dt,
                              v, yf32, 0);
}

/* ------------------------------------------------------------------ V in the FP8 recipe
 * TensorRT-LLM PR #21485, the commits on the per-tensor FP8 recipe: Q, K and V are cast to E4M3,
 * each with its own per-tensor scale.  V is not normalised: its amax is max |v| over the valid
 * rows of the V heads, and its codes are E4M3(v / descale_v).
 */

/* amax[0], amax[1] as h3ref_qk_amax; amax[2] = max |v| over the valid V rows (NaN propagates). */
int h3ref_qkv_amax(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                   const float *w_k, float amax[3]) {
    int rc = h3ref_qk_amax(P, qkv, in_dt, w_q, w_k, amax);
    if (rc) return rc;
    int H = P->H, D = P->D;
    amax[2] = 0.0f;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->valid_len[b]; ++i) {
            const uint16_t *row = (const uint16_t *)qkv + (int64_t)b * P->batch_stride + i * P->row_stride;
            for (int64_t e = 0; e < (int64_t)H * D; ++e) {
                float m = fabsf(load_in(row, in_dt, 2 * (int64_t)H * D + e));
                if (isnan(m) || isnan(amax[2])) amax[2] = NAN;
                else if (m > amax[2]) amax[2] = m;
            }
        }
    return 0;
}

/* Dynamic cast of Q, K and V: descale_s = amax_s / 448 (1 when amax_s is not > 0); Q, K, V codes
   head-major [B, H, T, D]; descale[3] receives the three descales. */
int h3ref_qkv_cast_e4m3(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q,
                        const float *w_k, const float amax[3], uint8_t *q, uint8_t *k, uint8_t *v,
                        float descale[3]) {
    store_opts so = {1, 1, {h3ref_descale(amax[0]), h3ref_descale(amax[1]), h3ref_descale(amax[2])}, 0};
    if (descale) { descale[0] = so.ds[0]; descale[1] = so.ds[1]; descale[2] = so.ds[2]; }
    return run_items(P, qkv, in_dt, w_q, w_k, &so, q, REF_E4M3, k, REF_E4M3, v);
}

/* ------------------------------------------------------------------ one separately projected tensor
 * TensorRT-LLM PR #21485, the norm_rope_tensor commit: a single [B, S, H, D] tensor of the asynchronous
 * Ulysses path (there Q, K and V come out of three projections) goes through norm + RoPE (Q, K) or the
 * identity (V) to a 16-bit dtype, or to E4M3 codes with a descale per tensor; and the split
 * launch mode that runs the packed QKV through these per-tensor passes with the packed row stride.
 * The problem's H is the tensor's head count; head h of token i of item b starts at element
 * b * batch_stride + i * row_stride + h * D.  Output layout 0 is [B, H, T, D], layout 1 is
 * [B, T, H, D].  Reading: with no weight (V) the value is the input itself, not normalised or
 * rotated.
 */

static int64_t out_index(const h3ref_problem *P, int layout, int b, int h, int64_t i, int d) {
    if (layout == 0) return (((int64_t)b * P->H + h) * P->T + i) * P->D + d;
    return (((int64_t)b * P->T + i) * P->H + h) * P->D + d;
}

/* y' [H][D] of token i of item b.  Returns 1 for a padded token, 0, or -1 (position off the tables). */
static int token_tensor(const h3ref_problem *P, const uint16_t *row, int in_dt, const float *w, int b,
                        int64_t i, float *y) {
    if (i >= P->valid_len[b]) return 1;
    int H = P->H, D = P->D;
    if (!w) {
        for (int64_t e = 0; e < (int64_t)H * D; ++e) y[e] = load_in(row, in_dt, e);
        return 0;
    }
    int rows[3];
    if (h3ref_token_rows(P, b, i, rows) != 0) return -1;
    const float *crow[3], *srow[3];
    for (int a = 0; a < 3; ++a) {
        crow[a] = P->cos_tab + (int64_t)rows[a] * P->n;
        srow[a] = P->sin_tab + (int64_t)rows[a] * P->n;
    }
    float x[256];
    for (int h = 0; h < H; ++h) {
        for (int d = 0; d < D; ++d) x[d] = load_in(row, in_dt, (int64_t)h * D + d);
        h3ref_norm_rope_row(x, D, w, P->eps, P->n, crow, srow, y + (int64_t)h * D);
    }
    return 0;
}

/* 16-bit or f32 output: out = RN_out_dt(y'), +0 for padded tokens. */
int h3ref_tensor_norm_rope(const h3ref_problem *P, const void *x, int in_dt, const float *w, void *out,
                           int out_dt, int layout) {
    static __thread float y[64 * 256];
    if (P->H > 64 || P->D > 256) return -2;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->T; ++i) {
            const uint16_t *row = (const uint16_t *)x + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_tensor(P, row, in_dt, w, b, i, y);
            if (rc < 0) return rc;
            for (int h = 0; h < P->H; ++h)
                for (int d = 0; d < P->D; ++d) {
                    int64_t o = out_index(P, layout, b, h, i, d);
                    if (rc == 1) memset((char *)out + o * dt_size(out_dt), 0, (size_t)dt_size(out_dt));
                    else store_out(out, out_dt, o, y[(int64_t)h * P->D + d]);
                }
        }
    return 0;
}

/* amax = max |y'| over the valid rows (NaN propagates; +0 when nothing is valid). */
int h3ref_tensor_amax(const h3ref_problem *P, const void *x, int in_dt, const float *w, float *amax) {
    static __thread float y[64 * 256];
    if (P->H > 64 || P->D > 256) return -2;
    *amax = 0.0f;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->valid_len[b]; ++i) {
            const uint16_t *row = (const uint16_t *)x + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_tensor(P, row, in_dt, w, b, i, y);
            if (rc < 0) return rc;
            for (int64_t e = 0; e < (int64_t)P->H * P->D; ++e) {
                float m = fabsf(y[e]);
                if (isnan(m) || isnan(*amax)) *amax = NAN;
                else if (m > *amax) *amax = m;
            }
        }
    return 0;
}

/* FP8 codes E4M3(y' / ds) with ds = descale(scale) (is_descale == 0: scale is the amax) or
   static_descale(scale) (is_descale == 1); *descale (optional) receives ds; *sat (optional) is
   overwritten with the count of valid elements whose quotient exceeds 448 in magnitude. */
int h3ref_tensor_cast_e4m3(const h3ref_problem *P, const void *x, int in_dt, const float *w, float scale,
                           int is_descale, uint8_t *out, int layout, float *descale, uint64_t *sat) {
    static __thread float y[64 * 256];
    if (P->H > 64 || P->D > 256) return -2;
    float ds = is_descale ? h3ref_static_descale(scale) : h3ref_descale(scale);
    if (descale) *descale = ds;
    if (sat) *sat = 0;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->T; ++i) {
            const uint16_t *row = (const uint16_t *)x + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_tensor(P, row, in_dt, w, b, i, y);
            if (rc < 0) return rc;
            for (int h = 0; h < P->H; ++h)
                for (int d = 0; d < P->D; ++d) {
                    int64_t o = out_index(P, layout, b, h, i, d);
                    out[o] = rc == 1 ? 0 : cast_one(y[(int64_t)h * P->D + d], ds, sat);
                }
        }
    return 0;
}

/* ------------------------------------------------------------------ sage emission
 * stable-diffusion.cpp PR #19, the commit on the sage path: the fused RoPE/permute op writes the
 * head-major tensors the sage attention reads (Q in binary32, K scaled by kv_scale in binary32, V
 * scaled by kv_scale in binary16), with
 * the arithmetic and rounding points of the unfused chain (scale, then cast).  Reading: K' =
 * RN32(y'_K * kv_scale); V' = RN16(RN32(v * kv_scale)) with v the input value as binary32; Q = y'_Q.
 * Padded tokens are +0.
 */
int h3ref_qk_sage(const h3ref_problem *P, const void *qkv, int in_dt, const float *w_q, const float *w_k,
                  float kv_scale, float *q, float *k, uint16_t *v) {
    static __thread float yqk[2 * 64 * 256];
    int H = P->H, D = P->D;
    if (H > 64 || D > 256) return -2;
    int64_t plane = (int64_t)H * P->T * D;
    for (int b = 0; b < P->B; ++b)
        for (int64_t i = 0; i < P->T; ++i) {
            const uint16_t *row = (const uint16_t *)qkv + (int64_t)b * P->batch_stride + i * P->row_stride;
            int rc = token_qk(P, row, in_dt, w_q, w_k, b, i, yqk);
            if (rc < 0) return rc;
            for (int h = 0; h < H; ++h)
                for (int d = 0; d < D; ++d) {
                    int64_t o = b * plane + ((int64_t)h * P->T + i) * D + d;
                    if (rc == 1) { q[o] = 0.0f; k[o] = 0.0f; v[o] = 0; continue; }
                    q[o] = yqk[(int64_t)h * D + d];
                    float ks = yqk[((int64_t)H + h) * D + d] * kv_scale;
                    k[o] = ks;
                    float vs = load_in(row, in_dt, ((int64_t)2 * H + h) * D + d) * kv_scale;
                    v[o] = h3ref_f16_encode(vs);
                }
        }
    return 0;
}

/* ------------------------------------------------------------------ decoder-block elementwise ops
 * vllm-omni PR #6607, "Operations" table, SwiGLU and scaled-residual rows (and the B300 isolated
 * measurements in the review thread): SwiGLU is the silu-and-multiply of the FP16 output of w1 (gate =
 * first half of the last dim, up = second half); the scaled residual adds to a binary32 residual
 * the binary16 branch multiplied by a binary32 scale, the product rounded on its own.
 */

/* binary64 -> binary16, one rounding to nearest even (overflow to infinity, NaN stays NaN). */
uint16_t h3ref_f16_encode_f64(double v) {
    uint64_t x; memcpy(&x, &v, 8);
    uint16_t sign = (uint16_t)((x >> 48) & 0x8000);
    uint64_t a = x & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7E00);
    if (a == 0) return sign;
    int E = (int)(a >> 52);
    uint64_t sig = (a & 0xFFFFFFFFFFFFFull) | (E ? (1ull << 52) : 0);
    int e = E ? E - 1023 : -1022;
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    uint64_t code;
    if (e >= -14) code = ((uint64_t)(e + 14) << 10) + rne_shift(sig, 42);
    else code = rne_shift(sig, 42 + (-14 - e));
    if (code >= 0x7C00) code = 0x7C00;  /* rounded past 65504 */
    return (uint16_t)(sign | code);
}

/* binary64 -> bfloat16, one rounding to nearest even (overflow to infinity, NaN stays NaN). */
uint16_t h3ref_bf16_encode_f64(double v) {
    uint64_t x; memcpy(&x, &v, 8);
    uint16_t sign = (uint16_t)((x >> 48) & 0x8000);
    uint64_t a = x & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7FC0);
    if (a == 0) return sign;
    int E = (int)(a >> 52);
    uint64_t sig = (a & 0xFFFFFFFFFFFFFull) | (E ? (1ull << 52) : 0);
    int e = E ? E - 1023 : -1022;
    if (e > 127) return (uint16_t)(sign | 0x7F80);
    uint64_t code;
    if (e >= -126) code = ((uint64_t)(e + 126) << 7) + rne_shift(sig, 45);
    else code = rne_shift(sig, 45 + (-126 - e));
    if (code >= 0x7F80) code = 0x7F80;  /* rounded past the largest finite value */
    return (uint16_t)(sign | code);
}

/* y = silu(g) * u with g = x[:, :F], u = x[:, F:], silu(g) = g / (1 + exp(-g)), evaluated in binary64
   (libm exp) and rounded once to binary16.  x, y are binary16 bits; x is [N][2F], y is [N][F]. */
void h3ref_swiglu(const uint16_t *x, uint16_t *y, int64_t N, int64_t F, int in_dt) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t f = 0; f < F; ++f) {
            double g = load_in(x, in_dt, n * 2 * F + f);
            double u = load_in(x, in_dt, n * 2 * F + F + f);
            double s = g / (1.0 + exp(-g));
            double v = s * u;
            y[n * F + f] = in_dt == REF_BF16 ? h3ref_bf16_encode_f64(v) : h3ref_f16_encode_f64(v);
        }
}

/* out[n][c] = res[n][c] + (branch[n][c] * scale[c or 0]) in binary32: the product rounded, then the
   sum (no fused multiply-add).  branch is 16-bit (in_dt), res / scale / out are fp32. */
void h3ref_scaled_residual(const float *res, const uint16_t *branch, const float *scale, int64_t scale_len,
                           float *out, int64_t N, int64_t C, int in_dt) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < C; ++c) {
            float b = load_in(branch, in_dt, n * C + c);
            float t = b * scale[scale_len == 1 ? 0 : c];
            out[n * C + c] = res[n * C + c] + t;
        }
}
