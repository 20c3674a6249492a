/*
 * libh3qk from plain C, with no Python or PyTorch in the process: device buffers from the HIP
 * runtime, then the fused store, the FP8 amax + cast pair and the static-scale cast with V codes
 * and clip counters, on ragged padded problems (two items with offsets and valid lengths, padded
 * row and batch strides).  Every output is compared bit for bit with the CPU oracle
 * (liboracle_h3ref, test infrastructure, linked by this test program only).  Exit status 0 when
 * everything matches; each mismatch is printed.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "h3qk.h"

/* The oracle's C interface (oracle/h3ref.c). */
typedef struct {
    int32_t B, T, H, D;
    int64_t row_stride, batch_stride;
    int32_t grid[3];
    const int32_t *pos_offset;
    const int32_t *valid_len;
    int32_t n;
    int32_t table_len[3];
    const float *cos_tab, *sin_tab;
    float eps;
} h3ref_problem;
int h3ref_qk_rmsnorm_rope_permute(const h3ref_problem *, const void *, int, const float *, const float *,
                                  void *, int, void *, int, void *);
int h3ref_qk_amax(const h3ref_problem *, const void *, int, const float *, const float *, float *);
int h3ref_qk_cast_e4m3(const h3ref_problem *, const void *, int, const float *, const float *, const float *,
                       uint8_t *, uint8_t *, void *, float *);
int h3ref_qk_cast_e4m3_static(const h3ref_problem *, const void *, int, const float *, const float *,
                              const float *, int, uint8_t *, uint8_t *, void *, uint64_t *);
uint16_t h3ref_f16_encode(float);
uint16_t h3ref_bf16_encode(float);

static int failures = 0;

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

#define H3_OK_CALL(call)                                                              \
    do {                                                                              \
        int r_ = (call);                                                              \
        if (r_ != H3_OK) {                                                            \
            fprintf(stderr, "%s:%d: %s -> %d: %s\n", __FILE__, __LINE__, #call, r_, h3_last_error()); \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

/* SplitMix64: the test's own input generator. */
static uint64_t sm_state;
static uint64_t sm_next(void) {
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float sm_uniform(float lo, float hi) { return lo + (hi - lo) * (float)((sm_next() >> 40) * (1.0 / 16777216.0)); }

static void *dev_upload(const void *h, size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    if (h) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void *dev_junk(size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemset(d, 0xA5, bytes)); /* junk: every element must be written */
    return d;
}

static void expect_same(const char *what, const void *dev, const void *ref, size_t bytes) {
    unsigned char *h = (unsigned char *)malloc(bytes);
    HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    size_t bad = 0, first = 0;
    for (size_t i = 0; i < bytes; ++i)
        if (h[i] != ((const unsigned char *)ref)[i]) {
            if (!bad) first = i;
            ++bad;
        }
    if (bad) {
        fprintf(stderr, "MISMATCH %s: %zu of %zu bytes differ, first at byte %zu\n", what, bad, bytes, first);
        ++failures;
    } else {
        printf("ok %s (%zu bytes)\n", what, bytes);
    }
    free(h);
}

typedef struct {
    const char *name;
    int B, T, H, D, n, in_dt;
    int grid[3];
    int valid[2];
    int off[2][3];
    int row_pad, batch_pad; /* extra elements per token row / per item */
} problem_case;

static void run_case(const problem_case *pc) {
    const int B = pc->B, T = pc->T, H = pc->H, D = pc->D, n = pc->n;
    printf("case %s: B=%d T=%d H=%d D=%d n=%d in=%s\n", pc->name, B, T, H, D, n, pc->in_dt == H3_BF16 ? "bf16" : "f16");
    const int64_t rs = 3LL * H * D + pc->row_pad, bs = (int64_t)T * rs + pc->batch_pad;
    const int64_t in_elems = (int64_t)(B - 1) * bs + (int64_t)T * rs;
    const int64_t out_elems = (int64_t)B * H * T * D;

    /* inputs: values uniform in [-3, 3) rounded to the input dtype, junk in the stride padding */
    uint16_t *qkv = (uint16_t *)malloc((size_t)in_elems * 2);
    for (int64_t e = 0; e < in_elems; ++e) {
        const float v = sm_uniform(-3.0f, 3.0f);
        qkv[e] = pc->in_dt == H3_BF16 ? h3ref_bf16_encode(v) : h3ref_f16_encode(v);
    }
    float *wq = (float *)malloc((size_t)D * 4), *wk = (float *)malloc((size_t)D * 4);
    for (int d = 0; d < D; ++d) {
        wq[d] = sm_uniform(0.7f, 1.3f);
        wk[d] = sm_uniform(0.7f, 1.3f);
    }
    int32_t off[2 * 3] = {0}, vlen[2] = {0};
    int32_t tl[3];
    for (int a = 0; a < 3; ++a) {
        int m = 0;
        for (int b = 0; b < B; ++b) {
            off[3 * b + a] = pc->off[b][a];
            if (pc->off[b][a] > m) m = pc->off[b][a];
        }
        tl[a] = pc->grid[a] + m;
    }
    for (int b = 0; b < B; ++b) vlen[b] = pc->valid[b];
    const int rows = tl[0] + tl[1] + tl[2];
    float *cs = (float *)malloc((size_t)rows * n * 4 + 4), *sn = (float *)malloc((size_t)rows * n * 4 + 4);
    for (int a = 0, base = 0; a < 3; base += tl[a], ++a)
        for (int p = 0; p < tl[a]; ++p)
            for (int j = 0; j < n; ++j) {
                const double ang = p * pow(10000.0, -(double)j / n);
                cs[(base + p) * n + j] = (float)cos(ang);
                sn[(base + p) * n + j] = (float)sin(ang);
            }

    /* the same problem for both sides */
    h3ref_problem rp;
    memset(&rp, 0, sizeof(rp));
    rp.B = B; rp.T = T; rp.H = H; rp.D = D; rp.row_stride = rs; rp.batch_stride = bs;
    memcpy(rp.grid, pc->grid, sizeof(rp.grid));
    rp.pos_offset = off; rp.valid_len = vlen; rp.n = n;
    memcpy(rp.table_len, tl, sizeof(tl));
    rp.cos_tab = cs; rp.sin_tab = sn; rp.eps = 1e-6f;

    uint16_t *d_qkv = (uint16_t *)dev_upload(qkv, (size_t)in_elems * 2);
    float *d_wq = (float *)dev_upload(wq, (size_t)D * 4), *d_wk = (float *)dev_upload(wk, (size_t)D * 4);
    float *d_cs = (float *)dev_upload(cs, (size_t)rows * n * 4 + 4), *d_sn = (float *)dev_upload(sn, (size_t)rows * n * 4 + 4);
    h3_qk_desc desc;
    memset(&desc, 0, sizeof(desc));
    desc.B = B; desc.T = T; desc.H = H; desc.D = D; desc.row_stride = rs; desc.batch_stride = bs;
    memcpy(desc.grid, pc->grid, sizeof(desc.grid));
    for (int b = 0; b < B; ++b) {
        for (int a = 0; a < 3; ++a) desc.pos_offset[b][a] = off[3 * b + a];
        desc.valid_len[b] = vlen[b];
    }
    desc.pairs_per_axis = n;
    memcpy(desc.table_len, tl, sizeof(tl));
    desc.cos_tab = d_cs; desc.sin_tab = d_sn; desc.eps = 1e-6f;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    /* 1. store: Q f32, K bf16, V copy */
    {
        void *q = dev_junk((size_t)out_elems * 4), *k = dev_junk((size_t)out_elems * 2), *v = dev_junk((size_t)out_elems * 2);
        H3_OK_CALL(h3_qk_rmsnorm_rope_permute(&desc, d_qkv, (h3_dtype)pc->in_dt, d_wq, d_wk, q, H3_F32, k, H3_BF16, v, s));
        HIP_OK(hipStreamSynchronize(s));
        float *rq = (float *)malloc((size_t)out_elems * 4);
        uint16_t *rk = (uint16_t *)malloc((size_t)out_elems * 2), *rv = (uint16_t *)malloc((size_t)out_elems * 2);
        if (h3ref_qk_rmsnorm_rope_permute(&rp, qkv, pc->in_dt, wq, wk, rq, H3_F32, rk, H3_BF16, rv)) exit(4);
        expect_same("store Q f32", q, rq, (size_t)out_elems * 4);
        expect_same("store K bf16", k, rk, (size_t)out_elems * 2);
        expect_same("store V copy", v, rv, (size_t)out_elems * 2);
        free(rq); free(rk); free(rv);
        HIP_OK(hipFree(q)); HIP_OK(hipFree(k)); HIP_OK(hipFree(v));
    }
    /* 2. amax, then the cast with those amaxes */
    float ram[2];
    if (h3ref_qk_amax(&rp, qkv, pc->in_dt, wq, wk, ram)) exit(4);
    {
        float *am = (float *)dev_junk(8), *ds = (float *)dev_junk(8);
        H3_OK_CALL(h3_qk_amax(&desc, d_qkv, (h3_dtype)pc->in_dt, d_wq, d_wk, am, s));
        void *q8 = dev_junk((size_t)out_elems), *k8 = dev_junk((size_t)out_elems), *v = dev_junk((size_t)out_elems * 2);
        H3_OK_CALL(h3_qk_cast_e4m3(&desc, d_qkv, (h3_dtype)pc->in_dt, d_wq, d_wk, am, q8, k8, v, ds, s));
        HIP_OK(hipStreamSynchronize(s));
        expect_same("amax", am, ram, 8);
        uint8_t *rq = (uint8_t *)malloc((size_t)out_elems), *rk = (uint8_t *)malloc((size_t)out_elems);
        uint16_t *rv = (uint16_t *)malloc((size_t)out_elems * 2);
        float rds[2];
        if (h3ref_qk_cast_e4m3(&rp, qkv, pc->in_dt, wq, wk, ram, rq, rk, rv, rds)) exit(4);
        expect_same("descale", ds, rds, 8);
        expect_same("Q codes", q8, rq, (size_t)out_elems);
        expect_same("K codes", k8, rk, (size_t)out_elems);
        expect_same("V copy (cast pass)", v, rv, (size_t)out_elems * 2);
        free(rq); free(rk); free(rv);
        HIP_OK(hipFree(am)); HIP_OK(hipFree(ds)); HIP_OK(hipFree(q8)); HIP_OK(hipFree(k8)); HIP_OK(hipFree(v));
    }
    /* 3. static descales at a third of the dynamic ones (a share of every tensor clips), V codes,
       clip counters */
    {
        const float sds[3] = {ram[0] / 448.0f / 3.0f, ram[1] / 448.0f / 3.0f, 3.0f / 448.0f / 3.0f};
        float *d_sds = (float *)dev_upload(sds, 12);
        uint64_t *sat = (uint64_t *)dev_junk((size_t)H3_SAT_WORDS * 8);
        void *q8 = dev_junk((size_t)out_elems), *k8 = dev_junk((size_t)out_elems), *v8 = dev_junk((size_t)out_elems);
        H3_OK_CALL(h3_qk_cast_e4m3_static(&desc, d_qkv, (h3_dtype)pc->in_dt, d_wq, d_wk, d_sds, q8, k8, v8, H3_E4M3FN,
                                          sat, s));
        HIP_OK(hipStreamSynchronize(s));
        uint8_t *rq = (uint8_t *)malloc((size_t)out_elems), *rk = (uint8_t *)malloc((size_t)out_elems),
                *rv = (uint8_t *)malloc((size_t)out_elems);
        uint64_t rsat[3];
        if (h3ref_qk_cast_e4m3_static(&rp, qkv, pc->in_dt, wq, wk, sds, 1, rq, rk, rv, rsat)) exit(4);
        expect_same("static Q codes", q8, rq, (size_t)out_elems);
        expect_same("static K codes", k8, rk, (size_t)out_elems);
        expect_same("static V codes", v8, rv, (size_t)out_elems);
        expect_same("clip counts", sat, rsat, 24);
        printf("  clip counts %llu %llu %llu\n", (unsigned long long)rsat[0], (unsigned long long)rsat[1],
               (unsigned long long)rsat[2]);
        if (!(rsat[0] && rsat[1] && rsat[2])) {
            fprintf(stderr, "MISMATCH static case clips nothing in some tensor\n");
            ++failures;
        }
        free(rq); free(rk); free(rv);
        HIP_OK(hipFree(d_sds)); HIP_OK(hipFree(sat)); HIP_OK(hipFree(q8)); HIP_OK(hipFree(k8)); HIP_OK(hipFree(v8));
    }
    /* 4. a rejected call enqueues nothing and reports why */
    {
        h3_qk_desc bad = desc;
        bad.D = 96;
        float *am = (float *)dev_junk(8);
        const int r = h3_qk_amax(&bad, d_qkv, (h3_dtype)pc->in_dt, d_wq, d_wk, am, s);
        if (r != H3_EUNSUPPORTED || strstr(h3_last_error(), "D") == NULL) {
            fprintf(stderr, "MISMATCH rejected call returned %d (%s)\n", r, h3_last_error());
            ++failures;
        } else {
            printf("ok rejected call: %s\n", h3_last_error());
        }
        HIP_OK(hipFree(am));
    }
    HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipFree(d_qkv)); HIP_OK(hipFree(d_wq)); HIP_OK(hipFree(d_wk)); HIP_OK(hipFree(d_cs)); HIP_OK(hipFree(d_sn));
    free(qkv); free(wq); free(wk); free(cs); free(sn);
}

int main(void) {
    if (h3_abi_version() != H3_ABI_VERSION) {
        fprintf(stderr, "ABI version %d, header %d\n", h3_abi_version(), H3_ABI_VERSION);
        return 5;
    }
    sm_state = 20261202ull;
    const problem_case cases[] = {
        {"D64 f16, two items, offsets, padded strides", 2, 45, 3, 64, 8, H3_F16, {3, 4, 4}, {45, 17},
         {{0, 0, 0}, {1, 2, 3}}, 8, 16},
        {"D128 bf16, one item, padding tail", 1, 37, 2, 128, 16, H3_BF16, {1, 5, 8}, {33, 0}, {{0, 0, 0}, {0, 0, 0}},
         0, 0},
        {"D64 f16, five heads, generic rotary split", 2, 20, 5, 64, 5, H3_F16, {2, 2, 5}, {20, 0},
         {{0, 1, 0}, {0, 0, 2}}, 24, 8},
    };
    for (size_t c = 0; c < sizeof(cases) / sizeof(cases[0]); ++c) run_case(&cases[c]);
    if (failures) {
        fprintf(stderr, "%d comparisons failed\n", failures);
        return 1;
    }
    printf("all outputs bit-identical to the oracle\n");
    return 0;
}
