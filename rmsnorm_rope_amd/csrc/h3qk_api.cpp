// C ABI of libh3qk: host-side validation of every argument, then one launch on the caller's
// stream.  A call that fails validation enqueues nothing.  See include/h3qk.h for the contract.
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <initializer_list>
#include <string>

#include "h3qk.h"
#include "h3qk_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
    g_err = msg;
    return code;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    const char *name;
};

// The address ranges of one call's inputs or outputs, held in place: validation of a call that
// succeeds allocates no memory.  A call has at most 6 inputs and 5 outputs; a list that would hold
// more than its capacity records that, and the overlap checks then fail the call (check_outputs).
class RangeList {
  public:
    RangeList() = default;
    RangeList(std::initializer_list<Range> l) {
        for (const Range &r : l) push_back(r);
    }
    void push_back(const Range &r) {
        if (n_ < kCap) r_[n_++] = r;
        else overflow_ = true;
    }
    bool overflow() const { return overflow_; }
    size_t size() const { return (size_t)n_; }
    const Range &operator[](size_t i) const { return r_[i]; }
    const Range *begin() const { return r_; }
    const Range *end() const { return r_ + n_; }

  private:
    static constexpr int kCap = 8;
    Range r_[kCap];
    int n_ = 0;
    bool overflow_ = false;
};

bool overlaps(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }

int elem_size(int dt) { return dt == H3_F32 ? 4 : (dt == H3_E4M3FN ? 1 : 2); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate the descriptor and the input pointers shared by the QK calls (tensors = 3: a fused
// Q | K | V row) and the one-tensor calls (tensors = 1: w_q is the tensor's weight, NULL for the
// identity; w_k unused); fill the kernel parameters.  Returns H3_OK or an error code with g_err set.
int check_desc(const h3_qk_desc *d, const void *qkv, int in_dt, const float *w_q, const float *w_k,
               h3::QkParams *p, RangeList *inputs, int tensors = 3) {
    if (!d) return fail(H3_EINVAL, "desc is NULL");
    if (tensors == 3 && (!qkv || !w_q || !w_k)) return fail(H3_EINVAL, "qkv, w_q and w_k must be non-NULL");
    if (tensors == 1 && !qkv) return fail(H3_EINVAL, "x must be non-NULL");
    if (d->pairs_per_axis > 0 && (!d->cos_tab || !d->sin_tab))
        return fail(H3_EINVAL, "cos_tab and sin_tab must be non-NULL when pairs_per_axis > 0");
    if (d->B < 1 || d->B > H3_MAX_BATCH) return fail(H3_EINVAL, "B must be in 1..H3_MAX_BATCH");
    if (d->T < 1 || d->H < 1) return fail(H3_EINVAL, "T and H must be >= 1");
    if (d->D != 64 && d->D != 128) return fail(H3_EUNSUPPORTED, "head dim D must be 64 or 128");
    if (in_dt != H3_F16 && in_dt != H3_BF16) return fail(H3_EUNSUPPORTED, "input dtype must be H3_F16 or H3_BF16");
    const int64_t B = d->B, T = d->T, H = d->H, D = d->D;
    if (d->pairs_per_axis < 0 || 6 * (int64_t)d->pairs_per_axis > D)
        return fail(H3_EUNSUPPORTED, "pairs_per_axis n must satisfy 0 <= 6n <= D");
    if (!std::isfinite(d->eps) || d->eps < 0.0f) return fail(H3_EINVAL, "eps must be finite and >= 0");
    if (d->row_stride < tensors * H * D)
        return fail(H3_EINVAL, tensors == 3 ? "row_stride must be >= 3*H*D" : "row_stride must be >= H*D");
    if (d->row_stride > ((int64_t)1 << 26)) return fail(H3_EINVAL, "row_stride must be <= 2^26 elements");
    if (B > 1 && d->batch_stride < T * d->row_stride) return fail(H3_EINVAL, "batch_stride must be >= T*row_stride");
    if (d->batch_stride < 0) return fail(H3_EINVAL, "batch_stride must be >= 0");
    if ((d->row_stride & 7) || (d->batch_stride & 7))
        return fail(H3_EALIGN, "row_stride and batch_stride must be multiples of 8 elements (16 bytes)");
    if (!aligned16(qkv) || !aligned16(w_q) || (tensors == 3 && !aligned16(w_k)))
        return fail(H3_EALIGN, tensors == 3 ? "qkv, w_q and w_k must be 16-byte aligned" : "x and w must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(d->cos_tab) & 3u) || (reinterpret_cast<uintptr_t>(d->sin_tab) & 3u))
        return fail(H3_EALIGN, "cos_tab and sin_tab must be 4-byte aligned");
    for (int a = 0; a < 3; ++a) {
        if (d->grid[a] < 1) return fail(H3_EINVAL, "grid extents must be >= 1");
        if (d->table_len[a] < 1) return fail(H3_EINVAL, "table_len entries must be >= 1");
    }
    const int64_t gsize = (int64_t)d->grid[0] * d->grid[1] * d->grid[2];
    const int64_t vmax = gsize < T ? gsize : T;
    for (int b = 0; b < d->B; ++b) {
        if (d->valid_len[b] < 0 || d->valid_len[b] > vmax)
            return fail(H3_ERANGE, "valid_len[" + std::to_string(b) + "] must be in 0..min(T, Gt*Gh*Gw)");
        for (int a = 0; a < 3; ++a) {
            const int64_t off = d->pos_offset[b][a];
            if (off < 0 || off + d->grid[a] > d->table_len[a])
                return fail(H3_ERANGE, "pos_offset[" + std::to_string(b) + "][" + std::to_string(a) +
                                           "] + grid extent exceeds table_len");
        }
    }
    const int64_t rows_total = (int64_t)d->table_len[0] + d->table_len[1] + d->table_len[2];
    if (rows_total * (int64_t)d->pairs_per_axis > ((int64_t)1 << 30) || T * H * D > ((int64_t)1 << 40))
        return fail(H3_EINVAL, "problem too large");

    const uintptr_t q0 = reinterpret_cast<uintptr_t>(qkv);
    const int64_t qkv_elems = (B - 1) * d->batch_stride + (T - 1) * d->row_stride + tensors * H * D;
    inputs->push_back({q0, q0 + (uintptr_t)qkv_elems * 2, tensors == 3 ? "qkv" : "x"});
    if (w_q)
        inputs->push_back({reinterpret_cast<uintptr_t>(w_q), reinterpret_cast<uintptr_t>(w_q) + (uintptr_t)D * 4,
                           tensors == 3 ? "w_q" : "w"});
    if (tensors == 3)
        inputs->push_back({reinterpret_cast<uintptr_t>(w_k), reinterpret_cast<uintptr_t>(w_k) + (uintptr_t)D * 4, "w_k"});
    const uintptr_t tab_bytes = (uintptr_t)(rows_total * d->pairs_per_axis) * 4;
    inputs->push_back({reinterpret_cast<uintptr_t>(d->cos_tab), reinterpret_cast<uintptr_t>(d->cos_tab) + tab_bytes, "cos_tab"});
    inputs->push_back({reinterpret_cast<uintptr_t>(d->sin_tab), reinterpret_cast<uintptr_t>(d->sin_tab) + tab_bytes, "sin_tab"});

    memset(p, 0, sizeof(*p));
    p->qkv = static_cast<const uint16_t *>(qkv);
    p->wq = w_q;
    p->wk = w_k;
    p->cos_tab = d->cos_tab;
    p->sin_tab = d->sin_tab;
    p->row_stride = d->row_stride;
    p->batch_stride = d->batch_stride;
    p->B = d->B;
    p->T = d->T;
    p->H = d->H;
    p->n = d->pairs_per_axis;
    p->Gh = d->grid[1];
    p->Gw = d->grid[2];
    p->base_h = d->table_len[0];
    p->base_w = d->table_len[0] + d->table_len[1];
    p->eps = d->eps;
    for (int b = 0; b < d->B; ++b) {
        for (int a = 0; a < 3; ++a) p->off[b][a] = d->pos_offset[b][a];
        p->vlen[b] = d->valid_len[b];
    }
    // Work items: 8 consecutive tokens x kHeadsPerWave (fused) or kTensorHeads heads, one wave each.
    const int hpw = tensors == 3 ? h3::kHeadsPerWave : h3::kTensorHeads;
    p->groups = (int32_t)((T + 7) / 8);
    p->head_chunks = (int32_t)((H + hpw - 1) / hpw);
    p->items = B * p->groups * p->head_chunks;
    if (p->items > INT32_MAX) return fail(H3_EINVAL, "problem too large");
    p->div_gw = h3::div_magic((uint32_t)d->grid[2]);
    p->div_gh = h3::div_magic((uint32_t)d->grid[1]);
    p->inv_n = d->pairs_per_axis > 0 ? 1.0f / (float)d->pairs_per_axis : 0.0f;
    p->tab_pairs = ((reinterpret_cast<uintptr_t>(d->cos_tab) | reinterpret_cast<uintptr_t>(d->sin_tab)) & 7u) == 0;
    return H3_OK;
}

int check_outputs(const RangeList &inputs, const RangeList &outputs) {
    if (inputs.overflow() || outputs.overflow()) return fail(H3_EINVAL, "internal: too many buffers to check for overlap");
    for (size_t i = 0; i < outputs.size(); ++i) {
        if (!aligned16(reinterpret_cast<const void *>(outputs[i].lo)))
            return fail(H3_EALIGN, std::string(outputs[i].name) + " must be 16-byte aligned");
        for (const Range &in : inputs)
            if (overlaps(outputs[i], in))
                return fail(H3_EALIAS, std::string(outputs[i].name) + " overlaps input " + in.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outputs[i], outputs[j]))
                return fail(H3_EALIAS, std::string(outputs[i].name) + " overlaps output " + outputs[j].name);
    }
    return H3_OK;
}

Range out_range(const void *p, int64_t n, int dt, const char *name) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + (uintptr_t)n * elem_size(dt), name};
}

int run(int mode, int D, int in_dt, int q_dt, int k_dt, h3::QkParams &p, hipStream_t stream) {
    std::string err;
    const int rc = h3::launch_qk(mode, D, in_dt, q_dt, k_dt, p, stream, &err);
    if (rc != H3_OK) return fail(rc, err);
    g_err.clear();
    return H3_OK;
}

}  // namespace

extern "C" {

int h3_qk_rmsnorm_rope_permute(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt,
                               const float *w_q, const float *w_k, void *q_out, h3_dtype q_dt,
                               void *k_out, h3_dtype k_dt, void *v_out, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!q_out || !k_out || !v_out) return fail(H3_EINVAL, "q_out, k_out and v_out must be non-NULL");
    if (q_dt != H3_F32 && q_dt != H3_F16 && q_dt != H3_BF16)
        return fail(H3_EUNSUPPORTED, "q_dt must be H3_F32, H3_F16 or H3_BF16");
    if (k_dt != H3_F32 && k_dt != H3_F16 && k_dt != H3_BF16)
        return fail(H3_EUNSUPPORTED, "k_dt must be H3_F32, H3_F16 or H3_BF16");
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    rc = check_outputs(inputs, {out_range(q_out, n, q_dt, "q_out"), out_range(k_out, n, k_dt, "k_out"),
                                out_range(v_out, n, in_dt, "v_out")});
    if (rc) return rc;
    p.q = q_out;
    p.k = k_out;
    p.v = v_out;
    return run(h3::MODE_STORE, desc->D, in_dt, q_dt, k_dt, p, stream);
}

int h3_qk_rmsnorm_rope_permute_sage(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                                    const float *w_k, float kv_scale, float *q_out, float *k_out, uint16_t *v_out,
                                    hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!q_out || !k_out || !v_out) return fail(H3_EINVAL, "q_out, k_out and v_out must be non-NULL");
    if (!std::isfinite(kv_scale)) return fail(H3_EINVAL, "kv_scale must be finite");
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    rc = check_outputs(inputs, {out_range(q_out, n, H3_F32, "q_out"), out_range(k_out, n, H3_F32, "k_out"),
                                out_range(v_out, n, H3_F16, "v_out")});
    if (rc) return rc;
    p.q = q_out;
    p.k = k_out;
    p.v = v_out;
    p.sage = 1;
    p.kv_scale = kv_scale;
    return run(h3::MODE_STORE, desc->D, in_dt, H3_F32, H3_F32, p, stream);
}

int h3_qk_amax(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
               const float *w_k, float *amax_qk, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!amax_qk) return fail(H3_EINVAL, "amax_qk must be non-NULL");
    if (reinterpret_cast<uintptr_t>(amax_qk) & 7u) return fail(H3_EALIGN, "amax_qk must be 8-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(amax_qk);
    for (const Range &in : inputs)
        if (overlaps({a, a + 8, "amax_qk"}, in)) return fail(H3_EALIAS, std::string("amax_qk overlaps input ") + in.name);
    p.amax = amax_qk;
    return run(h3::MODE_AMAX, desc->D, in_dt, H3_E4M3FN, H3_E4M3FN, p, stream);
}

int h3_qk_cast_e4m3(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                    const float *w_k, const float *amax_qk, uint8_t *q_codes, uint8_t *k_codes,
                    void *v_out, float *descale_qk, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!amax_qk || !q_codes || !k_codes || !v_out || !descale_qk)
        return fail(H3_EINVAL, "amax_qk, q_codes, k_codes, v_out and descale_qk must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(amax_qk) & 7u) || (reinterpret_cast<uintptr_t>(descale_qk) & 7u))
        return fail(H3_EALIGN, "amax_qk and descale_qk must be 8-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(amax_qk);
    inputs.push_back({a, a + 8, "amax_qk"});
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    const uintptr_t ds = reinterpret_cast<uintptr_t>(descale_qk);
    RangeList outs = {out_range(q_codes, n, H3_E4M3FN, "q_codes"), out_range(k_codes, n, H3_E4M3FN, "k_codes"),
                               out_range(v_out, n, in_dt, "v_out")};
    rc = check_outputs(inputs, outs);
    if (rc) return rc;
    const Range dr = {ds, ds + 8, "descale_qk"};
    for (const Range &r : inputs)
        if (overlaps(dr, r)) return fail(H3_EALIAS, std::string("descale_qk overlaps input ") + r.name);
    for (const Range &r : outs)
        if (overlaps(dr, r)) return fail(H3_EALIAS, std::string("descale_qk overlaps output ") + r.name);
    p.amax = const_cast<float *>(amax_qk);
    p.q = q_codes;
    p.k = k_codes;
    p.v = v_out;
    p.descale = descale_qk;
    return run(h3::MODE_CAST, desc->D, in_dt, H3_E4M3FN, H3_E4M3FN, p, stream);
}

}  // extern "C"

namespace {

// The static-scale cast with the clip counts written to `sat` (sat_words words, the counts in the
// first three) and the partial counts kept in `slots` (H3_SAT_SLOTS slots of 16 words): the
// caller's counter buffer for both (slots from its word 16 on), or the caller's three words and
// the library's static scratch.  sat == NULL: no counting.
int cast_static(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q, const float *w_k,
                const float *descale_qkv, uint8_t *q_codes, uint8_t *k_codes, void *v_out, h3_dtype v_dt,
                uint64_t *sat, int sat_words, const char *sat_name, bool own_slots, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!descale_qkv || !q_codes || !k_codes || !v_out)
        return fail(H3_EINVAL, "descale_qkv, q_codes, k_codes and v_out must be non-NULL");
    if (v_dt != in_dt && v_dt != H3_E4M3FN) return fail(H3_EUNSUPPORTED, "v_dt must be in_dt or H3_E4M3FN");
    const bool v_fp8 = v_dt == H3_E4M3FN;
    if (reinterpret_cast<uintptr_t>(descale_qkv) & 3u) return fail(H3_EALIGN, "descale_qkv must be 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(sat) & 7u) return fail(H3_EALIGN, std::string(sat_name) + " must be 8-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(descale_qkv);
    inputs.push_back({a, a + (v_fp8 ? 12u : 8u), "descale_qkv"});
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    RangeList outs = {out_range(q_codes, n, H3_E4M3FN, "q_codes"), out_range(k_codes, n, H3_E4M3FN, "k_codes"),
                      out_range(v_out, n, v_dt, "v_out")};
    rc = check_outputs(inputs, outs);
    if (rc) return rc;
    if (sat) {
        const uintptr_t sp = reinterpret_cast<uintptr_t>(sat);
        const Range sr = {sp, sp + (uintptr_t)sat_words * 8, sat_name};
        for (const Range &r : inputs)
            if (overlaps(sr, r)) return fail(H3_EALIAS, std::string(sat_name) + " overlaps input " + r.name);
        for (const Range &r : outs)
            if (overlaps(sr, r)) return fail(H3_EALIAS, std::string(sat_name) + " overlaps output " + r.name);
        p.sat = reinterpret_cast<unsigned long long *>(sat);
        if (own_slots) {
            p.sat_slots = p.sat + 16;
        } else {
            std::string err;
            if (!h3::scratch_slots(&p.sat_slots, &err)) return fail(H3_ELAUNCH, err);
        }
    }
    p.amax = const_cast<float *>(descale_qkv);
    p.static_scale = 1;
    p.v_fp8 = v_fp8 ? 1 : 0;
    p.q = q_codes;
    p.k = k_codes;
    p.v = v_out;
    return run(h3::MODE_CAST, desc->D, in_dt, H3_E4M3FN, H3_E4M3FN, p, stream);
}

}  // namespace

extern "C" {

int h3_qk_cast_e4m3_static(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                           const float *w_k, const float *descale_qkv, uint8_t *q_codes, uint8_t *k_codes,
                           void *v_out, h3_dtype v_dt, uint64_t *sat_qkv, hipStream_t stream) {
    return cast_static(desc, qkv, in_dt, w_q, w_k, descale_qkv, q_codes, k_codes, v_out, v_dt, sat_qkv, H3_SAT_WORDS,
                       "sat_qkv", true, stream);
}

int h3_qk_cast_e4m3_static_noalloc(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                                   const float *w_k, const float *descale_qkv, uint8_t *q_codes, uint8_t *k_codes,
                                   void *v_out, h3_dtype v_dt, uint64_t *sat_counts, hipStream_t stream) {
    return cast_static(desc, qkv, in_dt, w_q, w_k, descale_qkv, q_codes, k_codes, v_out, v_dt, sat_counts, 3,
                       "sat_counts", false, stream);
}

int h3_qkv_amax(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                const float *w_k, float *amax_qkv, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!amax_qkv) return fail(H3_EINVAL, "amax_qkv must be non-NULL");
    if (reinterpret_cast<uintptr_t>(amax_qkv) & 3u) return fail(H3_EALIGN, "amax_qkv must be 4-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(amax_qkv);
    for (const Range &in : inputs)
        if (overlaps({a, a + 12, "amax_qkv"}, in)) return fail(H3_EALIAS, std::string("amax_qkv overlaps input ") + in.name);
    p.amax = amax_qkv;
    p.v_fp8 = 1;
    return run(h3::MODE_AMAX, desc->D, in_dt, H3_E4M3FN, H3_E4M3FN, p, stream);
}

int h3_qkv_cast_e4m3(const h3_qk_desc *desc, const void *qkv, h3_dtype in_dt, const float *w_q,
                     const float *w_k, const float *amax_qkv, uint8_t *q_codes, uint8_t *k_codes,
                     uint8_t *v_codes, float *descale_qkv, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, qkv, in_dt, w_q, w_k, &p, &inputs);
    if (rc) return rc;
    if (!amax_qkv || !q_codes || !k_codes || !v_codes || !descale_qkv)
        return fail(H3_EINVAL, "amax_qkv, q_codes, k_codes, v_codes and descale_qkv must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(amax_qkv) & 3u) || (reinterpret_cast<uintptr_t>(descale_qkv) & 3u))
        return fail(H3_EALIGN, "amax_qkv and descale_qkv must be 4-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(amax_qkv);
    inputs.push_back({a, a + 12, "amax_qkv"});
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    RangeList outs = {out_range(q_codes, n, H3_E4M3FN, "q_codes"), out_range(k_codes, n, H3_E4M3FN, "k_codes"),
                               out_range(v_codes, n, H3_E4M3FN, "v_codes")};
    rc = check_outputs(inputs, outs);
    if (rc) return rc;
    const uintptr_t ds = reinterpret_cast<uintptr_t>(descale_qkv);
    const Range dr = {ds, ds + 12, "descale_qkv"};
    for (const Range &r : inputs)
        if (overlaps(dr, r)) return fail(H3_EALIAS, std::string("descale_qkv overlaps input ") + r.name);
    for (const Range &r : outs)
        if (overlaps(dr, r)) return fail(H3_EALIAS, std::string("descale_qkv overlaps output ") + r.name);
    p.amax = const_cast<float *>(amax_qkv);
    p.v_fp8 = 1;
    p.q = q_codes;
    p.k = k_codes;
    p.v = v_codes;
    p.descale = descale_qkv;
    return run(h3::MODE_CAST, desc->D, in_dt, H3_E4M3FN, H3_E4M3FN, p, stream);
}

namespace {

// Output strides of one tensor: [B, H, T, D] or [B, T, H, D].
int tensor_layout(const h3_qk_desc *d, int layout, h3::QkParams *p) {
    if (layout == H3_LAYOUT_BHTD) {
        p->out_hstride = (int64_t)d->T * d->D;
        p->out_tstride = d->D;
    } else if (layout == H3_LAYOUT_BTHD) {
        p->out_hstride = d->D;
        p->out_tstride = (int64_t)d->H * d->D;
    } else {
        return fail(H3_EUNSUPPORTED, "out_layout must be H3_LAYOUT_BHTD or H3_LAYOUT_BTHD");
    }
    return H3_OK;
}

int run_tensor(int mode, int D, int in_dt, int out_dt, bool norm, h3::QkParams &p, hipStream_t stream) {
    std::string err;
    const int rc = h3::launch_tensor(mode, D, in_dt, out_dt, norm, p, stream, &err);
    if (rc != H3_OK) return fail(rc, err);
    g_err.clear();
    return H3_OK;
}

}  // namespace

int h3_tensor_norm_rope(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w, void *out,
                        h3_dtype out_dt, h3_layout out_layout, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, x, in_dt, w, nullptr, &p, &inputs, 1);
    if (rc) return rc;
    if (!out) return fail(H3_EINVAL, "out must be non-NULL");
    if (out_dt != H3_F32 && out_dt != H3_F16 && out_dt != H3_BF16)
        return fail(H3_EUNSUPPORTED, "out_dt must be H3_F32, H3_F16 or H3_BF16");
    rc = tensor_layout(desc, out_layout, &p);
    if (rc) return rc;
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    rc = check_outputs(inputs, {out_range(out, n, out_dt, "out")});
    if (rc) return rc;
    p.wq = w;
    p.q = out;
    return run_tensor(h3::MODE_STORE, desc->D, in_dt, out_dt, w != nullptr, p, stream);
}

int h3_tensor_amax(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w, float *amax,
                   hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, x, in_dt, w, nullptr, &p, &inputs, 1);
    if (rc) return rc;
    if (!amax) return fail(H3_EINVAL, "amax must be non-NULL");
    if (reinterpret_cast<uintptr_t>(amax) & 3u) return fail(H3_EALIGN, "amax must be 4-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(amax);
    for (const Range &in : inputs)
        if (overlaps({a, a + 4, "amax"}, in)) return fail(H3_EALIAS, std::string("amax overlaps input ") + in.name);
    p.wq = w;
    p.amax = amax;
    return run_tensor(h3::MODE_AMAX, desc->D, in_dt, H3_E4M3FN, w != nullptr, p, stream);
}

int h3_tensor_cast_e4m3(const h3_qk_desc *desc, const void *x, h3_dtype in_dt, const float *w,
                        const float *scale, int scale_is_descale, uint8_t *codes, h3_layout out_layout,
                        float *descale, uint64_t *sat, hipStream_t stream) {
    h3::QkParams p;
    RangeList inputs;
    int rc = check_desc(desc, x, in_dt, w, nullptr, &p, &inputs, 1);
    if (rc) return rc;
    if (!scale || !codes) return fail(H3_EINVAL, "scale and codes must be non-NULL");
    if (scale_is_descale != 0 && scale_is_descale != 1) return fail(H3_EINVAL, "scale_is_descale must be 0 or 1");
    if ((reinterpret_cast<uintptr_t>(scale) & 3u) || (reinterpret_cast<uintptr_t>(descale) & 3u))
        return fail(H3_EALIGN, "scale and descale must be 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(sat) & 7u) return fail(H3_EALIGN, "sat must be 8-byte aligned");
    rc = tensor_layout(desc, out_layout, &p);
    if (rc) return rc;
    const uintptr_t a = reinterpret_cast<uintptr_t>(scale);
    inputs.push_back({a, a + 4, "scale"});
    const int64_t n = (int64_t)desc->B * desc->H * desc->T * desc->D;
    RangeList outs = {out_range(codes, n, H3_E4M3FN, "codes")};
    rc = check_outputs(inputs, outs);
    if (rc) return rc;
    if (descale) {
        const uintptr_t d = reinterpret_cast<uintptr_t>(descale);
        outs.push_back({d, d + 4, "descale"});
    }
    if (sat) {
        const uintptr_t sp = reinterpret_cast<uintptr_t>(sat);
        outs.push_back({sp, sp + (uintptr_t)H3_SAT_WORDS * 8, "sat"});
    }
    for (size_t i = 1; i < outs.size(); ++i) {
        for (const Range &r : inputs)
            if (overlaps(outs[i], r)) return fail(H3_EALIAS, std::string(outs[i].name) + " overlaps input " + r.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(H3_EALIAS, std::string(outs[i].name) + " overlaps output " + outs[j].name);
    }
    p.wq = w;
    p.amax = const_cast<float *>(scale);
    p.static_scale = scale_is_descale;
    p.descale = descale;
    p.sat = reinterpret_cast<unsigned long long *>(sat);
    p.sat_slots = sat ? p.sat + 16 : nullptr;
    p.q = codes;
    return run_tensor(h3::MODE_CAST, desc->D, in_dt, H3_E4M3FN, w != nullptr, p, stream);
}

int h3_swiglu(const void *x, h3_dtype dt, void *y, int64_t N, int64_t F, hipStream_t stream) {
    if (!x || !y) return fail(H3_EINVAL, "x and y must be non-NULL");
    if (dt != H3_F16 && dt != H3_BF16) return fail(H3_EUNSUPPORTED, "dt must be H3_F16 or H3_BF16");
    if (N < 1 || F < 1) return fail(H3_EINVAL, "N and F must be >= 1");
    if (F % 8) return fail(H3_EUNSUPPORTED, "F must be a multiple of 8");
    if (N * F / 8 >= ((int64_t)1 << 32) || F > ((int64_t)1 << 30)) return fail(H3_EINVAL, "problem too large");
    if (!aligned16(x) || !aligned16(y)) return fail(H3_EALIGN, "x and y must be 16-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), o = reinterpret_cast<uintptr_t>(y);
    if (overlaps({o, o + (uintptr_t)(N * F * 2), "y"}, {a, a + (uintptr_t)(N * F * 4), "x"}))
        return fail(H3_EALIAS, "y overlaps x");
    std::string err;
    const int rc = h3::launch_swiglu(dt, x, y, N, F, stream, &err);
    if (rc != H3_OK) return fail(rc, err);
    g_err.clear();
    return H3_OK;
}

int h3_scaled_residual(const float *res, const void *branch, h3_dtype branch_dt, const float *scale,
                       int64_t scale_len, float *out, int64_t N, int64_t C, hipStream_t stream) {
    if (!res || !branch || !scale || !out) return fail(H3_EINVAL, "res, branch, scale and out must be non-NULL");
    if (branch_dt != H3_F16 && branch_dt != H3_BF16) return fail(H3_EUNSUPPORTED, "branch_dt must be H3_F16 or H3_BF16");
    if (N < 1 || C < 1) return fail(H3_EINVAL, "N and C must be >= 1");
    if (C % 4) return fail(H3_EUNSUPPORTED, "C must be a multiple of 4");
    if (scale_len != 1 && scale_len != C) return fail(H3_EINVAL, "scale_len must be 1 or C");
    if (N * C / 4 >= ((int64_t)1 << 32) || C > ((int64_t)1 << 30)) return fail(H3_EINVAL, "problem too large");
    if (!aligned16(res) || !aligned16(out) || (scale_len != 1 && !aligned16(scale)) ||
        (reinterpret_cast<uintptr_t>(branch) & 7u) || (reinterpret_cast<uintptr_t>(scale) & 3u))
        return fail(H3_EALIGN, "res, out (and a per-channel scale) must be 16-byte aligned, branch 8-byte");
    const uintptr_t o = reinterpret_cast<uintptr_t>(out);
    const Range ro = {o, o + (uintptr_t)(N * C * 4), "out"};
    const uintptr_t r = reinterpret_cast<uintptr_t>(res), b = reinterpret_cast<uintptr_t>(branch);
    const uintptr_t sc = reinterpret_cast<uintptr_t>(scale);
    const Range ins[] = {{r, r + (uintptr_t)(N * C * 4), "res"}, {b, b + (uintptr_t)(N * C * 2), "branch"},
                         {sc, sc + (uintptr_t)(scale_len * 4), "scale"}};
    for (const Range &in : ins)
        if (overlaps(ro, in)) return fail(H3_EALIAS, std::string("out overlaps ") + in.name);
    std::string err;
    const int rc = h3::launch_scaled_residual(branch_dt, res, branch, scale, scale_len, out, N, C, stream, &err);
    if (rc != H3_OK) return fail(rc, err);
    g_err.clear();
    return H3_OK;
}

const char *h3_last_error(void) { return g_err.c_str(); }

int h3_abi_version(void) { return H3_ABI_VERSION; }

}  // extern "C"
