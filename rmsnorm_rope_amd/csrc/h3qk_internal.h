// Internal launch interface between the host-side validation (h3qk_api.cpp) and the gfx950
// kernels (h3qk_kernels.hip).  Not installed; the public interface is include/h3qk.h.
#pragma once

#include <stdint.h>
#include <string>

#include "h3qk.h"

namespace h3 {

enum Mode : int { MODE_STORE = 0, MODE_AMAX = 1, MODE_CAST = 2 };

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
    float *amax;        // MODE_AMAX: reduced into (cleared first); MODE_CAST: read
    float *descale;     // MODE_CAST: written by the first wave
    int64_t row_stride;
    int64_t batch_stride;
    int32_t B, T, H, n;
    int32_t Gh, Gw;
    int32_t base_h, base_w;      // first table row of the h and w parts
    int32_t groups;              // token groups of 8 per item: ceil(T / 8)
    int32_t head_chunks;         // work items per token group (heads split across waves)
    int32_t heads_per_chunk;
    int32_t pad_;
    int64_t items;               // B * groups * head_chunks
    float eps;
    int32_t off[H3_MAX_BATCH][3];
    int32_t vlen[H3_MAX_BATCH];
};

// Launch one QK pass.  Returns H3_OK or H3_ELAUNCH / H3_EUNSUPPORTED with *err filled.
int launch_qk(int mode, int D, int in_dt, int q_dt, int k_dt, QkParams &p, hipStream_t stream,
              std::string *err);

}  // namespace h3
