/* A C99 caller of libh3qk: include/h3qk.h must compile as C and every entry point must link.
   No GPU: each call below fails host validation, so nothing reaches the HIP runtime. */
#include <stdio.h>
#include <string.h>

#include "h3qk.h"

int main(void) {
    h3_qk_desc d;
    memset(&d, 0, sizeof d);
    int fails = 0;
    int rc = h3_qk_rmsnorm_rope_permute(&d, 0, H3_F16, 0, 0, 0, H3_F32, 0, H3_F16, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qk_amax(0, 0, H3_BF16, 0, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qk_cast_e4m3(0, 0, H3_BF16, 0, 0, 0, 0, 0, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qk_cast_e4m3_static(0, 0, H3_BF16, 0, 0, 0, 0, 0, 0, H3_E4M3FN, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qk_cast_e4m3_static_noalloc(0, 0, H3_BF16, 0, 0, 0, 0, 0, 0, H3_E4M3FN, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qk_rmsnorm_rope_permute_sage(0, 0, H3_F16, 0, 0, 0.125f, 0, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qkv_amax(0, 0, H3_BF16, 0, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_qkv_cast_e4m3(0, 0, H3_BF16, 0, 0, 0, 0, 0, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_tensor_norm_rope(0, 0, H3_F16, 0, 0, H3_F16, H3_LAYOUT_BTHD, 0);
    fails += rc != H3_EINVAL;
    rc = h3_tensor_amax(0, 0, H3_F16, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_tensor_cast_e4m3(0, 0, H3_F16, 0, 0, 0, 0, H3_LAYOUT_BHTD, 0, 0, 0);
    fails += rc != H3_EINVAL;
    rc = h3_swiglu(0, H3_F16, 0, 1, 8, 0);
    fails += rc != H3_EINVAL;
    rc = h3_scaled_residual(0, 0, H3_F16, 0, 1, 0, 1, 4, 0);
    fails += rc != H3_EINVAL;
    fails += h3_abi_version() != H3_ABI_VERSION;
    fails += h3_last_error() == 0;
    printf("abi_check: %d failure(s); last error: %s\n", fails, h3_last_error());
    return fails != 0;
}
