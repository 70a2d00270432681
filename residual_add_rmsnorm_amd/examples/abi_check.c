/*
 * A C client of libfusednorm that needs no GPU: it includes the public header
 * as C (not C++), links the library, and makes only calls that return before
 * any HIP work (an empty batch and rejected arguments), printing the status
 * and detail of each.
 *
 *   cc -std=c11 -I include residual_add_rmsnorm_amd/examples/abi_check.c \
 *      -L residual_add_rmsnorm_amd -lfusednorm -Wl,-rpath,<dir of the library>
 */
#include <stdio.h>

#include "fusednorm.h"

static int expect(const char* what, int got, int want) {
    printf("%-40s %-18s %s\n", what, fusednorm_status_string(got), fusednorm_last_error());
    return got == want ? 0 : 1;
}

int main(void) {
    int bad = 0;
    const void* parts[2] = {0, 0};
    if (fusednorm_version() != FUSEDNORM_VERSION) {
        printf("library version %d, header %d\n", fusednorm_version(), FUSEDNORM_VERSION);
        return 1;
    }
    bad |= expect("empty batch", fused_add_rmsnorm(parts, 2, 0, 0, 0, 1024, 1e-6f, 0, 0, 0),
                  FUSEDNORM_OK);
    bad |= expect("P = 0", fused_add_rmsnorm(parts, 0, 0, 0, 4, 1024, 1e-6f, 0, 0, 0),
                  FUSEDNORM_ERR_INVALID_ARGUMENT);
    bad |= expect("H not a multiple of 8",
                  fused_add_rmsnorm(parts, 2, 0, 0, 4, 1001, 1e-6f, 0, 0, 0),
                  FUSEDNORM_ERR_UNSUPPORTED);
    bad |= expect("NULL partial", fused_add_rmsnorm(parts, 2, 0, 0, 4, 1024, 1e-6f, 0, 0, 0),
                  FUSEDNORM_ERR_INVALID_ARGUMENT);
    bad |= expect("block FP8 group 64",
                  fused_add_rmsnorm_quant_fp8_block(parts, 2, 0, 0, 4, 1024, 1e-6f, 64, 0, 0, 0, 0,
                                                    0),
                  FUSEDNORM_ERR_UNSUPPORTED);
    bad |= expect("QK mode B without var_in",
                  qk_rmsnorm(0, 4, 8192, 6144, 1024, 0, 0, 1e-6f, 4, 0, 0, 0, 0),
                  FUSEDNORM_ERR_INVALID_ARGUMENT);
    bad |= expect("reduce-scatter pattern 3 (FP4)",
                  fused_rs_epilogue(3, parts, 2, 0, 0, 0, 0, 4, 1024, 1e-6f, 0, 0, 0, 0, 0, 0),
                  FUSEDNORM_ERR_UNSUPPORTED);
    bad |= expect("all-gather pattern 2, q_lora_rank 1000",
                  ag_dual_rmsnorm(2, 0, 4, 2112, 1000, 512, 0, 0, 1e-6f, 1e-6f, 0, 0, 0, 0, 0),
                  FUSEDNORM_ERR_UNSUPPORTED);
    printf(bad ? "FAILED\n" : "ok\n");
    return bad;
}
