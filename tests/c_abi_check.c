/* Plain C client of include/gdr.h: compiles the header as C and calls the
 * host-side entry points (no kernel launch, no GPU needed).  Built and run by
 * tests/test_c_abi.py; prints one line per check and exits non-zero on a
 * failure. */
#include <stdio.h>
#include <string.h>

#include "gdr.h"

static int fails = 0;
#define CHECK(cond, what)                                   \
    do {                                                    \
        if (cond) {                                         \
            printf("ok %s\n", what);                        \
        } else {                                            \
            printf("FAIL %s\n", what);                      \
            ++fails;                                        \
        }                                                   \
    } while (0)

int main(void) {
    CHECK(gdr_abi_version() == GDR_ABI_VERSION, "abi version");
    CHECK(strcmp(gdr_strerror(GDR_OK), "ok") == 0, "strerror ok");
    CHECK(strcmp(gdr_strerror(GDR_EWORKSPACE), "workspace too small") == 0, "strerror workspace");

    gdr_fwd_args a;
    memset(&a, 0, sizeof a);
    a.B = 1; a.T = 256; a.H_q = 2; a.H_v = 4; a.K = 128; a.V = 128;
    a.dtype = GDR_BF16; a.out_dtype = GDR_F32; a.scale = 0.088f; a.cp_mode = GDR_CP_OFF;
    size_t bytes = 0;
    /* 4 chunks x 4 v heads of the forward's 13,312-byte T blocks */
    CHECK(gdr_fwd_workspace(&a, &bytes) == GDR_OK && bytes == 4 * 4 * 13312, "fwd workspace");
    a.H_v = 3;
    CHECK(gdr_fwd_workspace(&a, &bytes) == GDR_EINVAL, "fwd H_v % H_q");
    a.H_v = 4; a.K = 96;
    CHECK(gdr_fwd_workspace(&a, &bytes) == GDR_ENOTSUP, "fwd K");
    a.K = 128;
    CHECK(gdr_fwd(&a, NULL) == GDR_EINVAL, "fwd null pointers rejected before any launch");
    CHECK(gdr_fwd_noalloc(&a, NULL) == GDR_EINVAL, "fwd_noalloc null pointers rejected before any launch");
    CHECK(strcmp(gdr_strerror(GDR_ESCRATCH), "problem needs more than the library's static scratch buffer") == 0,
          "strerror scratch");
    CHECK(gdr_tblocks_bytes(&a, &bytes) == GDR_OK && bytes == 4 * 4 * 13312, "T blocks for the backward");
    a.h_bwd = (void *)16;
    a.cp_mode = GDR_CP_WARMUP;
    CHECK(gdr_fwd_workspace(&a, &bytes) == GDR_EINVAL, "fwd states for the backward need an exact scan");
    a.cp_mode = GDR_CP_OFF;
    a.h_bwd = NULL;

    gdr_bwd_args b;
    memset(&b, 0, sizeof b);
    b.B = 1; b.T = 256; b.H_q = 2; b.H_v = 4; b.K = 128; b.V = 128;
    b.dtype = GDR_BF16; b.grad_dtype = GDR_BF16; b.scale = 0.088f; b.cp_mode = GDR_CP_OFF;
    CHECK(gdr_bwd_workspace(&b, &bytes) == GDR_OK && bytes == 4 * 4 * (13312 + 2 * 4 * 128 * 128),
          "bwd workspace");
    b.h_bwd = (const void *)16;
    b.tblk_bwd = (const void *)16;
    CHECK(gdr_bwd_workspace(&b, &bytes) == GDR_OK && bytes == 4 * 4 * 4 * 128 * 128,
          "bwd workspace with the forward's states and T blocks");
    b.h_bwd = b.tblk_bwd = NULL;
    b.cp_mode = GDR_CP_WARMUP;
    CHECK(gdr_bwd_workspace(&b, &bytes) == GDR_EINVAL, "bwd has no warm-up split");
    return fails != 0;
}
