/* A plain C caller of libkda: includes include/kda.h, links libkda.so and
 * exercises the host side of every entry point -- identification, status
 * strings, workspace queries and argument validation.  Every argument set
 * below is rejected (or is empty) before any launch, so no GPU is touched:
 * the fake device addresses are never dereferenced.  Prints "ok" and exits
 * 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

int main(void) {
    void* P = (void*)(uintptr_t)0x100000; /* aligned fake device address */
    void* MIS = (void*)(uintptr_t)0x100002;
    float* PF = (float*)P;

    CHECK(strstr(kda_version(), "gfx950") != NULL);
    CHECK(strncmp(kda_status_str(KDA_OK), "KDA_OK", 6) == 0);
    CHECK(strncmp(kda_status_str(KDA_ERR_WORKSPACE), "KDA_ERR_WORKSPACE", 17) == 0);

    /* workspace queries */
    CHECK(kda_chunk_fwd_workspace_bytes(8, 8192, 32, 128, 128, 64, KDA_BF16) == 0);
    CHECK(kda_chunk_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, KDA_BF16) > 0);
    CHECK(kda_chunk_fwd_workspace_bytes(1, 256, 1, 96, 64, 64, KDA_F32) == 0);
    CHECK(kda_out_gate_workspace_bytes(8, 8192, 32, 128, 2304, KDA_BF16, 1) ==
          (size_t)8 * 8192 * 4096 * 2);
    CHECK(kda_recurrent_layer_step_workspace_bytes(256, 32, 128, 2304, KDA_BF16, 0) == 0);
    CHECK(kda_gdn_chunk_fwd_workspace_bytes(8, 8192, 32, 128, 128, 64, KDA_BF16) ==
          (size_t)8 * 8192 * 32 * 128 * 2);

    /* argument validation, before any launch */
    CHECK(kda_chunk_fwd(P, P, P, P, P, -5.f, NULL, P, PF, 1, 128, 2, 96, 128, 64, KDA_BF16, NULL, 0, NULL) ==
          KDA_ERR_UNSUPPORTED);
    CHECK(kda_chunk_fwd(P, P, P, P, P, 0.f, NULL, P, PF, 1, 128, 2, 128, 128, 64, KDA_BF16, NULL, 0, NULL) ==
          KDA_ERR_ARG);
    CHECK(kda_chunk_fwd(P, MIS, P, P, P, -5.f, NULL, P, PF, 1, 128, 2, 128, 128, 64, KDA_BF16, NULL, 0, NULL) ==
          KDA_ERR_ALIGN);
    CHECK(kda_chunk_fwd(P, P, P, P, P, -5.f, NULL, P, PF, 1, 4096, 2, 128, 128, 64, KDA_BF16, NULL, 0, NULL) ==
          KDA_ERR_WORKSPACE);
    CHECK(kda_chunk_fwd(P, P, P, P, P, -5.f, NULL, P, PF, 0, 128, 2, 128, 128, 64, KDA_BF16, NULL, 0, NULL) ==
          KDA_OK);
    CHECK(kda_chunk_fwd_noalloc(P, P, P, P, P, -5.f, NULL, P, PF, 1, 32768, 64, 128, 128, 64, KDA_BF16, NULL) ==
          KDA_ERR_SCRATCH);
    CHECK(kda_chunk_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, KDA_BF16) <= KDA_NOALLOC_SCRATCH_BYTES);
    CHECK(kda_recurrent_step(P, P, P, P, P, -5.f, NULL, P, 4, 2, 128, 128, KDA_BF16, NULL) == KDA_ERR_NULL);
    CHECK(kda_recurrent_step(P, P, P, P, P, -5.f, PF, P, -1, 2, 128, 128, KDA_BF16, NULL) == KDA_ERR_SHAPE);
    CHECK(kda_out_gate(P, P, -1.f, NULL, P, 2, 8, 4, 128, 0, KDA_BF16, NULL, 0, NULL) == KDA_ERR_ARG);
    CHECK(kda_out_gate(P, P, 1e-6f, P, P, 2, 8, 4, 128, 64, KDA_F32, P, 1u << 30, NULL) == KDA_ERR_UNSUPPORTED);
    CHECK(kda_recurrent_layer_step(P, P, P, P, P, -5.f, PF, NULL, 1e-6f, NULL, NULL, P, 4, 2, 128, 128, 0,
                                   KDA_BF16, NULL, 0, NULL) == KDA_ERR_NULL);
    CHECK(kda_recurrent_layer_step(P, P, P, P, P, -5.f, PF, P, 1e-6f, P, NULL, P, 4, 2, 128, 128, 64, KDA_BF16,
                                   NULL, 0, NULL) == KDA_ERR_WORKSPACE);
    CHECK(kda_gdn_chunk_fwd(P, P, P, NULL, P, -5.f, NULL, P, PF, 1, 128, 2, 128, 128, 64, KDA_BF16, P,
                            (size_t)1 << 30, NULL) == KDA_ERR_NULL);
    CHECK(kda_gdn_recurrent_step(P, P, P, MIS, P, -5.f, PF, P, 4, 2, 128, 128, KDA_BF16, NULL) == KDA_ERR_ALIGN);

    CHECK(kda_chunk_layer_fwd_workspace_bytes(8, 8192, 32, 128, 128, 64, 2304, KDA_BF16, 1) ==
          (size_t)2 * 8 * 8192 * 4096 * 2);
    CHECK(kda_chunk_layer_fwd(P, P, P, P, P, -5.f, NULL, NULL, 1e-6f, NULL, NULL, P, NULL, 1, 128, 2, 128, 128,
                              64, 0, KDA_BF16, P, (size_t)1 << 30, NULL) == KDA_ERR_NULL);
    CHECK(kda_chunk_layer_fwd(P, P, P, P, P, -5.f, NULL, P, 1e-6f, P, NULL, P, NULL, 1, 128, 2, 128, 128, 64,
                              64, KDA_BF16, NULL, 0, NULL) == KDA_ERR_WORKSPACE);

    CHECK(kda_recurrent_bwd_workspace_bytes(1, 32768, 32, 128, 128) == (size_t)32 * 576 * 128 * 128 * 4);
    CHECK(kda_recurrent_bwd(P, P, P, P, P, -5.f, NULL, P, NULL, PF, PF, PF, PF, NULL, NULL, 1, 128, 2, 128, 128,
                            KDA_BF16, P, (size_t)1 << 30, NULL) == KDA_ERR_NULL);

    CHECK(kda_dplr_fwd(P, P, P, P, P, NULL, -5.f, NULL, P, PF, 1, 128, 2, 128, 128, KDA_BF16, NULL) ==
          KDA_ERR_NULL);
    CHECK(kda_dplr_recurrent_step(P, P, P, P, P, P, -5.f, PF, P, 4, 2, 64, 96, KDA_F32, NULL) ==
          KDA_ERR_UNSUPPORTED);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
