/* A plain C99 program against include/fc.h and include/fc_envelope.h: the
 * headers compile as C (no C++ in the declarations) and the library's
 * host-only entry points answer from C.  Every library call here either never
 * touches a device or is rejected by argument validation before any HIP call
 * (the pointers are fake host addresses).  Prints one "name value" line per
 * check; exit status 0. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fc.h"
#include "fc_envelope.h"

int main(void)
{
    const int plan4[1] = {4}, plan13[2] = {1, 3}, plan1111[4] = {1, 1, 1, 1}, bad[2] = {2, 3};
    const uint16_t *fake = (const uint16_t *)(uintptr_t)0x10000;
    uint16_t *fake_out = (uint16_t *)(uintptr_t)0x100000000ull;  /* far from every input range */
    const float ab[2] = {1.0f, 0.0f};
    fc_stage st[4];
    int vg = -1, waves = -1;

    printf("version %s\n", fc_version());
    printf("plan_bytes_4 %llu\n", (unsigned long long)fc_plan_bytes(4096, 4096, 4096, plan4, 1, 2));
    printf("plan_bytes_13 %llu\n", (unsigned long long)fc_plan_bytes(4096, 4096, 4096, plan13, 2, 2));
    printf("plan_bytes_1111 %llu\n", (unsigned long long)fc_plan_bytes(4096, 4096, 4096, plan1111, 4, 2));
    printf("plan_launches_1111 %d\n", fc_plan_launches(plan1111, 4));
    printf("chain_bytes_fused %llu\n", (unsigned long long)fc_chain_bytes(16777216, 8, FC_CHAIN_FUSED));
    printf("chain_bytes_naive %llu\n", (unsigned long long)fc_chain_bytes(16777216, 8, FC_CHAIN_NAIVE));
    printf("softmax_bytes_t64 %llu\n", (unsigned long long)fc_softmax_bytes(128, 2048, 64, FC_SOFTMAX_FUSED));
    printf("workspace_13 %zu\n", fc_gemm_workspace_bytes(4096, 4096, 4096, plan13, 2));
    printf("gemm_bad_plan %d\n", fc_gemm_epilogue(fake, fake, fake, fake, fake_out, 16, 64, 64, bad, 2,
                                                  NULL, 0, (fc_stream)0));
    printf("gemm_null %d\n", fc_gemm_epilogue(NULL, fake, fake, fake, fake_out, 16, 64, 64, plan4, 1, NULL, 0,
                                              (fc_stream)0));
    printf("noalloc_scratch %d\n", fc_gemm_epilogue_noalloc(fake, fake, fake, fake, fake_out, 4096, 8256, 64,
                                                            plan13, 2, (fc_stream)0));
    printf("chain_k0 %d\n", fc_chain((const float *)fake, (float *)fake_out, 16, ab, ab, 0, 1, FC_CHAIN_FUSED,
                                     NULL, 0, (fc_stream)0));
    printf("softmax_bad_tile %d\n", fc_causal_softmax(fake, fake_out, 1, 64, 0.125f, 48, FC_SOFTMAX_FUSED,
                                                      NULL, 0, (fc_stream)0));
    printf("stages %d\n", fc_gemm_epilogue_stages(16, 4096, 4096, st));
    printf("kernel_info %d\n", fc_kernel_info("fc::attention_fwd_kernel", &vg, NULL, NULL, NULL, NULL, &waves));
    printf("kernel_vgprs %d\n", vg);
    printf("status_scratch %s\n", fc_status_string(FC_ERR_SCRATCH));
    printf("noalloc_limit %zu\n", (size_t)FC_GEMM_NOALLOC_SCRATCH_BYTES);
    printf("envelope_chunk %zu\n", fce_chunk_bytes());
    printf("envelope_bad %d\n", fce_flat(NULL, NULL, 4096, (fc_stream)0));
    return 0;
}
