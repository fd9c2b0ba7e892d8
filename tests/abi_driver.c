/* Host-side driver for the sanitizer test (tests/test_host_sanitizers.py):
 * calls every entry point of include/moegg.h down its argument-validation
 * paths and the pure host helpers.  No call reaches a kernel launch, so no GPU
 * is needed.  Prints "ok" and exits 0 when every status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../include/moegg.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        int got_ = (int)(call);                                                         \
        if (got_ != (int)(want)) {                                                      \
            fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

int main(void) {
    void* fake = (void*)(uintptr_t)0x100000;       /* aligned, never dereferenced */
    void* odd = (void*)(uintptr_t)0x100002;
    size_t ws = moegg_workspace_bytes(64, 32768);
    if (ws == 0 || ws % 256) ++fails;
    EXPECT(moegg_workspace_bytes(0, 1), 0);
    EXPECT(moegg_workspace_bytes(4097, 1), 0);
    for (int s = 0; s < 6; ++s)
        if (!moegg_status_string((moegg_status_t)s)) ++fails;
    if (moegg_version() < 1) ++fails;

    EXPECT(moegg_schedule(NULL, 8, 132, 1, 0, 256, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_schedule(fake, 8, 132, 1, 48, 256, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_schedule(fake, 8, 132, 1, 0, 256, fake, 8, NULL), MOEGG_ERR_WORKSPACE);
    EXPECT(moegg_schedule_exemplar(fake, 8, 132, 1, 256, NULL, 4, 0, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_schedule_exemplar(fake, 8, 132, 1, 256, fake, 300, 0, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_schedule_exemplar(fake, 8, 132, 1, 256, fake, 4, -1, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);

    EXPECT(moegg_grouped_gemm_contiguous(NULL, NULL, fake, NULL, fake, fake, 8, 132, 512, 256, 1, MOEGG_BF16,
                                         MOEGG_B_KN, 0, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_contiguous(fake, NULL, fake, NULL, fake, fake, 8, 132, 100, 256, 1, MOEGG_BF16,
                                         MOEGG_B_KN, 0, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_contiguous(fake, fake, fake, fake, fake, fake, 8, 132, 512, 512, 1,
                                         MOEGG_FP8_E4M3_FP4_E2M1, MOEGG_B_KN, 0, fake, ws, NULL),
           MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_contiguous(fake, fake, fake, odd, fake, fake, 8, 132, 512, 512, 1,
                                         MOEGG_FP8_E4M3_E8M0, MOEGG_B_NK, 0, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_contiguous(fake, NULL, fake, NULL, fake, fake, 8, 132, 512, 256, 1, MOEGG_BF16,
                                         MOEGG_B_KN, 0, NULL, 0, NULL), MOEGG_ERR_WORKSPACE);
    EXPECT(moegg_grouped_gemm_contiguous_scheduled(fake, NULL, fake, NULL, fake, 8, 132, 512, 256, MOEGG_BF16,
                                                   MOEGG_B_KN, 96, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_swiglu_scheduled(fake, NULL, fake, NULL, fake, NULL, 8, 132, 512, 64, MOEGG_BF16,
                                               MOEGG_B_NK, 0, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_swiglu_scheduled(fake, NULL, fake, NULL, fake, odd, 8, 132, 512, 128, MOEGG_BF16,
                                               MOEGG_B_NK, 0, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_masked(fake, NULL, fake, NULL, fake, fake, 32, 0, 2048, 7168, MOEGG_BF16, MOEGG_B_KN,
                                     NULL, 0, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_masked(fake, fake, fake, fake, fake, fake, 31, 255, 2048, 7168, MOEGG_FP8_E4M3_E8M0,
                                     MOEGG_B_KN, NULL, 0, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_k_grouped(fake, fake, fake, fake, 16, 100, 2000, 7168, fake, ws, NULL),
           MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_k_grouped(NULL, NULL, fake, fake, 16, 1, 2048, 7168, fake, ws, NULL),
           MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_k_grouped_fp8(fake, fake, fake, fake, fake, fake, 16, 100, 2048, 7168, 0, fake, ws,
                                            NULL), MOEGG_ERR_INVALID_ARG);          /* rows but no scale groups */
    EXPECT(moegg_grouped_gemm_k_grouped_fp8(fake, NULL, fake, fake, fake, fake, 16, 100, 2048, 7168, 16, fake, ws,
                                            NULL), MOEGG_ERR_INVALID_ARG);          /* missing X scales */
    EXPECT(moegg_grouped_gemm_k_grouped_fp8(fake, odd, fake, fake, fake, fake, 16, 100, 2048, 7168, 16, fake, ws,
                                            NULL), MOEGG_ERR_INVALID_ARG);          /* misaligned scales */
    EXPECT(moegg_grouped_gemm_k_grouped_fp8(fake, fake, fake, fake, fake, fake, 16, 100, 2048, 7168, 80000, fake,
                                            ws, NULL), MOEGG_ERR_UNSUPPORTED);      /* scale offsets past 2^31 */
    EXPECT(moegg_grouped_gemm_k_grouped_fp8(fake, fake, fake, fake, fake, fake, 16, 100, 2000, 7168, 16, fake, ws,
                                            NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_grouped_gemm_k_grouped_e8m0(fake, NULL, fake, fake, fake, fake, 16, 100, 2048, 7168, 16, fake, ws,
                                             NULL), MOEGG_ERR_INVALID_ARG);         /* missing X scales */
    EXPECT(moegg_grouped_gemm_k_grouped_e8m0(fake, (const uint8_t*)odd, fake, fake, fake, fake, 16, 100, 2048, 7168,
                                             16, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);   /* misaligned scales */
    EXPECT(moegg_grouped_gemm_k_grouped_e8m0(fake, fake, fake, fake, fake, fake, 16, 100, 2048, 7168, 300000, fake,
                                             ws, NULL), MOEGG_ERR_UNSUPPORTED);     /* scale offsets past 2^31 */
    EXPECT(moegg_grouped_gemm_k_grouped_e8m0(fake, fake, fake, fake, fake, fake, 16, 100, 2048, 7168, 80000, NULL,
                                             0, NULL), MOEGG_ERR_WORKSPACE);        /* 80000 groups fit bytes */
    {
        moegg_stats_t st = {0};
        moegg_report_t rep;
        st.U = 132;
        st.sum_sq = 2180;
        st.P_exec = 192;
        st.P_at[0] = 160;
        EXPECT(moegg_stats_report(&st, &rep), MOEGG_OK);
        if (rep.padding_fraction[0] != 28.0 / 160.0 || rep.padding_fraction[1] != 0.0) ++fails;
        EXPECT(moegg_stats_report(NULL, &rep), MOEGG_ERR_INVALID_ARG);
        st.U = -1;
        EXPECT(moegg_stats_report(&st, &rep), MOEGG_ERR_INVALID_ARG);
    }
    EXPECT(moegg_expert_mlp_fused(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 8, 132, 512, 256, 512, 1,
                                  MOEGG_BF16, MOEGG_B_NK, fake, ws, NULL), MOEGG_ERR_UNSUPPORTED);
    EXPECT(moegg_expert_mlp_fused(fake, fake, fake, fake, fake, fake, fake, NULL, fake, fake, 8, 132, 512, 256, 512, 1,
                                  MOEGG_FP8_E4M3, MOEGG_B_NK, fake, ws, NULL), MOEGG_ERR_INVALID_ARG);
    /* allocation-free variant: argument errors, and a workspace beyond its fixed array, before any HIP call */
    EXPECT(moegg_grouped_gemm_contiguous_noalloc(NULL, NULL, fake, NULL, fake, fake, 8, 132, 512, 256, 1, MOEGG_BF16,
                                                 MOEGG_B_KN, 0, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_grouped_gemm_contiguous_noalloc(fake, NULL, fake, NULL, fake, fake, 64, 8 << 20, 256, 256, 1,
                                                 MOEGG_BF16, MOEGG_B_KN, 0, NULL), MOEGG_ERR_WORKSPACE);
    if (moegg_workspace_bytes(64, 8 << 20) <= MOEGG_NOALLOC_SCRATCH_BYTES) ++fails;
    EXPECT(moegg_stats_read(NULL, NULL, NULL), MOEGG_ERR_INVALID_ARG);
    EXPECT(moegg_selection_read(NULL, NULL, NULL), MOEGG_ERR_INVALID_ARG);
    int64_t n = 0;
    EXPECT(moegg_tile_list_read(fake, NULL, 5, &n, NULL), MOEGG_ERR_INVALID_ARG);
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
