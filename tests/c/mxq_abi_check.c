/* mxq_abi_check.c -- a C11 caller of include/mxq.h: every declared entry point is
 * called through the header's own prototypes and types (so the compiler checks the
 * arguments), on paths that the library answers on the host before anything is
 * enqueued: the version and status strings, the two workspace-size queries, and
 * argument errors of each quantizing call.  The device addresses are fake (never
 * dereferenced on these paths); the program is run where no GPU is visible.
 * Exit status: 0 when every check holds, else the number of failed checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mxq.h"

static int failures = 0;

#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

/* A 16-byte aligned address that no buffer holds. */
#define DEV(T) ((T*)(uintptr_t)(1u << 20))
#define DEV_OFF(T, off) ((T*)(uintptr_t)((1u << 20) + (off)))

static void strings(void) {
    const mxq_status all[] = {MXQ_OK, MXQ_ERR_INVALID_ARGUMENT, MXQ_ERR_MISALIGNED,
                              MXQ_ERR_WORKSPACE_TOO_SMALL, MXQ_ERR_UNSUPPORTED, MXQ_ERR_HIP};
    size_t i, j;
    for (i = 0; i < sizeof all / sizeof all[0]; ++i) {
        const char* s = mxq_status_string(all[i]);
        CHECK(s != NULL && s[0] != '\0');
        for (j = 0; j < i; ++j) CHECK(strcmp(s, mxq_status_string(all[j])) != 0);
    }
    CHECK(strcmp(mxq_status_string(MXQ_OK), "MXQ_OK") == 0);
    CHECK(mxq_version() != NULL && strstr(mxq_version(), "gfx950") != NULL);
}

static void workspace_sizes(void) {
    /* grouped: a fixed 135,680 bytes, then 8 bytes per 16 rows x 1024 columns (or
     * part), rounded to 256 */
    CHECK(mxq_group_rht_quant_nvfp4_workspace_size(16384, 4096, 8, MXQ_ROWWISE | MXQ_COLUMNWISE) ==
          (size_t)(135680 + 8 * 1024 * 4));
    CHECK(mxq_group_rht_quant_nvfp4_workspace_size(128, 128, 1, MXQ_ROWWISE) == (size_t)(135680 + 256));
    CHECK(mxq_group_rht_quant_nvfp4_workspace_size(65536, 7168, 32, MXQ_ROWWISE) ==
          (size_t)(135680 + 8 * 4096 * 7));
    CHECK(mxq_group_rht_quant_nvfp4_workspace_size(16384, 4096, 8, MXQ_FP8_ROWWISE) == 0);
    CHECK(mxq_group_rht_quant_nvfp4_workspace_size(-1, 4096, 8, MXQ_ROWWISE) == 0);
    /* DSA NVFP4: 2 KB of table, then 4 bytes per 64 rows, rounded to 256 */
    CHECK(mxq_hadamard_quant_nvfp4_workspace_size(262144) == (size_t)(2048 + 4 * 4096));
    CHECK(mxq_hadamard_quant_nvfp4_workspace_size(0) == 0);
}

static void fp8_calls(void) {
    CHECK(mxq_quant_fp8_1x128(DEV(const uint16_t), 4, 200, 200, DEV(uint8_t), 208, DEV(float), 2, 1, NULL) ==
          MXQ_ERR_MISALIGNED);
    CHECK(mxq_quant_fp8_1x128(NULL, 4, 256, 256, DEV(uint8_t), 256, DEV(float), 2, 1, NULL) ==
          MXQ_ERR_INVALID_ARGUMENT);
    CHECK(mxq_quant_fp8_1x128(DEV_OFF(const uint16_t, 8), 4, 256, 256, DEV(uint8_t), 256, DEV(float), 2, 1,
                              NULL) == MXQ_ERR_MISALIGNED);
    CHECK(mxq_quant_fp8_1x128(NULL, 0, 256, 256, NULL, 256, NULL, 2, 1, NULL) == MXQ_OK);   /* empty */

    {
        mxq_fp8_block_out row = {DEV(uint8_t), 256, DEV(float), 2, 1};
        CHECK(mxq_quant_fp8_blockwise(DEV(const uint16_t), 4, 256, 256, 2u, &row, NULL, NULL) ==
              MXQ_ERR_INVALID_ARGUMENT);                                   /* unknown option */
        CHECK(mxq_quant_fp8_blockwise(DEV(const uint16_t), 4, 256, 256, MXQ_FP8_UE8M0, NULL, NULL, NULL) ==
              MXQ_ERR_INVALID_ARGUMENT);                                   /* no output */
    }
    CHECK(mxq_hadamard_quant_fp8(DEV(const uint16_t), 64, 129, DEV(const uint16_t), 64, 8, DEV(uint8_t),
                                 DEV(float), NULL) == MXQ_ERR_INVALID_ARGUMENT);
    CHECK(mxq_hadamard_quant_fp8(DEV(const uint16_t), 60, 60, DEV(const uint16_t), 68, 8, DEV(uint8_t),
                                 DEV(float), NULL) == MXQ_ERR_MISALIGNED);
    CHECK(mxq_hadamard_quant_fp8_ex(DEV(const uint16_t), 64, 64, DEV(const uint16_t), 64, 8, 0u, 0,
                                    DEV(uint8_t), DEV(float), 1, 1, NULL) == MXQ_ERR_INVALID_ARGUMENT);
    CHECK(mxq_swiglu_quant_fp8(DEV(const uint16_t), 256, DEV(const uint16_t), 256, 8, 200, DEV(uint8_t), 256,
                               DEV(float), 2, 1, NULL) == MXQ_ERR_MISALIGNED);
}

static void nvfp4_calls(void) {
    const int64_t sections[2] = {128, 256};
    const int64_t bad[2] = {128, 192};
    mxq_nvfp4_out row = {DEV(uint8_t), DEV(uint8_t), DEV(float)};
    mxq_nvfp4_out col = {DEV(uint8_t), DEV(uint8_t), DEV(float)};
    mxq_fp8_out f8 = {DEV(uint8_t), DEV(float)};
    const size_t need = mxq_group_rht_quant_nvfp4_workspace_size(384, 256, 2, MXQ_ROWWISE | MXQ_COLUMNWISE);
    const uint64_t offs[2] = {1, 2};
    const mxq_sr sr = {7, offs, NULL};
    const mxq_amax half = {DEV(const float), NULL, NULL, NULL};          /* one direction only */

    CHECK(mxq_group_rht_quant_nvfp4(DEV(const uint16_t), 256, bad, 2, 0, MXQ_ROWWISE | MXQ_COLUMNWISE, NULL,
                                    &row, &col, NULL, DEV(void), need, NULL) == MXQ_ERR_MISALIGNED);
    CHECK(mxq_group_rht_quant_nvfp4(DEV(const uint16_t), 256, sections, 2, 0, 0u, NULL, &row, &col, NULL,
                                    DEV(void), need, NULL) == MXQ_ERR_INVALID_ARGUMENT);
    CHECK(mxq_group_rht_quant_nvfp4(DEV(const uint16_t), 256, sections, 2, 0,
                                    MXQ_ROWWISE | MXQ_COLUMNWISE | MXQ_FP8_ROWWISE, &sr, &row, &col, NULL,
                                    DEV(void), need, NULL) == MXQ_ERR_INVALID_ARGUMENT);   /* FP8 out missing */
    CHECK(mxq_group_rht_quant_nvfp4(DEV(const uint16_t), 256, sections, 2, 0, MXQ_ROWWISE | MXQ_COLUMNWISE,
                                    &sr, &row, &col, &f8, DEV(void), need - 1, NULL) ==
          MXQ_ERR_WORKSPACE_TOO_SMALL);
    CHECK(mxq_group_rht_quant_nvfp4_with_amax(DEV(const uint16_t), 256, sections, 2, 0,
                                              MXQ_ROWWISE | MXQ_COLUMNWISE, NULL, &row, &col, NULL, &half,
                                              DEV(void), need, NULL) == MXQ_ERR_INVALID_ARGUMENT);
    CHECK(mxq_group_rht_quant_nvfp4_noalloc(DEV(const uint16_t), 256, bad, 2, 0, MXQ_ROWWISE, NULL, &row, NULL,
                                            NULL, NULL) == MXQ_ERR_MISALIGNED);
    CHECK(mxq_hadamard_quant_nvfp4(DEV(const uint16_t), 64, 64, DEV(const uint16_t), 64, 8, NULL, NULL,
                                   DEV(uint8_t), DEV(uint8_t), DEV(float), DEV(void),
                                   mxq_hadamard_quant_nvfp4_workspace_size(8) - 1, NULL) ==
          MXQ_ERR_WORKSPACE_TOO_SMALL);
    CHECK(mxq_hadamard_quant_nvfp4(DEV(const uint16_t), 64, 64, DEV(const uint16_t), 64, 8, NULL, NULL,
                                   DEV(uint8_t), DEV(uint8_t), NULL, DEV(void), 4096, NULL) ==
          MXQ_ERR_INVALID_ARGUMENT);                                       /* no global scale */
}

int main(void) {
    strings();
    workspace_sizes();
    fp8_calls();
    nvfp4_calls();
    if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
    else printf("mxq ABI: all checks passed\n");
    return failures;
}
