/* A C99 program against include/q2_0.h and libq2_0.so: the header compiles as C, the
 * library links from C, and the host-side contract holds without a GPU -- version and
 * status strings, and calls that every argument check rejects (or that are empty
 * no-ops), which launch nothing.  Device pointers are stand-in addresses: no call made
 * here dereferences them.  Prints "ok" and exits 0, or names the first failed check. */
#include <stdio.h>
#include <string.h>

#include "q2_0.h"

static int failures = 0;

#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__);   \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

int main(void) {
    void *w = (void *)(uintptr_t)0x100000; /* 16-byte aligned stand-ins */
    float *x = (float *)(uintptr_t)0x200000;
    float *y = (float *)(uintptr_t)0x300000;
    int32_t *ids = (int32_t *)(uintptr_t)0x400000;
    int st;

    CHECK(q2_0_version() != NULL && strstr(q2_0_version(), "gfx950") != NULL);
    for (st = Q2_0_OK; st <= Q2_0_ERR_TOO_LARGE; ++st) CHECK(q2_0_status_string(st) != NULL);
    CHECK(strncmp(q2_0_status_string(Q2_0_ERR_SHAPE), "Q2_0_ERR_SHAPE", 14) == 0);
    CHECK(q2_0_status_string(12345) != NULL);

    /* get_rows */
    CHECK(q2_0_get_rows(w, 10, 100, ids, 4, x, 100, NULL) == Q2_0_ERR_SHAPE);   /* K % 64 */
    CHECK(q2_0_get_rows(w, 10, 64, ids, 0, x, 64, NULL) == Q2_0_OK);            /* empty */
    CHECK(q2_0_get_rows(w, 10, 64, NULL, 4, x, 64, NULL) == Q2_0_ERR_NULL);
    CHECK(q2_0_get_rows(w, 10, 64, ids, 4, x, 63, NULL) == Q2_0_ERR_LAYOUT);
    CHECK(q2_0_get_rows((char *)w + 1, 10, 64, ids, 4, x, 64, NULL) == Q2_0_ERR_ALIGN);

    /* mat-vec */
    CHECK(q2_0_mul_mat_vec(w, 10, 64, x, 64, 0, y, 10, NULL) == Q2_0_OK);       /* N = 0 */
    CHECK(q2_0_mul_mat_vec(w, -1, 64, x, 64, 1, y, 10, NULL) == Q2_0_ERR_SHAPE);
    CHECK(q2_0_mul_mat_vec(w, 10, 64, NULL, 64, 1, y, 10, NULL) == Q2_0_ERR_NULL);
    CHECK(q2_0_mul_mat_vec(w, 10, 64, x, 63, 1, y, 10, NULL) == Q2_0_ERR_LAYOUT);
    CHECK(q2_0_mul_mat_vec(w, 10, 64, x, 64, 1, y, 9, NULL) == Q2_0_ERR_LAYOUT);
    CHECK(q2_0_mul_mat_vec(w, 10, 64, x, 64, Q2_0_MAT_VEC_MAX_N + 1, y, 10, NULL) == Q2_0_ERR_UNSUPPORTED);

    /* GEMM: precisions, workspace sizes and checks */
    CHECK(q2_0_mul_mat(w, 10, 64, x, 64, 20, y, 10, 3, NULL, 0, NULL) == Q2_0_ERR_UNSUPPORTED);
    CHECK(q2_0_mul_mat_workspace_bytes(4096, 4096, 512, Q2_0_PREC_F32) == 0);
    CHECK(q2_0_mul_mat_workspace_bytes(4096, 4096, 8, Q2_0_PREC_F16_MFMA) == 0);
    {
        const size_t f16 = q2_0_mul_mat_workspace_bytes(65536, 4096, 512, Q2_0_PREC_F16_MFMA);
        const size_t f32m = q2_0_mul_mat_workspace_bytes(65536, 4096, 512, Q2_0_PREC_F32_MFMA);
        const size_t need = q2_0_mul_mat_workspace_bytes(10, 64, 20, Q2_0_PREC_F16_MFMA);
        CHECK(f16 >= (size_t)512 * 4096 * 2 && f32m >= 2 * (size_t)512 * 4096 * 2);
        CHECK(need > 0);
        CHECK(q2_0_mul_mat(w, 10, 64, x, 64, 20, y, 10, Q2_0_PREC_F16_MFMA, w, need - 1, NULL) ==
              Q2_0_ERR_WORKSPACE);
    }
    CHECK(q2_0_mul_mat_noalloc(w, 4096, 12288, x, 12288, 4096, y, 4096, Q2_0_PREC_F16_MFMA, NULL) ==
          Q2_0_ERR_TOO_LARGE);

    /* groups and batches: empty calls are no-ops, bad items are rejected */
    {
        q2_0_mat_vec_item items[2];
        items[0].w = w; items[0].M = 10; items[0].y = y; items[0].ldy = 10;
        items[1].w = w; items[1].M = 5; items[1].y = y; items[1].ldy = 4;   /* ldy < M */
        CHECK(q2_0_mul_mat_vec_group(NULL, 0, 64, x, 64, 1, NULL) == Q2_0_OK);
        CHECK(q2_0_mul_mat_vec_group(items, 2, 64, x, 64, 1, NULL) == Q2_0_ERR_LAYOUT);
        CHECK(q2_0_mul_mat_group(items, 2, 64, x, 64, 20, Q2_0_PREC_F16_MFMA, w, 1 << 20, NULL) ==
              Q2_0_ERR_LAYOUT);
    }
    CHECK(q2_0_mul_mat_vec_batch(NULL, 0, Q2_0_ACT_F32, 1, NULL) == Q2_0_OK);

    /* activation types and the expert product */
    CHECK(q2_0_mul_mat_vec_act(w, 10, 64, x, 7, 64, 1, y, 10, NULL) == Q2_0_ERR_UNSUPPORTED);
    CHECK(q2_0_mul_mat_id(w, 0, 10, 64, x, Q2_0_ACT_F32, 64, 1, ids, 2, 3, y, 10, Q2_0_PREC_F32, w, 1 << 20,
                          NULL) == Q2_0_ERR_SHAPE);
    CHECK(q2_0_mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, Q2_0_PREC_F32_MFMA) ==
          q2_0_mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, Q2_0_PREC_F32));

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
