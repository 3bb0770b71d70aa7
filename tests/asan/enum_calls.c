/* Out-of-range enum values through the C ABI, as C callers pass them (a C enum is an int):
 * the status text is never NULL and every out-of-range field of a description is rejected
 * with GEMM_STATUS_INVALID_VALUE.  Returns the number of failed checks. */
#include <stdio.h>
#include <string.h>

#include "../../include/gemm.h"

int enum_calls(void) {
    int failures = 0;
    for (int s = -1; s < 8; ++s)
        if (!gemm_status_string((gemm_status_t)s)) {
            fprintf(stderr, "FAILED: status string %d\n", s);
            ++failures;
        }
    const int bad[3] = {-1, 9, 1 << 20};
    for (int field = 0; field < 11; ++field)
        for (int b = 0; b < 3; ++b) {
            gemm_desc_t d;
            memset(&d, 0, sizeof d);
            d.M = d.N = d.K = 64;
            d.lda = d.ldb = d.ldc = 64;
            d.ab_type = GEMM_F16;
            d.cd_type = GEMM_F16;
            d.batch = 1;
            int *fields[11] = {(int *)&d.op_a, (int *)&d.op_b, (int *)&d.ab_type, (int *)&d.cd_type,
                               (int *)&d.epilogue, (int *)&d.transform_a, (int *)&d.transform_b,
                               (int *)&d.transform_c, (int *)&d.kind_a, (int *)&d.kind_b, (int *)&d.algo};
            *fields[field] = bad[b];
            gemm_plan_t p = NULL;
            if (gemm_plan_create_desc(&p, &d) != GEMM_STATUS_INVALID_VALUE || p) {
                fprintf(stderr, "FAILED: field %d value %d accepted\n", field, bad[b]);
                ++failures;
            }
            gemm_plan_t q = NULL;
            if (field < 5 &&
                gemm_plan_create(&q, 64, 64, 64, field == 0 ? (gemm_op_t)bad[b] : GEMM_OP_N,
                                 field == 1 ? (gemm_op_t)bad[b] : GEMM_OP_N, 64, 64, 64,
                                 field == 2 ? (gemm_dtype_t)bad[b] : GEMM_F16,
                                 field == 3 ? (gemm_dtype_t)bad[b] : GEMM_F16,
                                 field == 4 ? (gemm_epilogue_t)bad[b] : GEMM_EPI_NONE) != GEMM_STATUS_INVALID_VALUE) {
                fprintf(stderr, "FAILED: gemm_plan_create field %d value %d accepted\n", field, bad[b]);
                ++failures;
            }
        }
    return failures;
}
