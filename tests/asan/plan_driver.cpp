// Exercises the host side of the C ABI (plan creation over a grid of descriptions, the texts,
// destruction, argument checks of both run entry points) for an AddressSanitizer build.  No
// call here reaches a kernel: runs are made only where they return before any launch.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/gemm.h"

extern "C" int enum_calls(void);

static int failures = 0;
static void expect(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

int main() {
    const int64_t sizes[] = {0, 1, 7, 16, 64, 65, 256, 257, 1000, 4095, 8192};
    const gemm_dtype_t ab_types[] = {GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_I8, GEMM_I32, GEMM_CF16, GEMM_DF16};
    const gemm_dtype_t cd_types[] = {GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_I32, GEMM_CF32, GEMM_CF16, GEMM_DF32};
    long plans = 0;
    for (int64_t M : sizes)
        for (int64_t N : sizes)
            for (int64_t K : {(int64_t)0, (int64_t)64, (int64_t)333, (int64_t)4096}) {
                for (int ops = 0; ops < 4; ++ops)
                    for (gemm_dtype_t ab : ab_types)
                        for (gemm_dtype_t cd : cd_types) {
                            gemm_desc_t d;
                            std::memset(&d, 0, sizeof(d));
                            d.M = M; d.N = N; d.K = K;
                            d.op_a = (gemm_op_t)(ops & 1); d.op_b = (gemm_op_t)(ops >> 1);
                            d.lda = (d.op_a == GEMM_OP_N ? K : M) + (ops == 3 ? 3 : 0);
                            d.ldb = (d.op_b == GEMM_OP_N ? N : K) + (ops == 1 ? 1 : 0);
                            if (d.lda < 1) d.lda = 1;
                            if (d.ldb < 1) d.ldb = 1;
                            d.ldc = N > 0 ? N : 1;
                            d.ab_type = ab; d.cd_type = cd;
                            d.epilogue = (gemm_epilogue_t)((M + N + ops) % 4);
                            d.batch = (M + K) % 3 == 0 ? 3 : 1;
                            d.stride_a = d.batch > 1 ? (M + 1) * (K + 1) : 0;
                            d.stride_b = 0;
                            d.stride_c = d.batch > 1 ? M * d.ldc + 8 : 0;
                            d.stride_bias = d.batch > 1 ? N : 0;
                            const int v = (int)((M * 7 + N * 3 + K + ops) % 8);
                            d.transform_a = (gemm_transform_t)(v & 3);
                            d.transform_b = (gemm_transform_t)((v >> 1) & 3);
                            d.transform_c = (gemm_transform_t)(v == 5 ? 1 : 0);
                            d.kind_a = (v == 7 && K == M) ? GEMM_OPERAND_DIAGONAL : GEMM_OPERAND_DENSE;
                            d.kind_b = GEMM_OPERAND_DENSE;
                            d.algo = (gemm_algo_t)(v % 8);
                            // tile 128 with NOSPLIT, and with SPLIT for half the shapes (the
                            // 128x128 tiles' pinned K split)
                            d.tile = (v == 6 || (v == 5 && (M + N) % 2 == 0)) ? 128 : 0;
                            gemm_plan_t p = nullptr;
                            const gemm_status_t st = gemm_plan_create_desc(&p, &d);
                            expect((st == GEMM_STATUS_SUCCESS) == (p != nullptr), "plan iff success");
                            if (!p) continue;
                            ++plans;
                            char small[8], big[256];
                            expect(gemm_plan_describe(p, small, sizeof(small)) == GEMM_STATUS_SUCCESS, "describe");
                            expect(std::strlen(small) < sizeof(small), "describe truncates");
                            expect(gemm_plan_describe(p, big, sizeof(big)) == GEMM_STATUS_SUCCESS, "describe");
                            expect(gemm_plan_describe(p, big, 0) == GEMM_STATUS_INVALID_VALUE, "len 0");
                            const void *fake = reinterpret_cast<const void *>((uintptr_t)0x10000);
                            // argument errors return before any launch
                            if (M > 0 && N > 0 && d.batch > 0) {
                                expect(gemm_run(p, fake, fake, fake, nullptr, fake, 1.0f, 0.0f, nullptr) ==
                                           GEMM_STATUS_INVALID_VALUE, "NULL D");
                                expect(gemm_run_noalloc(p, fake, fake, fake, nullptr, fake, 1.0f, 0.0f, nullptr) ==
                                           GEMM_STATUS_INVALID_VALUE, "NULL D (noalloc)");
                                // (int8 plans reject any alpha other than 1 first)
                                expect(gemm_run(p, fake, fake, fake, (void *)fake, fake, NAN, 0.0f, nullptr) ==
                                           (ab == GEMM_I8 ? GEMM_STATUS_NOT_SUPPORTED : GEMM_STATUS_INVALID_VALUE),
                                       "NaN alpha");
                                // a run whose route needs scratch stops at the sizing pass or at the
                                // device lookup (no device here): SCRATCH_LIMIT or HIP_ERROR
                                if (K > 0 && (std::strstr(big, "ksplit") || std::strstr(big, "repack") ||
                                    std::strstr(big, "convert") || std::strstr(big, "as real"))) {
                                    const gemm_status_t r = gemm_run_noalloc(p, fake, fake, fake, (void *)fake,
                                                                             fake, 1.0f, 1.0f, nullptr);
                                    expect(r == GEMM_STATUS_SCRATCH_LIMIT || r == GEMM_STATUS_HIP_ERROR ||
                                               r == GEMM_STATUS_NOT_SUPPORTED, "noalloc stops before launching");
                                }
                            } else {
                                expect(gemm_run(p, nullptr, nullptr, nullptr, nullptr, nullptr, 1.0f, 0.0f, nullptr) ==
                                           GEMM_STATUS_SUCCESS, "empty run");
                            }
                            expect(gemm_plan_destroy(p) == GEMM_STATUS_SUCCESS, "destroy");
                        }
            }
    expect(gemm_plan_destroy(nullptr) == GEMM_STATUS_SUCCESS, "destroy NULL");
    // out-of-range enum values, passed as a C caller passes them (ints): see enum_calls.c
    failures += enum_calls();
    gemm_plan_t p = nullptr;
    expect(gemm_plan_create_desc(&p, nullptr) == GEMM_STATUS_INVALID_VALUE && !p, "NULL desc");
    std::printf("%ld plans checked, %d failures\n", plans, failures);
    return failures ? 1 : 0;
}
