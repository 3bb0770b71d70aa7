// Host-only stand-ins for the kernel translation units, so that the plan and run logic of
// gemm_api.cpp can be built and exercised under AddressSanitizer on a machine with no GPU.
// Every entry has the tile shape of the real one; a launch through them is a test failure.
#include <cstdio>
#include <cstdlib>

#include "../../tiled_gemm_epilogues_amd/csrc/gemm_internal.h"

namespace tge {
namespace {
hipError_t no_launch(const GemmParams &, unsigned, hipStream_t) {
    std::fprintf(stderr, "stub: a kernel launch was reached\n");
    std::abort();
}
hipError_t no_finish(const GemmParams &, hipStream_t) {
    std::fprintf(stderr, "stub: a finishing kernel was reached\n");
    std::abort();
}
const KernelEntry *entry(int bm, int bn, int bk, const char *name) {
    static KernelEntry table[64];
    static int used = 0;
    for (int i = 0; i < used; ++i)
        if (table[i].bm == bm && table[i].bn == bn && table[i].bk == bk && table[i].name == name) return &table[i];
    table[used] = {no_launch, bm, bn, bk, 2, 2, name};
    return &table[used++];
}
const KernelEntry *general(int a, int b, int cfg) {
    if (a < 0 || a > 1 || b < 0 || b > 1 || cfg < 0 || cfg >= CFG_COUNT) return nullptr;
    static const char *names[3] = {"gemm_mfma_256x256", "gemm_mfma_128x128", "gemm_mfma_64x64"};
    const int t[3] = {256, 128, 64};
    return entry(t[cfg], t[cfg], 64, names[cfg]);
}
const KernelEntry *fast(int a, int b, int rs) {
    if (a < 0 || a > 1 || b < 0 || b > 1) return nullptr;
    return entry(256, 256, 64, rs ? "gemm_fast_256x256_rs" : "gemm_fast_256x256");
}
const KernelEntry *fast128(int a, int b) {
    if (a < 0 || a > 1 || b < 0 || b > 1) return nullptr;
    return entry(128, 128, 64, "gemm_fast_128x128");
}
const KernelEntry *skinny(int b, int mt, int narrow) {
    if (b < 0 || b > 1 || mt < 1 || mt > 4 || (narrow && b != 1)) return nullptr;
    return entry(16 * mt, narrow ? 16 : 64, 32, narrow ? "gemm_skinny_n16" : "gemm_skinny");
}
const KernelEntry *diag(int a, int b, int dg) {
    if (a < 0 || a > 1 || b < 0 || b > 1 || dg < 1 || dg > 3) return nullptr;
    return entry(64, 64, 64, "gemm_diag");
}
const KernelEntry *cplx(int a, int b) {
    if (a < 0 || a > 1 || b < 0 || b > 1) return nullptr;
    return entry(128, 128, 32, "gemm_complex");
}
}  // namespace

const KernelEntry *kernels_f32_f32(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *kernels_f16_f16(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *kernels_f16_f32(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *kernels_bf16_bf16(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *kernels_bf16_f32(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *kernels_i8_i32(int a, int b, int c) { return general(a, b, c); }
const KernelEntry *diag_f32_f32(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *diag_f16_f16(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *diag_f16_f32(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *diag_bf16_bf16(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *diag_bf16_f32(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *diag_i8_i32(int a, int b, int d) { return diag(a, b, d); }
const KernelEntry *fast_f16_f16(int a, int b, int r) { return fast(a, b, r); }
const KernelEntry *fast_f16_f32(int a, int b, int r) { return fast(a, b, r); }
const KernelEntry *fast_bf16_bf16(int a, int b, int r) { return fast(a, b, r); }
const KernelEntry *fast_bf16_f32(int a, int b, int r) { return fast(a, b, r); }
const KernelEntry *fast_i8_i32(int a, int b, int r) { return fast(a, b, r); }
const KernelEntry *fast128_f16_f16(int a, int b) { return fast128(a, b); }
const KernelEntry *fast128_f16_f32(int a, int b) { return fast128(a, b); }
const KernelEntry *fast128_bf16_bf16(int a, int b) { return fast128(a, b); }
const KernelEntry *fast128_bf16_f32(int a, int b) { return fast128(a, b); }
const KernelEntry *fast128_i8_i32(int a, int b) { return fast128(a, b); }
const KernelEntry *skinny_f16_f16(int b, int m, int n) { return skinny(b, m, n); }
const KernelEntry *skinny_f16_f32(int b, int m, int n) { return skinny(b, m, n); }
const KernelEntry *skinny_bf16_bf16(int b, int m, int n) { return skinny(b, m, n); }
const KernelEntry *skinny_bf16_f32(int b, int m, int n) { return skinny(b, m, n); }
const KernelEntry *skinny_i8_i32(int b, int m, int n) { return b == 1 ? skinny(b, m, n) : nullptr; }
const KernelEntry *complex_cf16_cf32(int a, int b) { return cplx(a, b); }
const KernelEntry *complex_cf16_cf16(int a, int b) { return cplx(a, b); }
const KernelEntry *complex_df16_df32(int a, int b) { return cplx(a, b); }
const KernelEntry *complex_df16_df16(int a, int b) { return cplx(a, b); }
hipError_t finish_f16_f16(const GemmParams &p, hipStream_t s) { return no_finish(p, s); }
hipError_t finish_f16_f32(const GemmParams &p, hipStream_t s) { return no_finish(p, s); }
hipError_t finish_bf16_bf16(const GemmParams &p, hipStream_t s) { return no_finish(p, s); }
hipError_t finish_bf16_f32(const GemmParams &p, hipStream_t s) { return no_finish(p, s); }
hipError_t finish_i8_i32(const GemmParams &p, hipStream_t s) { return no_finish(p, s); }
int64_t repack_blocks(const RepackJob &) { return 1; }
hipError_t repack_launch(const RepackJob &, const RepackJob &, hipStream_t) { std::abort(); }
int64_t convert_blocks(const ConvertJob &) { return 1; }
hipError_t convert_launch(const ConvertJob &, const ConvertJob &, hipStream_t) { std::abort(); }
int64_t pair_blocks(const PairJob &) { return 1; }
hipError_t pair_launch(const PairJob &, const PairJob &, hipStream_t) { std::abort(); }
}  // namespace tge
