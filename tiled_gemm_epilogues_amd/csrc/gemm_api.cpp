// C ABI of the library: plan creation and validation, kernel selection, launch.
// Host code only; the kernels live in gemm_kernels.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "../../include/gemm.h"
#include "gemm_internal.h"

using tge::GemmParams;
using tge::KernelEntry;

struct gemm_plan {
    int64_t M, N, K, lda, ldb, ldc;
    int64_t batch, stride_a, stride_b, stride_c, stride_bias;
    // a second batch mode (1: none): product (b1, b2) at b1 * stride + b2 * stride2
    int64_t batch2, stride2_a, stride2_b, stride2_c, stride2_bias;
    int xform_a, xform_b, xform_c;
    int op_a, op_b, ab, cd, epi;
    const KernelEntry *kernel;       // general kernel (always valid)
    const KernelEntry *fast;         // fast or skinny kernel when the plan qualifies, else nullptr
    bool fast_is_skinny;             // `fast` is the skinny kernel (grid: k splits x 64-column blocks)
    int ksplit;                      // skinny or fast kernel: k splits S over workgroups
    // fast kernel with K split: the product as a batch of S products over K chunks into fp32
    // partial sums in ws, then the finishing kernel (nullptr: no split)
    const KernelEntry *fast_part;
    hipError_t (*finish)(const GemmParams &, hipStream_t);
    int ws_dev;                      // device of the skinny split-K workspace (-1: none yet)
    float *ws;                       // skinny split-K partial sums: batch * S * M * N floats
    const KernelEntry *fast_rs;      // register-staged fast kernel: any alignment, else nullptr
    // direct-load fast kernel on aligned copies of the operands it cannot read in place
    const KernelEntry *fast_pk;      // nullptr: no repacking for this plan
    int pk_need;                     // bit 0 / bit 1: A / B always copied (ld, stride or extent)
    int pk_want;                     // bit 0: A copied by choice although readable in place
    // A stored transposed, B not: A's copies are transposed into K-contiguous rows and the
    // kernels of the non-transposed layout run on them (the 16x16 schedule)
    bool pk_tr;
    const KernelEntry *fast_pk_tr;   // direct-load kernel on a transposed copy of A
    const KernelEntry *fast_part_tr; // its K-split variant (nullptr: no split)
    const KernelEntry *fast_part128; // K split of the 128x128 tiles (nullptr: none)
    const KernelEntry *fast_part128_tr; // the same on a transposed copy of A
    int64_t pk_ld_a, pk_ld_b;        // leading dimensions of the copies (whole 128-byte lines)
    int64_t pk_kpad;                 // K rounded up to whole slabs: the copies are zero there
    int64_t pk_off_b, pk_bytes;      // byte offset of B's copy in the workspace, total size
    int pk_dev;                      // device of the copy workspace (-1: none yet)
    void *pk_ws;
    // complex / dual numbers as a real fp16 product M x 2N x 2K on rewritten operands
    gemm_plan *cx;                   // that real plan; nullptr: the complex kernel runs
    int64_t cx_ld_a, cx_ld_b;        // rewritten A (A transposed only) and B: leading dimensions
    int64_t cx_off_b, cx_bytes;      // byte offset of B's rewrite in the workspace, total size
    int cx_dev;
    void *cx_ws;
    // operands stored as fp32 or int8 and converted to the 16-bit input type as they are
    // loaded: a conversion pass into the workspace, then the plan cv on the converted rows
    gemm_plan *cv;                   // nullptr: no conversion
    int cv_src_a, cv_src_b;          // -1: not converted, else tge::ConvertSrc
    int64_t cv_rows_a, cv_rows_b;    // stored rows of one product's operand
    int64_t cv_len_a, cv_len_b;      // elements per stored row
    int64_t cv_ld_a, cv_ld_b;        // pitch (elements) of the converted rows
    int64_t cv_off_b, cv_bytes;      // byte offset of B's converted rows, workspace size
    int cv_dev;
    void *cv_ws;
    int tiles_m, tiles_n, group_m;
    unsigned grid;
    char desc[256];
};

namespace {

// The integer held by an enum argument.  Callers across the C ABI may pass any int (C enums are
// ints); reading an out-of-range value as the C++ enum type is undefined, so arguments are
// checked through their bits before they are used as enums.
template <class E>
int enum_bits(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "C ABI enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}
template <class E>
void copy_enum(E &dst, const E &src) { memcpy(&dst, &src, sizeof dst); }

const char *dtype_name(int t) {
    switch (t) {
    case GEMM_F32: return "f32";
    case GEMM_F16: return "f16";
    case GEMM_BF16: return "bf16";
    case GEMM_I8: return "i8";
    case GEMM_I32: return "i32";
    case GEMM_CF16: return "cf16";
    case GEMM_CF32: return "cf32";
    case GEMM_DF16: return "df16";
    case GEMM_DF32: return "df32";
    }
    return "?";
}

int elem_bytes(int t) {
    switch (t) {
    case GEMM_F16:
    case GEMM_BF16: return 2;
    case GEMM_I8: return 1;
    case GEMM_CF16:
    case GEMM_DF16: return 4;
    case GEMM_CF32:
    case GEMM_DF32: return 8;
    default: return 4;
    }
}

using Lookup = const KernelEntry *(*)(int, int, int);

using FastLookup = const KernelEntry *(*)(int, int, int);

FastLookup fast_table(int ab, int cd) {
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::fast_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::fast_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::fast_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::fast_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::fast_i8_i32;
    return nullptr;
}

using Fast128Lookup = const KernelEntry *(*)(int, int);

Fast128Lookup fast128_table(int ab, int cd) {
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::fast128_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::fast128_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::fast128_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::fast128_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::fast128_i8_i32;
    return nullptr;
}

using SkinnyLookup = const KernelEntry *(*)(int, int, int);

using FinishFn = hipError_t (*)(const GemmParams &, hipStream_t);

FinishFn finish_table(int ab, int cd) {
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::finish_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::finish_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::finish_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::finish_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::finish_i8_i32;
    return nullptr;
}

SkinnyLookup skinny_table(int ab, int cd) {
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::skinny_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::skinny_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::skinny_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::skinny_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::skinny_i8_i32;
    return nullptr;
}

using ComplexLookup = const KernelEntry *(*)(int, int);

ComplexLookup complex_table(int ab, int cd) {
    if (ab == GEMM_CF16 && cd == GEMM_CF32) return tge::complex_cf16_cf32;
    if (ab == GEMM_CF16 && cd == GEMM_CF16) return tge::complex_cf16_cf16;
    if (ab == GEMM_DF16 && cd == GEMM_DF32) return tge::complex_df16_df32;
    if (ab == GEMM_DF16 && cd == GEMM_DF16) return tge::complex_df16_df16;
    return nullptr;
}

Lookup diag_table(int ab, int cd) {
    if (ab == GEMM_F32 && cd == GEMM_F32) return tge::diag_f32_f32;
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::diag_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::diag_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::diag_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::diag_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::diag_i8_i32;
    return nullptr;
}

Lookup pair_table(int ab, int cd) {
    if (ab == GEMM_F32 && cd == GEMM_F32) return tge::kernels_f32_f32;
    if (ab == GEMM_F16 && cd == GEMM_F16) return tge::kernels_f16_f16;
    if (ab == GEMM_F16 && cd == GEMM_F32) return tge::kernels_f16_f32;
    if (ab == GEMM_BF16 && cd == GEMM_BF16) return tge::kernels_bf16_bf16;
    if (ab == GEMM_BF16 && cd == GEMM_F32) return tge::kernels_bf16_f32;
    if (ab == GEMM_I8 && cd == GEMM_I32) return tge::kernels_i8_i32;
    return nullptr;
}

// Bytes from the first to one past the last element a rows x cols row-major view touches.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int eb) {
    if (rows == 0 || cols == 0) return 0;
    return ((rows - 1) * ld + cols) * eb;
}

// Tile choice: the largest tile that still gives at least one tile per compute unit (256 CUs,
// counting every product of a batch), else the smallest tile.  int8 and fp32 K-slabs are 128
// bytes like the 16-bit ones.
int choose_cfg(int64_t M, int64_t N, int64_t batch) {
    const int64_t cus = 256;
    const int sizes[tge::CFG_COUNT] = {256, 128, 64};
    for (int c = 0; c < tge::CFG_COUNT; ++c) {
        int64_t t = ((M + sizes[c] - 1) / sizes[c]) * ((N + sizes[c] - 1) / sizes[c]) *
                    (batch > 1 ? batch : 1);
        if (t >= cus) return c;
    }
    return tge::CFG_64;
}

}  // namespace

// A plan-owned workspace on the current device, allocated by the first run there that needs it
// (not while the stream is being captured into a graph).
static gemm_status_t lazy_workspace(void **ws, int *ws_dev, size_t bytes, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
    if (*ws && *ws_dev == dev) return GEMM_STATUS_SUCCESS;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
    if (cs != hipStreamCaptureStatusNone) return GEMM_STATUS_NOT_SUPPORTED;
    if (*ws) (void)hipFree(*ws);
    *ws = nullptr;
    *ws_dev = -1;
    if (hipMalloc(ws, bytes) != hipSuccess) {
        *ws = nullptr;
        (void)hipGetLastError();
        return GEMM_STATUS_ALLOC_FAILED;
    }
    *ws_dev = dev;
    return GEMM_STATUS_SUCCESS;
}

// ---- scratch of gemm_run_noalloc -------------------------------------------------------------
// One array per device, loaded with the library's code object and held until the process ends.
// Host code never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[GEMM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` on each device (nullptr: not yet)
}  // namespace

// Device address of the scratch array on the current device (resolved on the first call there).
static gemm_status_t scratch_address(uint8_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return GEMM_STATUS_HIP_ERROR;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return GEMM_STATUS_HIP_ERROR;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return GEMM_STATUS_SUCCESS;
}

// Scratch of gemm_run_noalloc: a bump allocator over the library's static device array (see
// below).  dry: a sizing pass that takes regions and skips every launch and memory access.
// Whether a transposed copy of A (stored transposed, B not) into K-contiguous rows repays its
// cost when A could be read in place.  The copy moves 2 * M * K elements through HBM; the
// kernel of the non-transposed layout saves up to ~10 % of the product's time, which grows with
// N as well, so the copy pays from a wide enough N.  Measured (copy and product, graph-timed):
// bf16 5000^3 284 -> 252 us, fp16 8192^3 827 -> 758 us, fp16 4096^3 114 -> 112 us, but fp16
// 4096 x 2048 x 4096 85 -> 87 us and 8192 x 1536 x 8192 171 -> 231 us; int8 4096^3 no change.
constexpr int64_t KMAJOR_MIN_N_BYTES = 6144;
constexpr int64_t FAST128_MAX_T256 = 128;
constexpr int64_t SHORT_M_MIN_CHUNK = 4;
constexpr int64_t SPLIT128_MIN_SLABS = 48;
static bool kmajor_pays(int64_t M, int64_t N, int64_t K, int eab) {
    (void)M; (void)K;
    return N * eab >= KMAJOR_MIN_N_BYTES;
}

// Whether the 128x128 tiles of the fast kernel beat the 256x256 ones: when the 256-wide tiles
// would leave at least half of the 256 CUs idle.  They beat the general kernel at every size
// measured, down to 16 workgroups.  Measured (fp16 NN, graph-timed): 512^3 general 10.3 us ->
// 7.0 us, 768^3 13.8 -> 8.4, 256 x 1024 x 4096 56.8 -> 24.9, 1024^3 18.0 -> 9.9, 1536^3
// 30.4 -> 18.6, 2048^3 fast 256 41.0 -> 25.5, 4096 x 2048 x 2048 42.8 -> 35.0; but 3072^3 (144
// wide tiles) 58.6 -> 74.7.
static bool fast128_pays(int64_t M, int64_t N, int64_t nprod) {
    const int64_t nb = nprod > 1 ? nprod : 1;
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256) * nb;
    return t256 <= FAST128_MAX_T256;
}

// Whether the 128x128 tiles on aligned copies of the operands (an extra pass over them, one
// more kernel) beat the general kernel reading them in place: from about 2^31 multiply-adds.
// Measured (fp16 NN, odd leading dimensions, graph-timed; general -> copies and 128-wide tiles):
// 1024^3 17.8 vs 18.6 us, 1280^3 26.9 -> 25.6, 1536^3 33.5 -> 27.9, 2048^3 50.6 -> 35.5.
constexpr double COPY128_MIN_MACS = 2147483648.0;
static bool copy128_pays(int64_t M, int64_t N, int64_t K, int64_t nprod) {
    return (double)M * (double)N * (double)K * (double)(nprod > 1 ? nprod : 1) >= COPY128_MIN_MACS;
}

// Whether a product with fewer 128x128 tiles than CUs (M > 64, and shorter ones the skinny
// kernel cannot take: below) takes those tiles with K split rather than the 256x256 ones with their finer split or the
// 128x128 tiles unsplit: from 48 slabs of K.  Measured (fp16 NN unless noted, graph-timed;
// 256-wide split -> 128-wide split): 96 x 4096 x 4096 27.3 -> 17.0 us, 128 x 4096 x 4096
// 28.3 -> 18.2, 256 x 4096 x 4096 35.8 -> 23.0, 128 x 8192 x 8192 45.1 -> 36.2, 256 x 14336 x
// 4096 53.8 -> 46.8, 1024^2 x 8192 39.4 -> 31.5, 1024 x 2048 x 8192 55.1 -> 51.9; (unsplit
// 128-wide -> split) 256 x 1024 x 4096 25.0 -> 18.5, 512^2 x 8192 71.5 -> 21.2, 288 x 416 x
// 7168 72.6 -> 16.5, 640^2 x 4096 41.8 -> 18.5, 1024^2 x 4096 41.1 -> 23.8, 2048 x 1024 x 4096
// 40.1 -> 32.8, 768^2 x 3072 32.2 -> 20.9, 1024^2 x 3072 32.8 -> 23.5, bf16 -> fp32 1024^2 x
// 8192 73.2 -> 32.2, int8 512^2 x 6144 20.1 -> 16.6; 256 x 2048 x 3072 is the one 48-slab
// case measured slower (19.9 vs 20.5 us).  At 32 slabs the results are mixed (128 x 4096 x
// 2048 15.0 vs 18.8 us, 640^2 x 2048 14.7 vs 16.2; 1024^2 x 2048 23.0 vs 21.3): unsplit.
// Exactly one 128x128 tile per CU splits in two (two workgroups per CU) from 64 slabs, where the
// 256-wide tiles' split would cut chunks shorter than 32 slabs: 2048^2 x 4096 56.7 -> 50.5 us
// (256-wide split 4 ways), bf16 -> fp32 55.0 -> 48.3, int8 2048^2 x 8192 56.0 -> 49.2; from 128
// slabs even (2048^2 x 8192 76.5 vs 76.1: the 256-wide split stays); at 48 slabs unsplit
// (2048^2 x 3072 37.2 vs 41.3), and with more tiles the 256-wide tiles stay ahead (2048 x 3072 x
// 4096 65.6 vs 74.5).
// Short products (M <= 64) the skinny kernel cannot take (int8 inputs, or A transposed) split
// from 8 slabs, as they did on the 256-wide tiles: 256-wide split -> 128-wide split, int8 16 x
// 4096 x 4096 17.1 -> 10.2 us, 64 x 8192 x 4096 NT 24.9 -> 16.0, 32 x 4096 x 8192 NT 21.2 ->
// 13.7, 16 x 4096 x 1024 14.1 -> 8.8; fp16 16 x 4096 x 4096 TN 26.7 -> 13.8, 32 x 1024 x 1024
// TN 18.6 -> 8.6; bf16 -> fp32 64 x 8192 x 4096 TT 30.4 -> 21.1.
static bool split128_pays(int64_t M, int64_t N, int64_t slabs, bool skinny_cannot) {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (M <= 64) return skinny_cannot && t128 < 256 && slabs >= 8;
    return (t128 < 256 && slabs >= SPLIT128_MIN_SLABS) || (t128 == 256 && slabs >= 64 && slabs < 128);
}

struct Scratch {
    uint8_t *base;
    size_t cap, used;
    bool dry;
};

// `bytes` of workspace for one run: from the scratch when there is one (SCRATCH_LIMIT when it
// is too small), else the plan-owned buffer *ws allocated on first use (lazy_workspace).
static gemm_status_t workspace(Scratch *sc, void **ws, int *ws_dev, size_t bytes, hipStream_t stream,
                               void **out) {
    if (!sc) {
        const gemm_status_t st = lazy_workspace(ws, ws_dev, bytes, stream);
        *out = st == GEMM_STATUS_SUCCESS ? *ws : nullptr;
        return st;
    }
    const size_t off = (sc->used + 255) & ~(size_t)255;
    if (off > sc->cap || bytes > sc->cap - off) return GEMM_STATUS_SCRATCH_LIMIT;
    sc->used = off + bytes;
    // the sizing pass never dereferences or launches with the region
    *out = sc->dry ? reinterpret_cast<void *>((uintptr_t)0x100 + off) : sc->base + off;
    return GEMM_STATUS_SUCCESS;
}

static bool launched(Scratch *sc, hipError_t (*fn)(const GemmParams &, hipStream_t), const GemmParams &prm,
                     hipStream_t s) {
    return (sc && sc->dry) || fn(prm, s) == hipSuccess;
}

// One run of plan p: validation, kernel choice per run, launches.  Workspaces come from the
// plan (gemm_run: allocated on first use, optional ones skipped when they cannot be had) or
// from the scratch (gemm_run_noalloc: every region the plan's route needs, or SCRATCH_LIMIT).
static gemm_status_t run_impl(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                              const void *bias, float alpha, float beta, void *stream, Scratch *sc) {
    if (!p) return GEMM_STATUS_INVALID_VALUE;
    if (p->M == 0 || p->N == 0 || p->batch == 0) return GEMM_STATUS_SUCCESS;
    const bool has_bias = p->epi == GEMM_EPI_BIAS || p->epi == GEMM_EPI_BIAS_RELU;
    const bool relu = p->epi == GEMM_EPI_RELU || p->epi == GEMM_EPI_BIAS_RELU;
    if (!D) return GEMM_STATUS_INVALID_VALUE;
    if (p->K > 0 && (!A || !B)) return GEMM_STATUS_INVALID_VALUE;
    if (beta != 0.0f && !C) return GEMM_STATUS_INVALID_VALUE;
    if (has_bias && !bias) return GEMM_STATUS_INVALID_VALUE;
    if (p->ab == GEMM_I8 && (alpha != 1.0f || (beta != 0.0f && beta != 1.0f)))
        return GEMM_STATUS_NOT_SUPPORTED;
    if (alpha != alpha || beta != beta) return GEMM_STATUS_INVALID_VALUE;  // NaN scalars
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool dry = sc && sc->dry;

    // operands stored as fp32 or int8: convert them into 16-bit rows of the workspace, then run
    // the plan on the converted rows (the conversion needs its workspace: a first run inside a
    // stream capture returns NOT_SUPPORTED, as a failed allocation returns ALLOC_FAILED)
    if (p->cv) {
        if (p->K == 0) return run_impl(p->cv, A, B, C, D, bias, alpha, beta, stream, sc);
        void *w = nullptr;
        const gemm_status_t st = workspace(sc, &p->cv_ws, &p->cv_dev, (size_t)p->cv_bytes, hs, &w);
        if (st != GEMM_STATUS_SUCCESS) return st;
        uint8_t *ws = static_cast<uint8_t *>(w);
        const int to_bf16 = p->ab == GEMM_BF16 ? 1 : 0;
        const auto src_bytes = [](int src) { return src == tge::CONVERT_FROM_F32 ? 4 : 1; };
        tge::ConvertJob ja = {}, jb = {};
        if (p->cv_src_a >= 0) {
            const int sb = src_bytes(p->cv_src_a);
            const int64_t na = p->batch > 1 && p->stride_a ? p->batch : 1;
            ja = {static_cast<const uint8_t *>(A), ws, p->cv_rows_a, p->cv_len_a, p->lda * sb,
                  p->cv_ld_a * 2, p->stride_a * sb, p->cv_rows_a * p->cv_ld_a * 2, na, p->cv_src_a, to_bf16};
        }
        if (p->cv_src_b >= 0) {
            const int sb = src_bytes(p->cv_src_b);
            const int64_t nbb = p->batch > 1 && p->stride_b ? p->batch : 1;
            jb = {static_cast<const uint8_t *>(B), ws + p->cv_off_b, p->cv_rows_b, p->cv_len_b,
                  p->ldb * sb, p->cv_ld_b * 2, p->stride_b * sb, p->cv_rows_b * p->cv_ld_b * 2, nbb,
                  p->cv_src_b, to_bf16};
        }
        if (!dry && tge::convert_launch(ja, jb, hs) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
        return run_impl(p->cv, p->cv_src_a >= 0 ? ws : A, p->cv_src_b >= 0 ? ws + p->cv_off_b : B, C, D,
                        bias, alpha, beta, stream, sc);
    }

    // complex / dual product as a real one: rewrite B (and a transposed A) into the workspace,
    // then run the real plan; without a plan-owned workspace (first run inside a capture, or no
    // memory) the complex kernel below runs instead
    void *cxw = nullptr;
    if (p->cx) {
        const gemm_status_t st = workspace(sc, &p->cx_ws, &p->cx_dev, (size_t)p->cx_bytes, hs, &cxw);
        if (sc && st != GEMM_STATUS_SUCCESS) return st;
    }
    if (p->cx && cxw) {
        const bool dual = p->ab == GEMM_DF16;
        uint8_t *ws = static_cast<uint8_t *>(cxw);
        const int64_t na = p->batch > 1 && p->stride_a ? p->batch : 1;
        const int64_t nbb = p->batch > 1 && p->stride_b ? p->batch : 1;
        tge::PairJob ja = {}, jb = {};
        const void *Ar = A;
        if (p->op_a == GEMM_OP_T) {
            ja = {static_cast<const uint8_t *>(A), ws, p->K, p->M, p->lda * 4, p->cx_ld_a * 2,
                  p->stride_a * 4, 2 * p->K * p->cx_ld_a * 2, na, tge::PAIR_PARTS, dual};
            Ar = ws;
        }
        const bool bn = p->op_b == GEMM_OP_N;
        const int64_t rows_b = bn ? p->K : p->N;
        jb = {static_cast<const uint8_t *>(B), ws + p->cx_off_b, rows_b, bn ? p->N : p->K, p->ldb * 4,
              p->cx_ld_b * 2, p->stride_b * 4, 2 * rows_b * p->cx_ld_b * 2, nbb,
              bn ? tge::PAIR_BLOCK_N : tge::PAIR_BLOCK_T, dual};
        if (!dry && tge::pair_launch(ja, jb, hs) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
        return run_impl(p->cx, Ar, ws + p->cx_off_b, C, D, nullptr, alpha, beta, stream, sc);
    }

    GemmParams prm;
    prm.A = A; prm.B = B; prm.C = C; prm.D = D; prm.bias = bias;
    prm.M = (int)p->M; prm.N = (int)p->N; prm.K = (int)p->K;
    prm.lda = (int)p->lda; prm.ldb = (int)p->ldb; prm.ldc = (int)p->ldc;
    prm.alpha = alpha; prm.beta = beta;
    prm.has_beta = beta != 0.0f;
    prm.has_bias = has_bias;
    prm.relu = relu;
    prm.group_m = p->group_m;
    prm.batch = (int)(p->batch * p->batch2);   // every product of both batch modes
    prm.batch2 = (int)p->batch2;
    prm.stride2_a = p->stride2_a; prm.stride2_b = p->stride2_b;
    prm.stride2_c = p->stride2_c; prm.stride2_bias = p->stride2_bias;
    prm.xform_a = p->xform_a; prm.xform_b = p->xform_b; prm.xform_c = p->xform_c;
    prm.stride_a = p->stride_a; prm.stride_b = p->stride_b;
    prm.stride_c = p->stride_c; prm.stride_bias = p->stride_bias;
    const KernelEntry *k = p->kernel;
    // Kernel choice per run.  The direct-load fast kernel reads an operand in place when its
    // rows are on the 16-byte grid (pointer included) and it carries no load transform.  Other
    // operands are copied first (aligned rows, the transform applied by the copy) when the plan
    // repacks and its workspace exists or can be had now.  Otherwise the fast kernel with fused
    // transforms (aligned operands), the register-staged variant, or the general kernel runs.
    const int kk = p->K > 0 ? 3 : 0;
    const int unaligned = (p->pk_need | (((uintptr_t)A % 16) ? 1 : 0) | (((uintptr_t)B % 16) ? 2 : 0)) & kk;
    const int xf = ((p->xform_a ? 1 : 0) | (p->xform_b ? 2 : 0)) & kk;
    int need = unaligned | (p->fast_pk && !p->fast_is_skinny ? xf : 0);
    // A stored transposed (B not) is copied transposed, which reads A element by element: its
    // pointer must be on the element grid (else that copy cannot be made)
    const int eab = elem_bytes(p->ab);
    const bool tr_ok = p->pk_tr && ((uintptr_t)A % eab) == 0;
    if (p->fast_pk && tr_ok && (p->pk_want & kk & ~need)) {
        // the copy made by choice, only where its workspace can be had (the scratch: if it fits)
        bool fits = true;
        if (sc) {
            const size_t off = (sc->used + 255) & ~(size_t)255;
            fits = off <= sc->cap && (size_t)p->pk_bytes <= sc->cap - off;
        }
        if (fits) need |= p->pk_want & kk;
    }
    const bool a_tr = p->pk_tr && (need & 1);
    void *pkw = nullptr;
    if (!(p->fast && !need) && p->fast_pk && need && (!a_tr || tr_ok)) {
        const gemm_status_t st = workspace(sc, &p->pk_ws, &p->pk_dev, (size_t)p->pk_bytes, hs, &pkw);
        if (sc && st != GEMM_STATUS_SUCCESS) return st;
    }
    if (p->fast && !need) k = p->fast;
    else if (pkw) {
        const bool sh_a = p->batch > 1 && p->stride_a, sh_b = p->batch > 1 && p->stride_b;
        tge::RepackJob ja = {}, jb = {};
        uint8_t *ws = static_cast<uint8_t *>(pkw);
        // stored rows of the copies: K-major operands get pk_kpad rows, the extra ones zero
        if (a_tr) {
            // K source rows of M elements -> M rows of pk_kpad elements (zero past K)
            ja = {static_cast<const uint8_t *>(A), ws, p->K, p->pk_kpad, p->M * eab, p->lda * eab,
                  p->pk_ld_a * eab, p->stride_a * eab, p->M * p->pk_ld_a * eab, sh_a ? p->batch : 1,
                  p->xform_a ? eab : 0, eab};
            prm.xform_a = 0;
            prm.A = ws;
            prm.lda = (int)p->pk_ld_a;
            prm.stride_a = sh_a ? p->M * p->pk_ld_a : 0;
        } else if (need & 1) {
            const bool an = p->op_a == GEMM_OP_N;
            const int64_t rows = an ? p->M : p->K, rows_out = an ? p->M : p->pk_kpad;
            const int64_t len = an ? p->K : p->M;
            ja = {static_cast<const uint8_t *>(A), ws, rows, rows_out, len * eab, p->lda * eab,
                  p->pk_ld_a * eab, p->stride_a * eab, rows_out * p->pk_ld_a * eab, sh_a ? p->batch : 1,
                  p->xform_a ? eab : 0, 0};
            prm.xform_a = 0;
            prm.A = ws;
            prm.lda = (int)p->pk_ld_a;
            prm.stride_a = sh_a ? rows_out * p->pk_ld_a : 0;
        }
        if (need & 2) {
            const bool bn = p->op_b == GEMM_OP_N;
            const int64_t rows = bn ? p->K : p->N, rows_out = bn ? p->pk_kpad : p->N;
            const int64_t len = bn ? p->N : p->K;
            jb = {static_cast<const uint8_t *>(B), ws + p->pk_off_b, rows, rows_out, len * eab,
                  p->ldb * eab, p->pk_ld_b * eab, p->stride_b * eab, rows_out * p->pk_ld_b * eab,
                  sh_b ? p->batch : 1, p->xform_b ? eab : 0, 0};
            prm.xform_b = 0;
            prm.B = ws + p->pk_off_b;
            prm.ldb = (int)p->pk_ld_b;
            prm.stride_b = sh_b ? rows_out * p->pk_ld_b : 0;
        }
        if (!dry && tge::repack_launch(ja, jb, hs) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
        // both operands from the copies: the products past K are 0 * 0, no tail slab
        if (need == 3) prm.K = (int)p->pk_kpad;
        k = a_tr ? p->fast_pk_tr : p->fast_pk;
    } else if (p->fast && !unaligned) {
        k = p->fast;              // no workspace: the direct loads with the transforms fused
    } else if (p->fast_rs) {
        k = p->fast_rs;
    }
    const bool sk = k == p->fast && p->fast_is_skinny;
    prm.tiles_m = sk ? p->ksplit : (int)((p->M + k->bm - 1) / k->bm);
    prm.tiles_n = (int)((p->N + k->bn - 1) / k->bn);
    prm.ws = nullptr;
    // split-K partial sums: batch * S * M * N floats (int32 for int8)
    const size_t split_bytes = (size_t)(p->batch * p->batch2 > 1 ? p->batch * p->batch2 : 1) * p->ksplit * p->M * p->N *
                               sizeof(float);
    // fast kernel with K split (needs its workspace; a first run inside a capture runs whole)
    void *spw = nullptr;
    const bool k_tr = p->fast_pk_tr && k == p->fast_pk_tr;   // A from its transposed copy
    // the partial products' kernel: the same tiles and layout as the kernel chosen above
    const KernelEntry *part_k = k->bm == 128 ? (k_tr ? p->fast_part128_tr : p->fast_part128)
                                             : k_tr ? p->fast_part_tr : p->fast_part;
    if ((k == p->fast || k == p->fast_pk || k_tr) && !sk && part_k) {
        const gemm_status_t st = workspace(sc, reinterpret_cast<void **>(&p->ws), &p->ws_dev, split_bytes, hs, &spw);
        if (sc && st != GEMM_STATUS_SUCCESS) return st;
    }
    if (spw) {
        const int S = p->ksplit;
        const int kc = (int)(p->K / S);                  // K of one chunk (whole slabs)
        GemmParams part = prm;
        part.K = kc;
        part.batch = S;
        part.batch2 = 1;
        part.stride2_a = part.stride2_b = part.stride2_c = part.stride2_bias = 0;
        // chunk offsets in the operands the kernel reads (the copies, when copied)
        part.stride_a = p->op_a == GEMM_OP_N || k_tr ? kc : (int64_t)kc * prm.lda;
        part.stride_b = p->op_b == GEMM_OP_N ? (int64_t)kc * prm.ldb : kc;
        part.C = nullptr;
        part.D = spw;
        part.bias = nullptr;
        part.alpha = 1.0f;
        part.beta = 0.0f;
        part.has_beta = 0;
        part.has_bias = 0;
        part.relu = 0;
        part.xform_c = 0;
        part.ldc = (int)p->N;
        part.stride_c = p->M * p->N;
        part.stride_bias = 0;
        const unsigned g1 = (unsigned)((int64_t)prm.tiles_m * prm.tiles_n * S);
        if (!dry && part_k->launch(part, g1, hs) != hipSuccess) return GEMM_STATUS_HIP_ERROR;
        GemmParams fin = prm;
        fin.tiles_m = S;
        fin.ws = static_cast<float *>(spw);
        return launched(sc, p->finish, fin, hs) ? GEMM_STATUS_SUCCESS : GEMM_STATUS_HIP_ERROR;
    }
    if (sk && p->ksplit > 1) {
        void *w = nullptr;
        const gemm_status_t st = workspace(sc, reinterpret_cast<void **>(&p->ws), &p->ws_dev, split_bytes, hs, &w);
        if (st != GEMM_STATUS_SUCCESS) return st;
        prm.ws = static_cast<float *>(w);
    }
    if (dry) return GEMM_STATUS_SUCCESS;
    const unsigned grid = (unsigned)((int64_t)prm.tiles_m * prm.tiles_n * p->batch * p->batch2);
    hipError_t e = k->launch(prm, grid, hs);
    return e == hipSuccess ? GEMM_STATUS_SUCCESS : GEMM_STATUS_HIP_ERROR;
}

extern "C" {

const char *gemm_status_string(gemm_status_t s) {
    switch (enum_bits(s)) {
    case GEMM_STATUS_SUCCESS: return "GEMM_STATUS_SUCCESS";
    case GEMM_STATUS_INVALID_VALUE: return "GEMM_STATUS_INVALID_VALUE";
    case GEMM_STATUS_NOT_SUPPORTED: return "GEMM_STATUS_NOT_SUPPORTED";
    case GEMM_STATUS_HIP_ERROR: return "GEMM_STATUS_HIP_ERROR";
    case GEMM_STATUS_ALLOC_FAILED: return "GEMM_STATUS_ALLOC_FAILED";
    case GEMM_STATUS_SCRATCH_LIMIT: return "GEMM_STATUS_SCRATCH_LIMIT";
    }
    return "GEMM_STATUS_UNKNOWN";
}

// The description of gemm_plan_create(_batched)'s arguments; the enum arguments are taken by
// reference and copied through their bits (they are checked by gemm_plan_create_desc).
static gemm_status_t create_from_args(gemm_plan_t *out, int64_t M, int64_t N, int64_t K, const gemm_op_t &op_a,
                                      const gemm_op_t &op_b, int64_t lda, int64_t ldb, int64_t ldc,
                                      const gemm_dtype_t &ab_type, const gemm_dtype_t &cd_type,
                                      const gemm_epilogue_t &epi, int64_t batch, int64_t stride_a,
                                      int64_t stride_b, int64_t stride_c, int64_t stride_bias) {
    gemm_desc_t d;
    d.M = M; d.N = N; d.K = K;
    copy_enum(d.op_a, op_a);
    copy_enum(d.op_b, op_b);
    d.lda = lda; d.ldb = ldb; d.ldc = ldc;
    copy_enum(d.ab_type, ab_type);
    copy_enum(d.cd_type, cd_type);
    copy_enum(d.epilogue, epi);
    d.batch = batch;
    d.stride_a = stride_a; d.stride_b = stride_b; d.stride_c = stride_c; d.stride_bias = stride_bias;
    d.transform_a = d.transform_b = d.transform_c = GEMM_TRANSFORM_NONE;
    d.kind_a = d.kind_b = GEMM_OPERAND_DENSE;
    d.algo = GEMM_ALGO_AUTO;
    d.tile = 0;
    d.batch2 = 1;
    d.stride2_a = d.stride2_b = d.stride2_c = d.stride2_bias = 0;
    return gemm_plan_create_desc(out, &d);
}

gemm_status_t gemm_plan_create(gemm_plan_t *out, int64_t M, int64_t N, int64_t K, gemm_op_t op_a,
                               gemm_op_t op_b, int64_t lda, int64_t ldb, int64_t ldc,
                               gemm_dtype_t ab_type, gemm_dtype_t cd_type, gemm_epilogue_t epi) {
    return create_from_args(out, M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epi, 1, 0, 0, 0, 0);
}

gemm_status_t gemm_plan_create_batched(gemm_plan_t *out, int64_t M, int64_t N, int64_t K,
                                       gemm_op_t op_a, gemm_op_t op_b, int64_t lda, int64_t ldb,
                                       int64_t ldc, gemm_dtype_t ab_type, gemm_dtype_t cd_type,
                                       gemm_epilogue_t epi, int64_t batch, int64_t stride_a,
                                       int64_t stride_b, int64_t stride_c, int64_t stride_bias) {
    return create_from_args(out, M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epi, batch, stride_a,
                            stride_b, stride_c, stride_bias);
}

gemm_status_t gemm_plan_create_desc(gemm_plan_t *out, const gemm_desc_t *desc) {
    if (!out) return GEMM_STATUS_INVALID_VALUE;
    *out = nullptr;
    if (!desc) return GEMM_STATUS_INVALID_VALUE;
    // every enum field in range (checked through its bits) before it is read as an enum
    {
        const auto in = [](int v, int lo, int hi) { return v >= lo && v <= hi; };
        if (!in(enum_bits(desc->op_a), GEMM_OP_N, GEMM_OP_T) || !in(enum_bits(desc->op_b), GEMM_OP_N, GEMM_OP_T) ||
            !in(enum_bits(desc->ab_type), GEMM_F32, GEMM_DF32) || !in(enum_bits(desc->cd_type), GEMM_F32, GEMM_DF32) ||
            !in(enum_bits(desc->epilogue), GEMM_EPI_NONE, GEMM_EPI_BIAS_RELU) ||
            !in(enum_bits(desc->transform_a), GEMM_TRANSFORM_NONE, GEMM_TRANSFORM_FROM_I8) ||
            !in(enum_bits(desc->transform_b), GEMM_TRANSFORM_NONE, GEMM_TRANSFORM_FROM_I8) ||
            !in(enum_bits(desc->transform_c), GEMM_TRANSFORM_NONE, GEMM_TRANSFORM_RELU) ||
            !in(enum_bits(desc->kind_a), GEMM_OPERAND_DENSE, GEMM_OPERAND_DIAGONAL) ||
            !in(enum_bits(desc->kind_b), GEMM_OPERAND_DENSE, GEMM_OPERAND_DIAGONAL) ||
            !in(enum_bits(desc->algo), GEMM_ALGO_AUTO, GEMM_ALGO_FAST_KMAJOR))
            return GEMM_STATUS_INVALID_VALUE;
    }
    const int64_t M = desc->M, N = desc->N, K = desc->K;
    const gemm_op_t op_a = desc->op_a, op_b = desc->op_b;
    const int64_t lda = desc->lda, ldb = desc->ldb, ldc = desc->ldc;
    const gemm_dtype_t ab_type = desc->ab_type, cd_type = desc->cd_type;
    const gemm_epilogue_t epi = desc->epilogue;
    const int64_t batch = desc->batch;
    int64_t stride_a = desc->stride_a, stride_b = desc->stride_b, stride_c = desc->stride_c,
            stride_bias = desc->stride_bias;
    // second batch mode: 0 or 1 means none
    if (desc->batch2 < 0 || desc->stride2_a < 0 || desc->stride2_b < 0 || desc->stride2_c < 0 ||
        desc->stride2_bias < 0)
        return GEMM_STATUS_INVALID_VALUE;
    const int64_t batch2 = desc->batch2 > 1 ? desc->batch2 : 1;
    int64_t stride2_a = desc->stride2_a, stride2_b = desc->stride2_b, stride2_c = desc->stride2_c,
            stride2_bias = desc->stride2_bias;
    if (batch2 <= 1) stride2_a = stride2_b = stride2_c = stride2_bias = 0;
    // products of both modes
    const int64_t nprod = batch * batch2;
    for (gemm_transform_t t : {desc->transform_a, desc->transform_b})
        if ((int)t < GEMM_TRANSFORM_NONE || (int)t > GEMM_TRANSFORM_FROM_I8) return GEMM_STATUS_INVALID_VALUE;
    // C has the type of D: no conversion on C
    if ((int)desc->transform_c != GEMM_TRANSFORM_NONE && (int)desc->transform_c != GEMM_TRANSFORM_RELU)
        return GEMM_STATUS_INVALID_VALUE;
    const auto converts = [](gemm_transform_t t) {
        return t == GEMM_TRANSFORM_FROM_F32 || t == GEMM_TRANSFORM_FROM_I8;
    };
    const bool cva = converts(desc->transform_a), cvb = converts(desc->transform_b);
    for (gemm_operand_t k : {desc->kind_a, desc->kind_b})
        if ((int)k != GEMM_OPERAND_DENSE && (int)k != GEMM_OPERAND_DIAGONAL) return GEMM_STATUS_INVALID_VALUE;
    if ((int)desc->algo < GEMM_ALGO_AUTO || (int)desc->algo > GEMM_ALGO_FAST_KMAJOR) return GEMM_STATUS_INVALID_VALUE;
    if (desc->tile != 0 && desc->tile != 256 && desc->tile != 128 && desc->tile != 64)
        return GEMM_STATUS_INVALID_VALUE;
    const bool diag_a = desc->kind_a == GEMM_OPERAND_DIAGONAL;
    const bool diag_b = desc->kind_b == GEMM_OPERAND_DIAGONAL;
    if ((diag_a && K != M) || (diag_b && K != N)) return GEMM_STATUS_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
    if (batch < 0 || stride_a < 0 || stride_b < 0 || stride_c < 0 || stride_bias < 0)
        return GEMM_STATUS_INVALID_VALUE;
    if ((op_a != GEMM_OP_N && op_a != GEMM_OP_T) || (op_b != GEMM_OP_N && op_b != GEMM_OP_T))
        return GEMM_STATUS_INVALID_VALUE;
    if ((int)ab_type < GEMM_F32 || (int)ab_type > GEMM_DF32 || (int)cd_type < GEMM_F32 ||
        (int)cd_type > GEMM_DF32)
        return GEMM_STATUS_INVALID_VALUE;
    if ((int)epi < GEMM_EPI_NONE || (int)epi > GEMM_EPI_BIAS_RELU) return GEMM_STATUS_INVALID_VALUE;
    // minimum leading dimensions (stored row length), never below 1
    int64_t min_lda = op_a == GEMM_OP_N ? K : M;
    int64_t min_ldb = op_b == GEMM_OP_N ? N : K;
    // a diagonal operand has no leading dimension (its vector is contiguous)
    if ((!diag_a && lda < (min_lda > 1 ? min_lda : 1)) || (!diag_b && ldb < (min_ldb > 1 ? min_ldb : 1)) ||
        ldc < (N > 1 ? N : 1))
        return GEMM_STATUS_INVALID_VALUE;
    Lookup table = pair_table(ab_type, cd_type);
    ComplexLookup ctable = complex_table(ab_type, cd_type);
    if (!table && !ctable) return GEMM_STATUS_NOT_SUPPORTED;
    // complex and dual numbers: the plain product with real alpha/beta only
    if (ctable && (epi != GEMM_EPI_NONE || desc->transform_a || desc->transform_b || desc->transform_c ||
                   diag_a || diag_b))
        return GEMM_STATUS_NOT_SUPPORTED;
    // type-converting load transforms: 16-bit inputs, dense operands
    if ((cva || cvb) && ((ab_type != GEMM_F16 && ab_type != GEMM_BF16) || diag_a || diag_b))
        return GEMM_STATUS_NOT_SUPPORTED;
    // 32-bit offsets inside the kernels: every matrix must span less than 2^31 bytes (a
    // converted operand: in its stored type)
    const int64_t lim = (int64_t)1 << 31;
    int eab = elem_bytes(ab_type), ecd = elem_bytes(cd_type);
    const auto stored_bytes = [&](gemm_transform_t t) {
        return t == GEMM_TRANSFORM_FROM_F32 ? 4 : t == GEMM_TRANSFORM_FROM_I8 ? 1 : eab;
    };
    const int esa = stored_bytes(desc->transform_a), esb = stored_bytes(desc->transform_b);
    int64_t sa = diag_a ? K * esa : op_a == GEMM_OP_N ? span_bytes(M, K, lda, esa) : span_bytes(K, M, lda, esa);
    int64_t sb = diag_b ? K * esb : op_b == GEMM_OP_N ? span_bytes(K, N, ldb, esb) : span_bytes(N, K, ldb, esb);
    int64_t sc = span_bytes(M, N, ldc, ecd);
    if (sa >= lim || sb >= lim || sc >= lim || lda >= lim || ldb >= lim || ldc >= lim)
        return GEMM_STATUS_NOT_SUPPORTED;
    // products of a batch never write the same element of D: with one mode, consecutive D's at
    // least one D apart; with two, the modes nest (the smaller stride at least one D, the larger
    // at least the whole run of the smaller mode)
    const int64_t dspan = (M > 0 && N > 0) ? (M - 1) * ldc + N : 0;
    if (batch > 1 && batch2 > 1 && dspan > 0) {
        const bool in1 = stride_c <= stride2_c;   // mode 1 inner
        const int64_t si = in1 ? stride_c : stride2_c, ni = in1 ? batch : batch2;
        const int64_t so = in1 ? stride2_c : stride_c;
        if (si < dspan || so / ni < si) return GEMM_STATUS_INVALID_VALUE;
    } else if (batch > 1 && dspan > 0 && stride_c < dspan) {
        return GEMM_STATUS_INVALID_VALUE;
    } else if (batch2 > 1 && dspan > 0 && stride2_c < dspan) {
        return GEMM_STATUS_INVALID_VALUE;
    }
    if (batch <= 1) stride_a = stride_b = stride_c = stride_bias = 0;
    // the byte offset of the last product must fit in 63 bits
    const int64_t big = (int64_t)1 << 62;
    if (batch > 1 && (stride_a > big / batch / 8 || stride_b > big / batch / 8 ||
                      stride_c > big / batch / 8 || stride_bias > big / batch / 8))
        return GEMM_STATUS_NOT_SUPPORTED;
    if (batch2 > 1 && (stride2_a > big / batch2 / 8 || stride2_b > big / batch2 / 8 ||
                       stride2_c > big / batch2 / 8 || stride2_bias > big / batch2 / 8))
        return GEMM_STATUS_NOT_SUPPORTED;
    // the kernels index products with 32-bit ints
    if (nprod >= ((int64_t)1 << 31)) return GEMM_STATUS_NOT_SUPPORTED;

    if ((cva || cvb) && batch2 > 1) return GEMM_STATUS_NOT_SUPPORTED;
    if (cva || cvb) {
        // the product runs as a plan on the converted operands: 16-bit rows, pitch whole
        // 128-byte lines, one converted copy per product (one for all when the stride is 0)
        const int64_t rows_a = op_a == GEMM_OP_N ? M : K, len_a = op_a == GEMM_OP_N ? K : M;
        const int64_t rows_b = op_b == GEMM_OP_N ? K : N, len_b = op_b == GEMM_OP_N ? N : K;
        const int64_t ld_a = ((len_a > 1 ? len_a : 1) + 63) / 64 * 64, ld_b = ((len_b > 1 ? len_b : 1) + 63) / 64 * 64;
        const int64_t na = batch > 1 && stride_a ? batch : 1, nbb = batch > 1 && stride_b ? batch : 1;
        gemm_desc_t r = *desc;
        if (cva) {
            r.transform_a = GEMM_TRANSFORM_NONE;
            r.lda = ld_a;
            r.stride_a = na > 1 ? rows_a * ld_a : 0;
        }
        if (cvb) {
            r.transform_b = GEMM_TRANSFORM_NONE;
            r.ldb = ld_b;
            r.stride_b = nbb > 1 ? rows_b * ld_b : 0;
        }
        const int64_t bytes_a = cva ? na * rows_a * ld_a * 2 : 0;
        const int64_t off_b = (bytes_a + 255) / 256 * 256;
        const int64_t bytes = off_b + (cvb ? nbb * rows_b * ld_b * 2 : 0);
        // the conversion grid (workgroups of 4 rows x 512 elements) fits 31 bits
        const int64_t blocks = (cva ? (ld_a / 8 + 63) / 64 * ((rows_a + 3) / 4) * na : 0) +
                               (cvb ? (ld_b / 8 + 63) / 64 * ((rows_b + 3) / 4) * nbb : 0);
        if (blocks >= lim) return GEMM_STATUS_NOT_SUPPORTED;
        gemm_plan *inner = nullptr;
        const gemm_status_t st = gemm_plan_create_desc(&inner, &r);
        if (st != GEMM_STATUS_SUCCESS) return st;
        gemm_plan *p = new (std::nothrow) gemm_plan();
        if (!p) {
            gemm_plan_destroy(inner);
            return GEMM_STATUS_ALLOC_FAILED;
        }
        p->M = M; p->N = N; p->K = K;
        p->lda = lda; p->ldb = ldb; p->ldc = ldc;
        p->batch = batch;
        p->batch2 = 1;
        p->stride_a = stride_a; p->stride_b = stride_b; p->stride_c = stride_c; p->stride_bias = stride_bias;
        p->op_a = op_a; p->op_b = op_b; p->ab = ab_type; p->cd = cd_type; p->epi = epi;
        p->xform_a = desc->transform_a; p->xform_b = desc->transform_b; p->xform_c = desc->transform_c;
        p->kernel = inner->kernel;
        p->ws_dev = p->pk_dev = p->cx_dev = p->cv_dev = -1;
        p->ksplit = 1;
        p->cv = inner;
        p->cv_src_a = cva ? (desc->transform_a == GEMM_TRANSFORM_FROM_F32 ? tge::CONVERT_FROM_F32 : tge::CONVERT_FROM_I8) : -1;
        p->cv_src_b = cvb ? (desc->transform_b == GEMM_TRANSFORM_FROM_F32 ? tge::CONVERT_FROM_F32 : tge::CONVERT_FROM_I8) : -1;
        p->cv_rows_a = rows_a; p->cv_rows_b = rows_b;
        p->cv_len_a = len_a; p->cv_len_b = len_b;
        p->cv_ld_a = ld_a; p->cv_ld_b = ld_b;
        p->cv_off_b = off_b; p->cv_bytes = bytes;
        p->grid = inner->grid;
        const auto src_name = [](int src) { return src == tge::CONVERT_FROM_F32 ? "f32" : "i8"; };
        char conv[64] = "";
        int cl = 0;
        if (cva) cl += snprintf(conv + cl, sizeof(conv) - cl, " convert A from %s", src_name(p->cv_src_a));
        if (cvb) snprintf(conv + cl, sizeof(conv) - cl, " convert B from %s", src_name(p->cv_src_b));
        snprintf(p->desc, sizeof(p->desc), "%s%s", inner->desc, conv);
        *out = p;
        return GEMM_STATUS_SUCCESS;
    }

    int cfg = (diag_a || diag_b || ctable) ? tge::CFG_128 : choose_cfg(M, N, nprod);
    // an explicit tile in the description pins the workgroup tile
    const int tile = desc->tile;
    if (tile == 256) cfg = tge::CFG_256;
    else if (tile == 128) cfg = tge::CFG_128;
    else if (tile == 64) cfg = tge::CFG_64;
    const KernelEntry *k = ctable ? ctable(op_a, op_b) : table(op_a, op_b, cfg);
    if (diag_a || diag_b) k = diag_table(ab_type, cd_type)(op_a, op_b, (diag_a ? 1 : 0) | (diag_b ? 2 : 0));
    if (!k) return GEMM_STATUS_NOT_SUPPORTED;

    // fast path: 16-bit inputs, 256x256 tiles worth it, shape/ld preconditions of gemm_fast
    const KernelEntry *fast = nullptr;
    FastLookup ft = fast_table(ab_type, cd_type);
    // an explicit algorithm in the description (gemm_algo_t) overrides the choices below
    const int algo = desc->algo;
    const bool staged = algo == GEMM_ALGO_FAST_STAGED;
    // the plan's own choice of kernel and tile (GEMM_ALGO_NOSPLIT: the same without a K split)
    const bool own = algo == GEMM_ALGO_AUTO || algo == GEMM_ALGO_NOSPLIT;
    // the fast kernel does ~3x the work per CU-round of the general 128x128 kernel: take it
    // when its rounds of 256x256 tiles cost less than 3x as many rounds of 128x128 tiles
    const int64_t nb = nprod > 1 ? nprod : 1;
    const int64_t r256 = (((M + 255) / 256) * ((N + 255) / 256) * nb + 255) / 256;
    const int64_t r128 = (((M + 127) / 128) * ((N + 127) / 128) * nb + 255) / 256;
    bool want_fast = cfg == tge::CFG_256 || (cfg == tge::CFG_128 && 4 * r256 <= 3 * r128);
    if (tile) want_fast = cfg == tge::CFG_256;
    if (algo == GEMM_ALGO_FAST || algo == GEMM_ALGO_FAST_KMAJOR || staged) want_fast = true;
    // K split of the fast kernel: few 256x256 tiles and a long K (64 slabs or more: K >= 4096
    // for 16-bit inputs, 8192 for int8).  K is cut into S equal chunks of whole slabs (at least
    // 16 each) so that tiles x S workgroups fill the chip (at least 128); the chunks' partial
    // sums (fp32, int32 for int8) go to a workspace and the finishing kernel adds them in chunk
    // order and applies the epilogue.  One product, no load transforms.  Such a plan takes the
    // fast kernel even where the general one would otherwise run: measured 1.1-2.9x faster
    // from 64 slabs, slower at 2048^3 (32 slabs).  Short products the skinny kernel cannot take
    // (M <= 64 with int8 inputs, or with A transposed) split down to chunks of 2 slabs: their
    // partial sums are small, and the split measured 1.1-6x faster than the general kernel
    // (int8 16 x 4096 x 4096: 97 -> 17 us; fp16 TN: 135 -> 28 us), from 8 slabs of K
    // (GEMM_ALGO_SPLIT: any S >= 2, chunks of one slab or more; GEMM_ALGO_NOSPLIT: never).
    int split_s = 0;
    const bool force_split = algo == GEMM_ALGO_SPLIT;
    const int64_t slab_k = 128 / elem_bytes(ab_type);   // K elements per slab of the fast kernel
    const int part_cd = ab_type == GEMM_I8 ? GEMM_I32 : GEMM_F32;
    if ((ab_type == GEMM_F16 || ab_type == GEMM_BF16 || ab_type == GEMM_I8) && nprod <= 1 &&
        !ctable && !diag_a && !diag_b && !desc->transform_a && !desc->transform_b &&
        K % slab_k == 0 && !staged &&
        algo != GEMM_ALGO_NOSPLIT && algo != GEMM_ALGO_GENERAL && algo != GEMM_ALGO_SKINNY &&
        !(tile == 128 && (own || algo == GEMM_ALGO_FAST))) {
        const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
        const int64_t slabs = K / slab_k;
        int64_t sp = tiles > 0 ? 256 / tiles : 0;
        const bool short_i8 = M <= 64 && (ab_type == GEMM_I8 || op_a == GEMM_OP_T);
        // one row of 256-wide tiles: chunks down to 4 slabs (fp16 96 x 4096 x 4096: general
        // kernel 77 us, split 16 ways 28 us; 128 x 4096 x 4096 64 -> 29 us); with 16-bit inputs
        // read in place the 128-wide tiles' split below takes most of these products instead
        const bool short_m = M <= 256;
        const int64_t min_chunk = force_split ? 1 : short_i8 ? 2 : short_m ? SHORT_M_MIN_CHUNK : 16;
        if (sp > slabs / min_chunk) sp = slabs / min_chunk;
        while (sp > 1 && slabs % sp) --sp;
        // short products split only from 8 slabs of K: with 4 slabs the two chunks and the
        // finishing kernel measured slower than the general kernel (fp16 64 x 8192 x 256 TN
        // 21.8 vs 8.3 us, int8 64 x 8192 x 512 NT 16.8 vs 5.8 us); from 8 slabs faster (fp16
        // 32 x 1024 x 1024 TN 18.2 vs 34.9 us, int8 16 x 4096 x 1024 13.5 vs 26.4 us)
        const bool worth = force_split || (short_i8 && slabs >= 8) || (tiles * sp >= 128 && slabs >= 64);
        if (sp >= 2 && worth && fast_table(ab_type, part_cd) && finish_table(ab_type, cd_type))
            split_s = (int)sp;
    }
    if (split_s) want_fast = true;
    if (algo == GEMM_ALGO_GENERAL) want_fast = false;
    const int ve = 16 / eab;   // elements per 16-byte chunk
    // elements per 128-byte line: the pitch of every copy the plan makes.  Rows that start off
    // a line boundary cost the direct loads a second line per row and slab (~10 % of the loop
    // time of a 5000-square product), so copies never have them
    const int vl = 128 / eab;
    // every product of a batch keeps the 16-byte alignment of product 0
    const bool strides16 = (stride_a * eab) % 16 == 0 && (stride_b * eab) % 16 == 0 &&
                           (stride2_a * eab) % 16 == 0 && (stride2_b * eab) % 16 == 0 && !diag_a && !diag_b;
    const bool direct_ok = K >= 128 / eab && (lda * eab) % 16 == 0 && (ldb * eab) % 16 == 0 &&
                           strides16 && (op_a == GEMM_OP_N || M % ve == 0) && (op_b == GEMM_OP_T || N % ve == 0);
    if (ft && want_fast && direct_ok)
        fast = ft(op_a, op_b, 0);
    // 128x128 tiles of the fast kernel (operands read in place, no load transforms on
    // op(A)/op(B)), for products whose 256x256 tiles would leave most CUs idle;
    // an explicit tile of 128 with the fast or automatic algorithm pins it
    const Fast128Lookup f128t = fast128_table(ab_type, cd_type);
    const KernelEntry *fast128 = nullptr;
    if (f128t && direct_ok && !desc->transform_a && !desc->transform_b && !diag_a && !diag_b && !ctable &&
        algo != GEMM_ALGO_GENERAL && !split_s &&
        ((tile == 128 && (own || algo == GEMM_ALGO_FAST)) || (tile == 0 && own && fast128_pays(M, N, nprod))))
        fast128 = f128t(op_a, op_b);
    if (fast128) fast = fast128;
    // products with fewer 128x128 tiles than CUs and a long K (short ones the skinny kernel
    // cannot take from 8 slabs) on those tiles with K split over workgroups: t128 tiles times
    // S chunks (whole slabs, at least 4 each) of at most one workgroup per CU (more, and some
    // CUs run two while the rest idle: fp16 768^2 x 4096 S = 8 23.9 us, S = 4 20.8; 768^2 x
    // 3072 S = 8 22.6, S = 6 20.9; 640 x 896 x 4096 S = 8 22.6, S = 4 21.2); the partial sums
    // are S * M * N fp32 values (int32 for int8).  Operands the direct loads cannot read in
    // place: the same split on their aligned copies, settled with the copies below.
    int split128 = 0, split128_copy = 0;
    const Fast128Lookup f128p = fast128_table(ab_type, part_cd);
    const bool pin_split128 = tile == 128 && algo == GEMM_ALGO_SPLIT;
    if (f128t && f128p && M > 0 && N > 0 && K > 0 && nprod <= 1 && K % slab_k == 0 &&
        !desc->transform_a && !desc->transform_b && !diag_a && !diag_b && !ctable &&
        finish_table(ab_type, cd_type) &&
        (pin_split128 || (tile == 0 && algo == GEMM_ALGO_AUTO &&
                          split128_pays(M, N, K / slab_k, ab_type == GEMM_I8 || op_a == GEMM_OP_T)))) {
        const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
        const int64_t slabs = K / slab_k;
        int64_t sp = 256 / t128;
        if (sp < 2) sp = 2;
        if (sp > slabs / SHORT_M_MIN_CHUNK) sp = slabs / SHORT_M_MIN_CHUNK;
        while (sp > 1 && slabs % sp) --sp;
        if (sp >= 2 && direct_ok) {
            split128 = (int)sp;
            fast = fast128 = f128t(op_a, op_b);
            split_s = 0;
        } else if (sp >= 2) {
            split128_copy = (int)sp;
        }
    }
    // the same choice for copies of operands the direct loads cannot read in place (also those
    // of a pointer found off the 16-byte grid at run time), or that carry a load transform (the
    // copy applies it): the 128x128 tiles run on the copies, with their K split, or unsplit for
    // products large enough to repay the copy
    const bool want128 = f128t && !diag_a && !diag_b && !ctable && algo != GEMM_ALGO_GENERAL &&
                         (split128 || split128_copy ||
                          (!split_s && ((tile == 128 && (own || algo == GEMM_ALGO_FAST)) ||
                                        (tile == 0 && own && fast128_pays(M, N, nprod) &&
                                         copy128_pays(M, N, K, nprod)))));
    // the register-staged variant takes every layout the direct loads cannot (odd leading
    // dimensions or strides, unaligned pointers, M/N-contiguous extents off the 16-byte grid)
    const KernelEntry *fast_rs = nullptr;
    if (ft && want_fast && K >= 128 / eab && !diag_a && !diag_b && (op_a == GEMM_OP_N || M >= ve) &&
        (op_b == GEMM_OP_T || N >= ve))
        fast_rs = ft(op_a, op_b, 1);

    // repacking: operands the direct loads cannot read in place are copied into aligned rows
    // padded to whole 128-byte lines, then the direct-load kernel runs on the copies
    // (GEMM_ALGO_FAST_STAGED keeps the register-staged variant for such operands)
    const KernelEntry *fast_pk = nullptr, *fast_pk_tr = nullptr;
    int pk_need = 0, pk_want = 0;
    bool pk_tr = false;
    int64_t pk_ld_a = 0, pk_ld_b = 0, pk_off_b = 0, pk_bytes = 0, pk_kpad = 0;
    // (one batch mode only: the copies lay products out along one stride)
    if (ft && (want_fast || want128) && K >= 128 / eab && !diag_a && !diag_b && !staged && batch2 <= 1) {
        // the copies hold K rounded up to whole slabs, zero past K: when both operands are
        // copied the kernel runs on that K and needs no guarded tail slab
        const int64_t slab = 128 / eab;
        pk_kpad = (K + slab - 1) / slab * slab;
        // A stored transposed with B not is the one layout whose fast kernel reads both
        // operands with transposing LDS reads, which leaves the 16x16 schedule short of
        // registers (it runs the 32x32 one, 10-15 % slower).  A copy of A is then made
        // transposed, into K-contiguous rows, and the kernel of the non-transposed layout runs
        pk_tr = op_a == GEMM_OP_T && op_b == GEMM_OP_N && ft(GEMM_OP_N, op_b, 0) != nullptr;
        const bool an = op_a == GEMM_OP_N || pk_tr;
        const int64_t rows_a = an ? M : pk_kpad, len_a = an ? pk_kpad : M;
        const int64_t rows_b = op_b == GEMM_OP_N ? pk_kpad : N, len_b = op_b == GEMM_OP_N ? N : pk_kpad;
        pk_ld_a = (len_a + vl - 1) / vl * vl;
        pk_ld_b = (len_b + vl - 1) / vl * vl;
        // a batch stride of 0 shares the operand between products: one copy
        const int64_t na = batch > 1 && stride_a ? batch : 1, nbb = batch > 1 && stride_b ? batch : 1;
        const int64_t one_a = rows_a * pk_ld_a * eab, one_b = rows_b * pk_ld_b * eab;
        // an M/N-contiguous operand (A transposed, B not) must also be whole chunks wide
        const bool need_a = (lda * eab) % 16 != 0 || (stride_a * eab) % 16 != 0 ||
                            (op_a == GEMM_OP_T && M % ve != 0);
        const bool need_b = (ldb * eab) % 16 != 0 || (stride_b * eab) % 16 != 0 ||
                            (op_b == GEMM_OP_N && N % ve != 0);
        pk_need = (need_a ? 1 : 0) | (need_b ? 2 : 0);
        // an A that could be read in place is still copied, transposed, when the product is
        // large enough to repay the copy (GEMM_ALGO_FAST_KMAJOR: always; GEMM_ALGO_FAST: never)
        // (the 128x128 tiles run the 16x16 schedule on this layout in place)
        if (pk_tr && !need_a && (algo == GEMM_ALGO_FAST_KMAJOR ||
                                 (own && !fast128 && !want128 && kmajor_pays(M, N, K, eab))))
            pk_want = 1;
        // the copies obey the 32-bit offset limit of the kernels; the copy grid (workgroups of
        // 4 rows x 1 KiB) fits 31 bits
        auto blocks = [&](int64_t rows, int64_t ld, int64_t n) {
            return ((ld * eab + 1023) / 1024) * ((rows + 3) / 4) * n;
        };
        if (one_a < lim && one_b < lim && blocks(rows_a, pk_ld_a, na) + blocks(rows_b, pk_ld_b, nbb) < lim) {
            pk_off_b = (na * one_a + 255) / 256 * 256;
            pk_bytes = pk_off_b + nbb * one_b;
            fast_pk = want128 ? f128t(op_a, op_b) : ft(op_a, op_b, 0);
            if (pk_tr) fast_pk_tr = want128 ? f128t(GEMM_OP_N, op_b) : ft(GEMM_OP_N, op_b, 0);
            if (split128_copy && want128) {
                split128 = split128_copy;
                split_s = 0;
            }
        } else {
            pk_need = pk_want = 0;
            pk_tr = false;
        }
    }

    // skinny path: M <= 64, memory bound; preferred over both tiled kernels when it applies
    bool skinny = false;
    SkinnyLookup st = skinny_table(ab_type, cd_type);
    // int8 (B transposed) up to 32 rows: from 64 the 128x128 tiles' K split measured as fast
    // (int8 NT, cache-hot, skinny vs split: 16 x 4096 x 4096 8.3 vs 10.1 us, 16 x 4096 x 1024 4.1
    // vs 8.5, 32 x 4096 x 8192 12.7 vs 13.8, 5 x 1000 x 2048 6.7 vs 8.5, 16 x 16384 x 4096 15.8
    // vs 18.7; 64 x 8192 x 4096 16.8 vs 16.2, 64 x 1024 x 2048 9.7 vs 9.0)
    bool want_skinny = M <= (ab_type == GEMM_I8 ? 32 : 64);
    if (algo == GEMM_ALGO_GENERAL) want_skinny = false;
    if (algo == GEMM_ALGO_FAST || algo == GEMM_ALGO_FAST_KMAJOR || staged || force_split) want_skinny = false;
    if (algo == GEMM_ALGO_SKINNY) want_skinny = true;
    // (K in whole 64-byte chunks; int8 inputs with B transposed only)
    if (st && want_skinny && M >= 1 && M <= 64 && op_a == GEMM_OP_N && K % (64 / eab) == 0 &&
        (lda * eab) % 16 == 0 && (ldb * eab) % 16 == 0 && strides16 &&
        (op_b == GEMM_OP_T || (eab == 2 && N % 8 == 0))) {
        // B transposed, M <= 16: 16-column blocks when they make one round of 192 to 256
        // workgroups and the 64-column ones would need a k split (no partial sums, no second
        // kernel).  Each narrow block reads as many bytes of A as of B, so larger M, or a
        // second round, measured slower than the split.
        const int64_t nbk = nprod > 1 ? nprod : 1;
        const int64_t nblk = ((N + 15) / 16) * nbk;
        const bool narrow = op_b == GEMM_OP_T && M <= 16 && ((N + 63) / 64) * nbk < 256 &&
                            nblk >= 192 && nblk <= 256;
        const KernelEntry *sk = st(op_b, (int)((M + 15) / 16), narrow ? 1 : 0);
        if (sk) {
            fast = sk;
            skinny = true;
        }
    }

    // complex and dual numbers where the real fast kernels apply: the product as a real fp16
    // GEMM M x 2N x 2K.  op(A) read as M x 2K reals is A itself when not transposed (parts
    // interleaved along K), else A's rows split into parts; every number of op(B) becomes a
    // 2 x 2 block (PairJob).  Elsewhere the complex kernel runs.
    gemm_plan *cx = nullptr;
    int64_t cx_ld_a = 0, cx_ld_b = 0, cx_off_b = 0, cx_bytes = 0;
    if (ctable && M > 0 && N > 0 && K > 0 && algo != GEMM_ALGO_GENERAL && batch2 <= 1) {
        gemm_desc_t r = *desc;
        r.N = 2 * N;
        r.K = 2 * K;
        cx_ld_a = op_a == GEMM_OP_N ? 2 * lda : (M + 63) / 64 * 64;
        cx_ld_b = op_b == GEMM_OP_N ? (2 * N + 63) / 64 * 64 : (2 * K + 63) / 64 * 64;
        const int64_t rows_b = op_b == GEMM_OP_N ? 2 * K : 2 * N;
        const int64_t na = batch > 1 && stride_a ? batch : 1, nbb = batch > 1 && stride_b ? batch : 1;
        r.lda = cx_ld_a;
        r.ldb = cx_ld_b;
        r.ldc = 2 * ldc;
        r.ab_type = GEMM_F16;
        r.cd_type = (cd_type == GEMM_CF32 || cd_type == GEMM_DF32) ? GEMM_F32 : GEMM_F16;
        r.stride_a = op_a == GEMM_OP_N ? 2 * stride_a : (na > 1 ? 2 * K * cx_ld_a : 0);
        r.stride_b = nbb > 1 ? rows_b * cx_ld_b : 0;
        r.stride_c = 2 * stride_c;
        r.stride_bias = 0;
        auto pblocks = [](int64_t pitch, int gb, int64_t rows, int64_t n) {
            return ((pitch / gb + 63) / 64) * ((rows + 3) / 4) * n;
        };
        const int64_t blocks = (op_a == GEMM_OP_T ? pblocks(cx_ld_a * 2, 8, K, na) : 0) +
                               pblocks(cx_ld_b * 2, 16, op_b == GEMM_OP_N ? K : N, nbb);
        gemm_plan *rp = nullptr;
        if (blocks < lim && gemm_plan_create_desc(&rp, &r) == GEMM_STATUS_SUCCESS) {
            // (a real product small enough that only the 128-wide tiles would take it keeps
            // the complex kernel: the rewrite pass would cost more than it saves)
            if ((rp->fast && !rp->fast_is_skinny && rp->fast->bm == 256) || (rp->fast_pk && rp->fast_pk->bm == 256) ||
                rp->fast_rs) {
                cx = rp;
                const int64_t bytes_a = op_a == GEMM_OP_T ? na * 2 * K * cx_ld_a * 2 : 0;
                cx_off_b = (bytes_a + 255) / 256 * 256;
                cx_bytes = cx_off_b + nbb * rows_b * cx_ld_b * 2;
            } else {
                gemm_plan_destroy(rp);
            }
        }
    }

    gemm_plan *p = new (std::nothrow) gemm_plan;
    if (!p) {
        if (cx) gemm_plan_destroy(cx);
        return GEMM_STATUS_ALLOC_FAILED;
    }
    p->M = M; p->N = N; p->K = K;
    p->batch = batch;
    p->batch2 = batch2;
    p->stride2_a = stride2_a; p->stride2_b = stride2_b; p->stride2_c = stride2_c; p->stride2_bias = stride2_bias;
    p->xform_a = desc->transform_a; p->xform_b = desc->transform_b; p->xform_c = desc->transform_c;
    p->stride_a = stride_a; p->stride_b = stride_b; p->stride_c = stride_c; p->stride_bias = stride_bias;
    p->lda = lda; p->ldb = ldb; p->ldc = ldc;
    p->op_a = op_a; p->op_b = op_b; p->ab = ab_type; p->cd = cd_type; p->epi = epi;
    p->kernel = k;
    p->fast = fast;
    p->fast_is_skinny = skinny;
    p->fast_rs = fast_rs;
    p->fast_pk = fast_pk;
    p->pk_need = pk_need;
    p->pk_want = pk_want;
    p->pk_tr = pk_tr;
    p->fast_pk_tr = fast_pk_tr;
    p->fast_part_tr = nullptr;
    p->fast_part128 = nullptr;
    p->fast_part128_tr = nullptr;
    p->pk_ld_a = pk_ld_a; p->pk_ld_b = pk_ld_b;
    p->pk_kpad = pk_kpad;
    p->pk_off_b = pk_off_b; p->pk_bytes = pk_bytes;
    p->pk_dev = -1;
    p->pk_ws = nullptr;
    p->cx = cx;
    p->cx_ld_a = cx_ld_a; p->cx_ld_b = cx_ld_b;
    p->cx_off_b = cx_off_b; p->cx_bytes = cx_bytes;
    p->cx_dev = -1;
    p->cx_ws = nullptr;
    p->ksplit = 1;
    p->ws_dev = -1;
    p->ws = nullptr;
    p->cv = nullptr;
    p->cv_src_a = p->cv_src_b = -1;
    p->cv_rows_a = p->cv_rows_b = p->cv_len_a = p->cv_len_b = p->cv_ld_a = p->cv_ld_b = 0;
    p->cv_off_b = p->cv_bytes = 0;
    p->cv_dev = -1;
    p->cv_ws = nullptr;
    // (an empty problem, N == 0 or a batch of 0, launches nothing and is never split)
    // (int8: one product, whose int32 partial sums the integer finishing kernel adds)
    if (skinny && fast->bn == 64 && N > 0 && nprod > 0 && algo != GEMM_ALGO_NOSPLIT &&
        !(ab_type == GEMM_I8 && nprod > 1)) {
        // split K over workgroups until there is about one workgroup per CU, keeping at least
        // eight 64-byte chunks per wave
        const int64_t blocks = ((N + 63) / 64) * (nprod > 1 ? nprod : 1);
        int64_t sp = (256 + blocks - 1) / blocks;
        const int64_t most = K / (64 / eab) / 32;
        if (sp > most) sp = most;
        if (sp > 64) sp = 64;
        p->ksplit = sp > 1 ? (int)sp : 1;
    }
    // the fast kernel's K split (above): on the operands in place or on their aligned copies
    p->fast_part = nullptr;
    p->finish = nullptr;
    if (split_s && (fast || fast_pk) && !skinny) {
        p->fast_part = fast_table(ab_type, ab_type == GEMM_I8 ? GEMM_I32 : GEMM_F32)(op_a, op_b, 0);
        if (pk_tr) p->fast_part_tr = fast_table(ab_type, ab_type == GEMM_I8 ? GEMM_I32 : GEMM_F32)(GEMM_OP_N, op_b, 0);
        p->finish = finish_table(ab_type, cd_type);
        p->ksplit = split_s;
    }
    if (split128 && !skinny) {
        p->fast_part128 = f128p(op_a, op_b);
        if (pk_tr) p->fast_part128_tr = f128p(GEMM_OP_N, op_b);
        p->finish = finish_table(ab_type, cd_type);
        p->ksplit = split128;
    }
    // a plan that always copies an operand (off the 16-byte grid, or carrying a load transform
    // that the copy applies) shows the direct kernel on the copies
    // (a skinny plan applies its transforms in its own kernel)
    const int pk_shown = fast_pk && !skinny ? (pk_need | pk_want | (desc->transform_a ? 1 : 0) |
                                               (desc->transform_b ? 2 : 0)) : 0;
    const bool shows_pk = pk_shown != 0;
    const bool shows_tr = pk_tr && (pk_shown & 1);
    const KernelEntry *shown = shows_tr ? fast_pk_tr : fast && !(shows_pk && fast_pk->bm != fast->bm) ? fast
                               : shows_pk ? fast_pk : fast_rs ? fast_rs : k;
    p->tiles_m = skinny ? p->ksplit : (int)((M + shown->bm - 1) / shown->bm);
    p->tiles_n = (int)((N + shown->bn - 1) / shown->bn);
    p->group_m = 8;
    const int64_t grid = (int64_t)p->tiles_m * p->tiles_n * nprod;
    if (grid >= ((int64_t)1 << 31)) {
        if (cx) gemm_plan_destroy(cx);
        delete p;
        return GEMM_STATUS_NOT_SUPPORTED;
    }
    p->grid = (unsigned)grid;
    char bdesc[64] = "";
    int bl = 0;
    if (batch2 > 1) bl = snprintf(bdesc, sizeof(bdesc), " batch %lldx%lld", (long long)batch, (long long)batch2);
    else if (batch != 1) bl = snprintf(bdesc, sizeof(bdesc), " batch %lld", (long long)batch);
    if (p->ksplit > 1) bl += snprintf(bdesc + bl, sizeof(bdesc) - bl, " ksplit %d", p->ksplit);
    if (shows_pk)
        bl += snprintf(bdesc + bl, sizeof(bdesc) - bl, " repack %s%s%s", pk_shown & 1 ? "A" : "",
                       pk_shown & 2 ? "B" : "", shows_tr ? " (A to K-major)" : "");
    if (diag_a || diag_b)
        bl += snprintf(bdesc + bl, sizeof(bdesc) - bl, " diag %s%s", diag_a ? "A" : "", diag_b ? "B" : "");
    if (desc->transform_a || desc->transform_b || desc->transform_c)
        snprintf(bdesc + bl, sizeof(bdesc) - bl, " relu-in %s%s%s", desc->transform_a ? "A" : "",
                 desc->transform_b ? "B" : "", desc->transform_c ? "C" : "");
    snprintf(p->desc, sizeof(p->desc), "%s %s->%s %c%c tile %dx%dx%d waves %dx%d grid %u%s",
             shown->name, dtype_name(ab_type), dtype_name(cd_type), op_a ? 'T' : 'N',
             op_b ? 'T' : 'N', shown->bm, shown->bn, shown->bk, shown->waves_m, shown->waves_n,
             p->grid, bdesc);
    if (cx)
        snprintf(p->desc, sizeof(p->desc), "%s->%s %c%c as real 2x2 blocks: %s", dtype_name(ab_type),
                 dtype_name(cd_type), op_a ? 'T' : 'N', op_b ? 'T' : 'N', cx->desc);
    *out = p;
    return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_plan_destroy(gemm_plan_t p) {
    if (p && p->ws) (void)hipFree(p->ws);
    if (p && p->pk_ws) (void)hipFree(p->pk_ws);
    if (p && p->cx_ws) (void)hipFree(p->cx_ws);
    if (p && p->cx) gemm_plan_destroy(p->cx);
    if (p && p->cv_ws) (void)hipFree(p->cv_ws);
    if (p && p->cv) gemm_plan_destroy(p->cv);
    delete p;
    return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_plan_describe(gemm_plan_t p, char *buf, size_t len) {
    if (!p || !buf || len == 0) return GEMM_STATUS_INVALID_VALUE;
    snprintf(buf, len, "%s", p->desc);
    return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_run(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                       const void *bias, float alpha, float beta, void *stream) {
    return run_impl(p, A, B, C, D, bias, alpha, beta, stream, nullptr);
}

gemm_status_t gemm_run_noalloc(gemm_plan_t p, const void *A, const void *B, const void *C, void *D,
                               const void *bias, float alpha, float beta, void *stream) {
    // sizing pass first (no HIP call): a run that needs more scratch than the array holds is
    // rejected before anything is enqueued
    Scratch size = {nullptr, (size_t)GEMM_NOALLOC_SCRATCH_BYTES, 0, true};
    const gemm_status_t st = run_impl(p, A, B, C, D, bias, alpha, beta, stream, &size);
    if (st != GEMM_STATUS_SUCCESS) return st;
    // the same route again, launching; a route that takes no region never needs the address
    Scratch sc = {nullptr, size.used, 0, false};
    if (size.used > 0) {
        const gemm_status_t sa = scratch_address(&sc.base);
        if (sa != GEMM_STATUS_SUCCESS) return sa;
    }
    return run_impl(p, A, B, C, D, bias, alpha, beta, stream, &sc);
}

}  // extern "C"
