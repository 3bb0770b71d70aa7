// Internal interface between the host plan/run code and the device kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tge {

// Everything a kernel needs for one launch; passed by value as the kernel argument.
struct GemmParams {
    const void *A, *B, *C;
    void *D;
    const void *bias;
    int M, N, K;
    int lda, ldb, ldc;       // elements of each matrix's own type
    float alpha, beta;
    int has_beta, has_bias, relu;
    int tiles_m, tiles_n;    // output tiles along M and N (of one product)
    int group_m;             // tile rows per raster group
    // strided batch: the launch computes `batch` independent products; product b reads and
    // writes the operands moved by b * stride (in elements of each operand's own type; C and D
    // share stride_c; a zero stride shares that operand between products).  With a second batch
    // mode (batch2 > 1) `batch` counts all products and product b = b1 * batch2 + b2 is moved by
    // b1 * stride + b2 * stride2
    int batch;
    int64_t stride_a, stride_b, stride_c, stride_bias;
    int batch2;
    int64_t stride2_a, stride2_b, stride2_c, stride2_bias;
    // load transforms (1: zero every element whose sign bit is set) on op(A), op(B) and C
    int xform_a, xform_b, xform_c;
    // split-K workspace of the skinny kernel (partial sums of every k split); unused elsewhere
    float *ws;
};

using LaunchFn = hipError_t (*)(const GemmParams &, unsigned grid, hipStream_t);

// One compiled kernel variant and its tile shape.
struct KernelEntry {
    LaunchFn launch;
    int bm, bn, bk;          // workgroup tile (bk in elements)
    int waves_m, waves_n;    // wave grid inside the workgroup
    const char *name;
};

// Tile configurations, largest first.
enum TileCfg { CFG_256 = 0, CFG_128 = 1, CFG_64 = 2, CFG_COUNT = 3 };

// Per type-pair lookup, defined by the kernel translation units (one per pair).
// op_a/op_b: 0 = N, 1 = T.  Returns nullptr for an unknown combination.
const KernelEntry *kernels_f32_f32(int op_a, int op_b, int cfg);
const KernelEntry *kernels_f16_f16(int op_a, int op_b, int cfg);
const KernelEntry *kernels_f16_f32(int op_a, int op_b, int cfg);
const KernelEntry *kernels_bf16_bf16(int op_a, int op_b, int cfg);
const KernelEntry *kernels_bf16_f32(int op_a, int op_b, int cfg);
const KernelEntry *kernels_i8_i32(int op_a, int op_b, int cfg);

// Products with a diagonal operand (gemm_diag.hip), streamed: dg bit 0 = A diagonal, bit 1 =
// B diagonal; the op of the dense operand picks the kernel.  No alignment preconditions.
const KernelEntry *diag_f32_f32(int op_a, int op_b, int dg);
const KernelEntry *diag_f16_f16(int op_a, int op_b, int dg);
const KernelEntry *diag_f16_f32(int op_a, int op_b, int dg);
const KernelEntry *diag_bf16_bf16(int op_a, int op_b, int dg);
const KernelEntry *diag_bf16_f32(int op_a, int op_b, int dg);
const KernelEntry *diag_i8_i32(int op_a, int op_b, int dg);

// Fast 256x256 path for 16- and 8-bit inputs (gemm_fast.hip); K >= one slab (64 elements, 128
// for int8).  rs = 0: direct-to-LDS loads; needs 16-byte aligned A/B pointers, leading dimensions
// and batch strides, and M (when A is stored transposed) and N (when B is not) multiples of
// 16 / element size.  rs = 1: register-staged loads, no alignment or extent preconditions.
const KernelEntry *fast_f16_f16(int op_a, int op_b, int rs);
const KernelEntry *fast_f16_f32(int op_a, int op_b, int rs);
const KernelEntry *fast_bf16_bf16(int op_a, int op_b, int rs);
const KernelEntry *fast_bf16_f32(int op_a, int op_b, int rs);
const KernelEntry *fast_i8_i32(int op_a, int op_b, int rs);
// The same kernel with 128x128 tiles (4 waves of 64x64, two workgroups per CU) for mid-size
// products: direct loads only (the same alignment preconditions), no load transforms on
// op(A)/op(B).
const KernelEntry *fast128_f16_f16(int op_a, int op_b);
const KernelEntry *fast128_f16_f32(int op_a, int op_b);
const KernelEntry *fast128_bf16_bf16(int op_a, int op_b);
const KernelEntry *fast128_bf16_f32(int op_a, int op_b);
const KernelEntry *fast128_i8_i32(int op_a, int op_b);

// Byte-exact copy of an operand into rows that are 16-byte aligned and zero-padded to whole
// 16-byte chunks (gemm_repack.hip), for operands the direct loads cannot take: row r < rows of
// product b goes from src + b * src_stride + r * src_pitch (row_bytes bytes) to
// dst + b * dst_stride + r * dst_pitch, rows rows .. rows_out - 1 are written as zeros (all in
// bytes; dst, dst_pitch and dst_stride multiples of 16, dst_pitch >= row_bytes, rows_out >=
// rows).  repack_launch copies a and b (rows_out == 0: no job) in one launch; the caller keeps
// the total of repack_blocks below 2^31.
// With xf_elem = 1 or 2 the copy also applies the load transform GEMM_TRANSFORM_RELU to
// elements of that many bytes (every element whose sign bit is set becomes +0).
// tr_elem = 1 or 2 makes the copy transposing, for elements of that many bytes: the source's
// `rows` rows (k) of row_bytes / tr_elem elements (m) become row_bytes / tr_elem destination
// rows of rows_out elements each (k; zero for k >= rows), row m at dst + b * dst_stride +
// m * dst_pitch; rows_out * tr_elem a multiple of 128, src_pitch a multiple of tr_elem.
struct RepackJob {
    const uint8_t *src;
    uint8_t *dst;
    int64_t rows, rows_out, row_bytes, src_pitch, dst_pitch, src_stride, dst_stride, batch;
    int xf_elem;
    int tr_elem;
};
int64_t repack_blocks(const RepackJob &j);
hipError_t repack_launch(const RepackJob &a, const RepackJob &b, hipStream_t stream);

// Type-converting copy (gemm_repack.hip): an operand stored as fp32 (src_type
// CONVERT_FROM_F32, rounded to nearest even) or int8 (CONVERT_FROM_I8, exact) becomes fp16 (or
// bf16 with to_bf16) rows.  Row r < rows of product b holds `elems` source elements at
// src + b * src_stride + r * src_pitch (bytes, any alignment); it is written to
// dst + b * dst_stride + r * dst_pitch (dst, dst_pitch and dst_stride multiples of 16;
// dst_pitch >= 2 * elems), zero past the row's elements.  convert_launch converts a and b
// (rows == 0: no job) in one launch; the caller keeps the total of convert_blocks below 2^31.
enum ConvertSrc { CONVERT_FROM_F32 = 0, CONVERT_FROM_I8 = 1 };
struct ConvertJob {
    const uint8_t *src;
    uint8_t *dst;
    int64_t rows, elems, src_pitch, dst_pitch, src_stride, dst_stride, batch;
    int src_type, to_bf16;
};
int64_t convert_blocks(const ConvertJob &j);
hipError_t convert_launch(const ConvertJob &a, const ConvertJob &b, hipStream_t stream);

// Complex / dual operands with fp16 parts rewritten as real fp16 matrices for the real kernels
// (gemm_repack.hip).  Source row r of product b holds `numbers` numbers (4 bytes each: real
// part low, other part high) at src + b * src_stride + r * src_pitch; it becomes destination
// rows 2r and 2r+1 at dst + b * dst_stride + (2r + h) * dst_pitch (bytes; dst_pitch a multiple
// of 16, zero-padded past the data):
//   PAIR_PARTS    row 2r: the real parts, row 2r+1: the other parts (numbers fp16 values each)
//   PAIR_BLOCK_N  row 2r: (re, im) pairs as stored, row 2r+1: (-im, re) pairs, dual (0, re)
//   PAIR_BLOCK_T  row 2r: (re, -im) pairs, dual (re, 0), row 2r+1: (im, re) pairs
// A complex product is then a real one: with op(A) read as M x 2K reals (parts interleaved
// along K) and each number b of op(B) replaced by the 2 x 2 block [re im; -im re] (dual:
// [re im; 0 re]), D read as M x 2N reals is op(A) times the 2K x 2N block matrix.
enum PairMode { PAIR_PARTS = 0, PAIR_BLOCK_N = 1, PAIR_BLOCK_T = 2 };
struct PairJob {
    const uint8_t *src;
    uint8_t *dst;
    int64_t rows, numbers, src_pitch, dst_pitch, src_stride, dst_stride, batch;
    int mode, dual;
};
int64_t pair_blocks(const PairJob &j);
hipError_t pair_launch(const PairJob &a, const PairJob &b, hipStream_t stream);

// Complex and dual GEMM (gemm_complex.hip): fp16 parts, fp32 accumulation, 128x128 tile.
const KernelEntry *complex_cf16_cf32(int op_a, int op_b);
const KernelEntry *complex_cf16_cf16(int op_a, int op_b);
const KernelEntry *complex_df16_df32(int op_a, int op_b);
const KernelEntry *complex_df16_df16(int op_a, int op_b);

// Memory-bound path for M <= 64 (gemm_skinny.hip); mt = ceil(M / 16).  Preconditions: 16-bit
// inputs, or int8 inputs with B transposed (op_b == T); op_a == N, K a whole number of 64-byte
// chunks (K % 32 == 0 for 16-bit inputs, K % 64 == 0 for int8), 16-byte aligned A/B pointers and
// leading dimensions, N % 8 == 0 when B is not transposed.  One workgroup per bn (64) columns and k split: the
// launch sets tiles_m = S (k splits), tiles_n = ceil(N / bn), grid = S * tiles_n * batch, and
// with S > 1 passes the workspace ws (batch * S * M * N floats); the entry then enqueues a
// second, finishing kernel.  narrow = 1 (B transposed only): 16 columns per workgroup, S = 1.
const KernelEntry *skinny_f16_f16(int op_b, int mt, int narrow);
const KernelEntry *skinny_f16_f32(int op_b, int mt, int narrow);
const KernelEntry *skinny_bf16_bf16(int op_b, int mt, int narrow);
const KernelEntry *skinny_bf16_f32(int op_b, int mt, int narrow);
const KernelEntry *skinny_i8_i32(int op_b, int mt, int narrow);   // op_b == T only; S > 1: one product

// The finishing step alone: D = epilogue(sum over the p.tiles_m splits of ws, in split order),
// ws laid out [product][split][M][N] floats; p otherwise as for the product (C, bias, ldc,
// alpha, beta, ReLU, the C transform).  Used by the fast kernel's K split too.
hipError_t finish_f16_f16(const GemmParams &p, hipStream_t s);
hipError_t finish_f16_f32(const GemmParams &p, hipStream_t s);
hipError_t finish_bf16_bf16(const GemmParams &p, hipStream_t s);
hipError_t finish_bf16_f32(const GemmParams &p, hipStream_t s);
// int8 -> int32 (gemm_repack.hip): int32 partial sums in ws, one product (batch 1)
hipError_t finish_i8_i32(const GemmParams &p, hipStream_t s);

}  // namespace tge
