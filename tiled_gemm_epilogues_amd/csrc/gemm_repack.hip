// Aligned copies of operands the direct-to-LDS loads cannot take.
//
// The fast kernel's direct loads move whole 16-byte chunks from global memory straight into
// LDS, so every stored row must start on a 16-byte boundary and hold a whole number of chunks.
// An operand whose pointer, leading dimension or batch stride is off that grid, or whose
// stored row length is not a whole number of chunks, is first copied here, once per run, into
// a workspace whose rows are 16-byte aligned and zero-padded to whole chunks; the fast kernel
// then reads the copy.  The pages make unaligned operands a compile-time switch to narrower
// loads ("Ragged" in the Julia GemmKernels design, "Layout modularity"); on gfx950 one
// streaming copy costs less than narrow or register-staged loads inside the pipelined loop.
//
// Complex and dual numbers (fp16 parts) on large shapes are rewritten here as real matrices so
// that the real fast kernel computes their product (pair_rows): "Flexible Performant GEMM
// Kernels on GPUs" (section 5.4) builds these GEMMs from four real products of the parts; the
// same four products are the 2 x 2 real block [re im; -im re] that replaces each number of
// op(B) (dual numbers: [re im; 0 re]), with op(A) read as reals whose parts alternate along K.
//
// A plan with a load transform (ReLU as loaded) on op(A) or op(B) copies that operand too and
// applies the transform in the copy: the fast kernel's 16x16 MFMA schedule has no registers to
// spare for transforming fragments, and one streaming pass costs less than the 32x32 schedule
// that can.
//
// The copy is byte-exact (any element type) unless it carries the transform: row r of product
// b goes from src + b * src_stride + r * src_pitch (row_bytes bytes) to
// dst + b * dst_stride + r * dst_pitch, followed by zeros up to dst_pitch; rows past the
// source's (K rounded up to whole slabs, for an operand stored K-major) are zeros.  One wave
// copies 64 consecutive chunks (1 KiB) of one row; a workgroup covers 4 rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int RP_ROWS = 4;     // rows per workgroup (one wave each)
constexpr int RP_CHUNKS = 64;  // 16-byte chunks per wave

__device__ __forceinline__ void repack_block(const RepackJob &j, uint32_t blk, int wave, int lane) {
    // workgroup blk -> (product, block of 4 rows, block of 64 chunks); uniform divisions
    const uint32_t cblk = (uint32_t)((j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS);
    const uint32_t rblk = (uint32_t)((j.rows_out + RP_ROWS - 1) / RP_ROWS);
    const uint32_t prod = blk / (cblk * rblk);
    const uint32_t rem = blk - prod * cblk * rblk;
    const uint32_t rb = rem / cblk, cb = rem - rb * cblk;
    const int64_t r = (int64_t)rb * RP_ROWS + wave;
    const int64_t c = (int64_t)cb * RP_CHUNKS + lane;
    if (r >= j.rows_out || c * 16 >= j.dst_pitch) return;
    const uint8_t *s = j.src + (int64_t)prod * j.src_stride + r * j.src_pitch + c * 16;
    // bytes of the source row from this chunk on (none in the zero rows past `rows`)
    const int64_t left = r < j.rows ? j.row_bytes - c * 16 : 0;
    u32x4 v = {0, 0, 0, 0};
    if (left >= 16) v = ldg16(s);
    else if (left > 0) v = ldg16_partial<1>(s, (int)left);
    // the load transform, when the copy carries it (branch-free on the uniform xf_elem)
    v = zero_negative<2>(v, j.xf_elem == 2);
    v = zero_negative<1>(v, j.xf_elem == 1);
    *reinterpret_cast<u32x4 *>(j.dst + (int64_t)prod * j.dst_stride + r * j.dst_pitch + c * 16) = v;
}

// ---- transposing copies ----------------------------------------------------------------------
// An operand stored M/N-contiguous (A stored K x M) copied into K-contiguous rows, so that the
// fast kernel runs the schedule of the other layout.  A workgroup moves one tile of TK source
// rows (k) x TM elements (m), TK and TM both 128 bytes' worth of elements: the source rows are
// read across the lanes (consecutive m, any alignment: one element per load), consecutive k are
// packed into dwords of a row of LDS per m, and each destination row's 128-byte piece leaves as
// eight 16-byte chunks.  Source rows k >= rows read as zeros, so the copy's K padding is zero.
constexpr int TR_LINE = 128;                 // bytes of k (destination) and of m (source) per tile
constexpr int TR_PITCH = TR_LINE + 16;       // LDS row pitch: 16-byte aligned rows, skewed banks
constexpr int TR_LDS = 128 * TR_PITCH;       // TM <= 128 rows

template <int EB>
__device__ __forceinline__ void transpose_block(const RepackJob &j, uint32_t blk, int tid, uint8_t *tile) {
    constexpr int TM = TR_LINE / EB;         // source elements (destination rows) per tile
    constexpr int PER = 4 / EB;              // k values per dword
    constexpr int GROUPS = 256 / TM;         // dword columns loaded at once
    const int64_t M = j.row_bytes / EB;
    const uint32_t kblk = (uint32_t)(j.rows_out * EB / TR_LINE);
    const uint32_t mblk = (uint32_t)((M + TM - 1) / TM);
    const uint32_t prod = blk / (kblk * mblk);
    const uint32_t rem = blk - prod * kblk * mblk;
    const uint32_t mb = rem / kblk, kb = rem - mb * kblk;
    const int64_t m0 = (int64_t)mb * TM, k0 = (int64_t)kb * (TR_LINE / EB);
    const uint8_t *src = j.src + (int64_t)prod * j.src_stride;
    {
        const int mi = tid % TM;
        const int64_t m = m0 + mi;
        // every load of the tile is issued before the first LDS write waits for one
#pragma unroll
        for (int it = 0; it < TR_LINE / 4 / GROUPS; ++it) {
            const int kd = tid / TM + it * GROUPS;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int64_t k = k0 + kd * PER + e;
                if (m < M && k < j.rows) {
                    const uint8_t *q = src + k * j.src_pitch + m * EB;
                    const uint32_t x = EB == 2 ? (uint32_t)*reinterpret_cast<const uint16_t *>(q) : (uint32_t)*q;
                    w |= x << (8 * EB * e);
                }
            }
            *reinterpret_cast<uint32_t *>(tile + mi * TR_PITCH + 4 * kd) = w;
        }
    }
    __syncthreads();
    uint8_t *dst = j.dst + (int64_t)prod * j.dst_stride + k0 * EB;
#pragma unroll
    for (int idx = tid; idx < TM * (TR_LINE / 16); idx += 256) {
        const int mm = idx / (TR_LINE / 16), c = idx % (TR_LINE / 16);
        if (m0 + mm >= M) continue;
        u32x4 v = *reinterpret_cast<const u32x4 *>(tile + mm * TR_PITCH + 16 * c);
        v = zero_negative<EB>(v, j.xf_elem != 0);
        *reinterpret_cast<u32x4 *>(dst + (m0 + mm) * j.dst_pitch + 16 * c) = v;
    }
}

__device__ __forceinline__ void copy_block(const RepackJob &j, uint32_t blk, int tid, uint8_t *tile) {
    // uniform per job
    if (j.tr_elem == 2) transpose_block<2>(j, blk, tid, tile);
    else if (j.tr_elem == 1) transpose_block<1>(j, blk, tid, tile);
    else repack_block(j, blk, __builtin_amdgcn_readfirstlane(tid >> 6), tid & 63);
}

// Grid: blocks_a workgroups for job a, then those of job b (none when b.rows_out == 0).
__global__ __launch_bounds__(RP_ROWS * 64) void repack_rows(RepackJob a, RepackJob b, uint32_t blocks_a) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[TR_LDS];
    if (blockIdx.x < blocks_a) copy_block(a, blockIdx.x, threadIdx.x, tile);
    else copy_block(b, blockIdx.x - blocks_a, threadIdx.x, tile);
}

uint32_t job_blocks(const RepackJob &j) {
    if (j.rows_out <= 0 || j.batch <= 0) return 0;
    if (j.tr_elem) {
        const int64_t tm = TR_LINE / j.tr_elem;
        const int64_t m = j.row_bytes / j.tr_elem;
        return (uint32_t)((j.rows_out * j.tr_elem / TR_LINE) * ((m + tm - 1) / tm) * j.batch);
    }
    const int64_t cblk = (j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS;
    const int64_t rblk = (j.rows_out + RP_ROWS - 1) / RP_ROWS;
    return (uint32_t)(cblk * rblk * j.batch);
}

// ---- complex and dual operands as real matrices -----------------------------------------------
// A number is one dword: real part in the low half, imaginary (or dual) part in the high half.
// A thread takes 4 consecutive numbers of a source row (a 16-byte load; numbers past the row
// read as 0) and writes its share of the two destination rows 2r and 2r+1.

constexpr uint32_t SIGN_LO = 0x8000u, SIGN_HI = 0x80000000u;

__device__ __forceinline__ void pair_block(const PairJob &j, uint32_t blk, int wave, int lane) {
    const int gb = j.mode == PAIR_PARTS ? 8 : 16;                 // destination bytes per group
    const uint32_t cblk = (uint32_t)((j.dst_pitch / gb + RP_CHUNKS - 1) / RP_CHUNKS);
    const uint32_t rblk = (uint32_t)((j.rows + RP_ROWS - 1) / RP_ROWS);
    const uint32_t prod = blk / (cblk * rblk);
    const uint32_t rem = blk - prod * cblk * rblk;
    const uint32_t rb = rem / cblk, cb = rem - rb * cblk;
    const int64_t r = (int64_t)rb * RP_ROWS + wave;
    const int64_t g = (int64_t)cb * RP_CHUNKS + lane;              // group of 4 numbers
    if (r >= j.rows || g * gb >= j.dst_pitch) return;
    const uint8_t *s = j.src + (int64_t)prod * j.src_stride + r * j.src_pitch + g * 16;
    const int64_t left = j.numbers - 4 * g;
    u32x4 v = {0, 0, 0, 0};
    if (left >= 4) v = ldg16(s);
    else if (left > 0) v = ldg16_partial<4>(s, (int)left);
    uint8_t *d0 = j.dst + (int64_t)prod * j.dst_stride + 2 * r * j.dst_pitch + g * gb;
    uint8_t *d1 = d0 + j.dst_pitch;
    if (j.mode == PAIR_PARTS) {
        // row 2r: the four real parts; row 2r+1: the four other parts
        u32x2 re, im;
        re[0] = (v[0] & 0xFFFFu) | (v[1] << 16);
        re[1] = (v[2] & 0xFFFFu) | (v[3] << 16);
        im[0] = (v[0] >> 16) | (v[1] & 0xFFFF0000u);
        im[1] = (v[2] >> 16) | (v[3] & 0xFFFF0000u);
        *reinterpret_cast<u32x2 *>(d0) = re;
        *reinterpret_cast<u32x2 *>(d1) = im;
        return;
    }
    u32x4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = v[i];
        const uint32_t swapped = (x >> 16) | (x << 16);            // (im, re)
        if (j.mode == PAIR_BLOCK_N) {
            // row 2k: (re, im) as stored; row 2k+1: (-im, re), dual (0, re)
            w0[i] = x;
            w1[i] = j.dual ? (x << 16) : (swapped ^ SIGN_LO);
        } else {
            // row 2n: (re, -im), dual (re, 0); row 2n+1: (im, re)
            w0[i] = j.dual ? (x & 0xFFFFu) : (x ^ SIGN_HI);
            w1[i] = swapped;
        }
    }
    *reinterpret_cast<u32x4 *>(d0) = w0;
    *reinterpret_cast<u32x4 *>(d1) = w1;
}

__global__ __launch_bounds__(RP_ROWS * 64) void pair_rows(PairJob a, PairJob b, uint32_t blocks_a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (blockIdx.x < blocks_a) pair_block(a, blockIdx.x, wave, lane);
    else pair_block(b, blockIdx.x - blocks_a, wave, lane);
}

uint32_t pair_job_blocks(const PairJob &j) {
    if (j.rows <= 0 || j.batch <= 0) return 0;
    const int gb = j.mode == PAIR_PARTS ? 8 : 16;
    const int64_t cblk = (j.dst_pitch / gb + RP_CHUNKS - 1) / RP_CHUNKS;
    const int64_t rblk = (j.rows + RP_ROWS - 1) / RP_ROWS;
    return (uint32_t)(cblk * rblk * j.batch);
}

// ---- type-converting copies ------------------------------------------------------------------
// An operand stored as fp32 or int8 whose load transform converts it to the 16-bit input type
// ("Flexible Performant GEMM Kernels on GPUs", section 4: a transform applied to every element
// after it is loaded, such as a type conversion) is converted here, once per run, into 16-bit
// rows that are 16-byte aligned and zero-padded to whole chunks; the product then reads the
// converted rows like any other operand.  fp32 -> fp16 / bf16 rounds to nearest even; int8
// converts exactly.  A thread writes one 16-byte chunk (8 elements) of a destination row,
// reading the 8 source elements it holds (32 bytes of fp32 or 8 bytes of int8; elements past the
// row read as 0); a wave covers 64 consecutive chunks of one row, a workgroup 4 rows.

template <int SRC, bool BF>
__device__ __forceinline__ void convert_block(const ConvertJob &j, uint32_t blk, int wave, int lane) {
    constexpr int SB = SRC == CONVERT_FROM_F32 ? 4 : 1;          // source element bytes
    const uint32_t cblk = (uint32_t)((j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS);
    const uint32_t rblk = (uint32_t)((j.rows + RP_ROWS - 1) / RP_ROWS);
    const uint32_t prod = blk / (cblk * rblk);
    const uint32_t rem = blk - prod * cblk * rblk;
    const uint32_t rb = rem / cblk, cb = rem - rb * cblk;
    const int64_t r = (int64_t)rb * RP_ROWS + wave;
    const int64_t c = (int64_t)cb * RP_CHUNKS + lane;
    if (r >= j.rows || c * 16 >= j.dst_pitch) return;
    const uint8_t *s = j.src + (int64_t)prod * j.src_stride + r * j.src_pitch + c * 8 * SB;
    const int64_t left = j.elems - c * 8;                          // source elements from here
    float x[8];
    if constexpr (SRC == CONVERT_FROM_F32) {
        u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        if (left >= 8) {
            lo = ldg16(s);
            hi = ldg16(s + 16);
        } else if (left > 0) {
            lo = ldg16_partial<4>(s, (int)(left < 4 ? left : 4));
            if (left > 4) hi = ldg16_partial<4>(s + 16, (int)(left - 4));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = __builtin_bit_cast(float, (uint32_t)lo[e]);
            x[e + 4] = __builtin_bit_cast(float, (uint32_t)hi[e]);
        }
    } else {
        uint8_t b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (left >= 8) {
            __builtin_memcpy(b, s, 8);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < left) b[e] = s[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)(int8_t)b[e];
    }
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    using T = typename std::conditional<BF, __bf16, _Float16>::type;
    typedef T t2 __attribute__((ext_vector_type(2)));
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // two-at-a-time conversion, round to nearest even
        const t2 h = __builtin_convertvector((f32x2){x[2 * e], x[2 * e + 1]}, t2);
        out[e] = __builtin_bit_cast(uint32_t, h);
    }
    *reinterpret_cast<u32x4 *>(j.dst + (int64_t)prod * j.dst_stride + r * j.dst_pitch + c * 16) = out;
}

uint32_t convert_job_blocks(const ConvertJob &j) {
    if (j.rows <= 0 || j.batch <= 0) return 0;
    const int64_t cblk = (j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS;
    const int64_t rblk = (j.rows + RP_ROWS - 1) / RP_ROWS;
    return (uint32_t)(cblk * rblk * j.batch);
}

template <int SRC, bool BF>
__device__ __forceinline__ void convert_one(const ConvertJob &j, uint32_t blk, int wave, int lane) {
    convert_block<SRC, BF>(j, blk, wave, lane);
}

__device__ __forceinline__ void convert_dispatch(const ConvertJob &j, uint32_t blk, int wave, int lane) {
    // uniform per job
    if (j.src_type == CONVERT_FROM_F32) {
        if (j.to_bf16) convert_one<CONVERT_FROM_F32, true>(j, blk, wave, lane);
        else convert_one<CONVERT_FROM_F32, false>(j, blk, wave, lane);
    } else {
        if (j.to_bf16) convert_one<CONVERT_FROM_I8, true>(j, blk, wave, lane);
        else convert_one<CONVERT_FROM_I8, false>(j, blk, wave, lane);
    }
}

__global__ __launch_bounds__(RP_ROWS * 64) void convert_rows(ConvertJob a, ConvertJob b, uint32_t blocks_a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (blockIdx.x < blocks_a) convert_dispatch(a, blockIdx.x, wave, lane);
    else convert_dispatch(b, blockIdx.x - blocks_a, wave, lane);
}

// ---- the K split's finishing step for int8 products ---------------------------------------------
// D[m][n] = ReLU?(sum of the S int32 partial sums [split][M][N] in ws, in split order,
// + beta * C (beta 0 or 1) + bias[n]); int32 arithmetic wraps exactly as the unsplit sum does.
// One thread per 4 consecutive columns (16-byte loads of the partial sums when N % 4 == 0, the
// split loop unrolled so that several loads are in flight).
__global__ __launch_bounds__(256) void finish_int(GemmParams p) {
    constexpr int CPT = 4, SPAN = 256 * CPT;
    const int tiles = (p.N + SPAN - 1) / SPAN;
    const int m = blockIdx.x / tiles;
    const int n0 = (blockIdx.x - m * tiles) * SPAN + (int)threadIdx.x * CPT;
    if (m >= p.M || n0 >= p.N) return;
    const int S = p.tiles_m;
    const int64_t plane = (int64_t)p.M * p.N;
    const uint32_t *ws = reinterpret_cast<const uint32_t *>(p.ws) + (int64_t)m * p.N + n0;
    uint32_t v[CPT] = {0, 0, 0, 0};
    if (p.N % CPT == 0) {
#pragma unroll 4
        for (int q = 0; q < S; ++q) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(ws + q * plane);
#pragma unroll
            for (int e = 0; e < CPT; ++e) v[e] += w[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < CPT; ++e)
            if (n0 + e < p.N)
                for (int q = 0; q < S; ++q) v[e] += ws[q * plane + e];
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        const int n = n0 + e;
        if (n >= p.N) break;
        const int64_t idx = (int64_t)m * p.ldc + n;
        uint32_t t = v[e];
        if (p.has_beta) t += (uint32_t)c_in_i(static_cast<const int *>(p.C)[idx], p.xform_c);
        if (p.has_bias) t += (uint32_t)static_cast<const int *>(p.bias)[n];
        int x = (int)t;
        if (p.relu) x = x > 0 ? x : 0;
        static_cast<int *>(p.D)[idx] = x;
    }
}

}  // namespace

hipError_t finish_i8_i32(const GemmParams &p, hipStream_t s) {
    const unsigned g = (unsigned)((int64_t)((p.N + 1023) / 1024) * p.M);
    hipLaunchKernelGGL(finish_int, dim3(g), dim3(256), 0, s, p);
    return hipGetLastError();
}

int64_t repack_blocks(const RepackJob &j) { return job_blocks(j); }

int64_t pair_blocks(const PairJob &j) { return pair_job_blocks(j); }

hipError_t pair_launch(const PairJob &a, const PairJob &b, hipStream_t stream) {
    const uint32_t na = pair_job_blocks(a), nb = pair_job_blocks(b);
    if (na + nb == 0) return hipSuccess;
    hipLaunchKernelGGL(pair_rows, dim3(na + nb), dim3(RP_ROWS * 64), 0, stream, a, b, na);
    return hipGetLastError();
}

int64_t convert_blocks(const ConvertJob &j) { return convert_job_blocks(j); }

hipError_t convert_launch(const ConvertJob &a, const ConvertJob &b, hipStream_t stream) {
    const uint32_t na = convert_job_blocks(a), nb = convert_job_blocks(b);
    if (na + nb == 0) return hipSuccess;
    hipLaunchKernelGGL(convert_rows, dim3(na + nb), dim3(RP_ROWS * 64), 0, stream, a, b, na);
    return hipGetLastError();
}

hipError_t repack_launch(const RepackJob &a, const RepackJob &b, hipStream_t stream) {
    const uint32_t na = job_blocks(a), nb = job_blocks(b);
    if (na + nb == 0) return hipSuccess;
    hipLaunchKernelGGL(repack_rows, dim3(na + nb), dim3(RP_ROWS * 64), 0, stream, a, b, na);
    return hipGetLastError();
}

}  // namespace tge
