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
// The copy is byte-exact (any element type): row r of product b goes from
// src + b * src_stride + r * src_pitch (row_bytes bytes) to dst + b * dst_stride + r * dst_pitch,
// followed by zeros up to dst_pitch.  One wave copies 64 consecutive chunks (1 KiB) of one row;
// a workgroup covers 4 rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

constexpr int RP_ROWS = 4;     // rows per workgroup (one wave each)
constexpr int RP_CHUNKS = 64;  // 16-byte chunks per wave

__device__ __forceinline__ void repack_block(const RepackJob &j, uint32_t blk, int wave, int lane) {
    // workgroup blk -> (product, block of 4 rows, block of 64 chunks); uniform divisions
    const uint32_t cblk = (uint32_t)((j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS);
    const uint32_t rblk = (uint32_t)((j.rows + RP_ROWS - 1) / RP_ROWS);
    const uint32_t prod = blk / (cblk * rblk);
    const uint32_t rem = blk - prod * cblk * rblk;
    const uint32_t rb = rem / cblk, cb = rem - rb * cblk;
    const int64_t r = (int64_t)rb * RP_ROWS + wave;
    const int64_t c = (int64_t)cb * RP_CHUNKS + lane;
    if (r >= j.rows || c * 16 >= j.dst_pitch) return;
    const uint8_t *s = j.src + (int64_t)prod * j.src_stride + r * j.src_pitch + c * 16;
    const int64_t left = j.row_bytes - c * 16;   // bytes of the source row from this chunk on
    u32x4 v = {0, 0, 0, 0};
    if (left >= 16) v = ldg16(s);
    else if (left > 0) v = ldg16_partial<1>(s, (int)left);
    *reinterpret_cast<u32x4 *>(j.dst + (int64_t)prod * j.dst_stride + r * j.dst_pitch + c * 16) = v;
}

// Grid: blocks_a workgroups for job a, then those of job b (none when b.rows == 0).
__global__ __launch_bounds__(RP_ROWS * 64) void repack_rows(RepackJob a, RepackJob b, uint32_t blocks_a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (blockIdx.x < blocks_a) repack_block(a, blockIdx.x, wave, lane);
    else repack_block(b, blockIdx.x - blocks_a, wave, lane);
}

uint32_t job_blocks(const RepackJob &j) {
    if (j.rows <= 0 || j.batch <= 0) return 0;
    const int64_t cblk = (j.dst_pitch / 16 + RP_CHUNKS - 1) / RP_CHUNKS;
    const int64_t rblk = (j.rows + RP_ROWS - 1) / RP_ROWS;
    return (uint32_t)(cblk * rblk * j.batch);
}

}  // namespace

int64_t repack_blocks(const RepackJob &j) { return job_blocks(j); }

hipError_t repack_launch(const RepackJob &a, const RepackJob &b, hipStream_t stream) {
    const uint32_t na = job_blocks(a), nb = job_blocks(b);
    if (na + nb == 0) return hipSuccess;
    hipLaunchKernelGGL(repack_rows, dim3(na + nb), dim3(RP_ROWS * 64), 0, stream, a, b, na);
    return hipGetLastError();
}

}  // namespace tge
