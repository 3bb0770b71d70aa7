// GEMM on complex and dual numbers with fp16 parts and fp32 accumulation, for gfx950.
//
// "Flexible Performant GEMM Kernels on GPUs" (section 5.4, Figure 12) builds these from two
// changes to the real GEMM: the multiply-accumulate of a tile becomes four real ones (A.re*B.re,
// A.re*B.im, A.im*B.re, A.im*B.im) combined per the number system, and the operands, stored
// interleaved (real and imaginary parts next to each other) in global memory, are kept split
// (one plane per part) in shared memory so the matrix units see plain real tiles.  Dual numbers
// a + b*eps with eps^2 = 0 reuse both layouts and drop the b*b' product:
//   complex: (a + bi)(c + di) = (ac - bd) + (ad + bc) i
//   dual:    (a + b eps)(c + d eps) = ac + (ad + bc) eps
//
// Here: 128x128 output tile per workgroup, 4 waves of 64x64 (2x2 MFMA 32x32x16 tiles, one
// accumulator set per part), K in slabs of 64 numbers.  Global -> registers with 16-byte loads
// along each operand's contiguous dimension, de-interleaved in registers (and transposed for
// M/N-contiguous operands) into the two planes, each stored in the XOR-swizzled K-contiguous
// layout of the real general kernel; double-buffered LDS, one barrier per slab.  The real part
// of a complex product subtracts A.im*B.im: the A.im fragment is negated (sign bits flipped)
// before that MFMA.  Epilogue: D = alpha * acc + beta * C with real alpha, beta, on both parts,
// interleaved store with edge masks.
//
// Compiled once; instantiated for complex/dual, fp32/fp16 output and the four layouts.  Plans
// large enough for the real fast kernel run the product as a real one on 2 x 2 blocks instead
// (PairJob in gemm_repack.hip, measured 1.3-1.45x faster at 4096^3); this kernel takes the
// smaller shapes and any run whose plan has no workspace for the rewritten operands yet.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

constexpr int CBM = 128, CBN = 128;      // output tile (numbers)
constexpr int CBK = 64;                  // numbers of K per slab
constexpr int CNT = 256;                 // 4 waves
constexpr int PLANE = 128 * 128;         // bytes of one part-plane of one operand: 128 rows x 64 fp16
constexpr int CSTAGE = 4 * PLANE;        // A.re, A.im, B.re, B.im

__device__ __forceinline__ int cswz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int coff(int row, int chunk) { return (row * 8 + (chunk ^ cswz(row))) * 16; }

// real / imaginary halves of two interleaved dwords (re | im << 16): the two reals, the two
// imaginaries packed as one dword each
__device__ __forceinline__ uint32_t lo2(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// K-contiguous operand (rows = M or N index, numbers along K at base[row*ld + k], 4 bytes each):
// a work item is 8 consecutive numbers of one row (two 16-byte loads), 4 items per thread.
struct CStagerK {
    u32x4 r[4][2];
    __device__ __forceinline__ void load(const uint8_t *base, int ld, int row0, int rows_valid,
                                         int k0, int K, int tid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + CNT * i, row = q >> 3, c = q & 7;   // 8 groups of 8 numbers
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = k0 + 8 * c + 4 * h;
                const uint8_t *p = base + ((int64_t)(row0 + row) * ld + k) * 4;
                if (row < rows_valid && k + 4 <= K) r[i][h] = ldg16(p);
                else if (row < rows_valid && k < K) r[i][h] = ldg16_partial<4>(p, K - k);
                else r[i][h] = u32x4{0, 0, 0, 0};
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t *re, uint8_t *im, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + CNT * i, row = q >> 3, c = q & 7;
            const u32x4 a = r[i][0], b = r[i][1];
            u32x4 vr, vi;
            vr[0] = lo2(a[0], a[1]); vr[1] = lo2(a[2], a[3]); vr[2] = lo2(b[0], b[1]); vr[3] = lo2(b[2], b[3]);
            vi[0] = hi2(a[0], a[1]); vi[1] = hi2(a[2], a[3]); vi[2] = hi2(b[0], b[1]); vi[3] = hi2(b[2], b[3]);
            *reinterpret_cast<u32x4 *>(re + coff(row, c)) = vr;
            *reinterpret_cast<u32x4 *>(im + coff(row, c)) = vi;
        }
    }
};

// M/N-contiguous operand (numbers of a row index at base[k*ld + row]): a work item is a block of
// 8 k x 4 rows (eight 16-byte loads), one per thread; it yields one 8-number chunk per row and
// part.
struct CStagerT {
    u32x4 r[8];
    __device__ __forceinline__ void load(const uint8_t *base, int ld, int row0, int rows_valid,
                                         int k0, int K, int tid) {
        const int mc = tid % 32, kg = tid / 32;                     // 32 row groups x 8 k groups
        const int rowl = 4 * mc;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = k0 + 8 * kg + kk;
            const uint8_t *p = base + ((int64_t)k * ld + row0 + rowl) * 4;
            if (k < K && rowl + 4 <= rows_valid) r[kk] = ldg16(p);
            else if (k < K && rowl < rows_valid) r[kk] = ldg16_partial<4>(p, rows_valid - rowl);
            else r[kk] = u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint8_t *re, uint8_t *im, int tid) const {
        const int mc = tid % 32, kg = tid / 32;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u32x4 vr, vi;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = r[2 * w][e], b = r[2 * w + 1][e];
                vr[w] = lo2(a, b);
                vi[w] = hi2(a, b);
            }
            *reinterpret_cast<u32x4 *>(re + coff(4 * mc + e, kg)) = vr;
            *reinterpret_cast<u32x4 *>(im + coff(4 * mc + e, kg)) = vi;
        }
    }
};

__device__ __forceinline__ u32x4 negate_f16x8(u32x4 v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] ^= 0x80008000u;
    return v;
}

template <class TO, bool DUAL, bool AT, bool BT>
__global__ __launch_bounds__(CNT, 1) void gemm_complex(GemmParams p) {
    using T = typename TO::T;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * CSTAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tile_m, tile_n;
    const int id = select_batch<4, 2 * (int)sizeof(T)>(p, xcd_remap(blockIdx.x, gridDim.x),
                                                     p.tiles_m * p.tiles_n);
    raster(id, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
    const int m0 = tile_m * CBM, n0 = tile_n * CBN;
    const int m_valid = p.M - m0, n_valid = p.N - n0;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);

    typename std::conditional<AT, CStagerT, CStagerK>::type sa;
    typename std::conditional<BT, CStagerK, CStagerT>::type sb;

    f32x16 accr[2][2], acci[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) accr[i][j][r] = acci[i][j][r] = 0.0f;

    auto stage_planes = [&](uint8_t *st) {
        sa.store(st, st + PLANE, tid);
        sb.store(st + 2 * PLANE, st + 3 * PLANE, tid);
    };
    const int nk = (p.K + CBK - 1) / CBK;
    if (nk > 0) {
        sa.load(A, p.lda, m0, m_valid, 0, p.K, tid);
        sb.load(B, p.ldb, n0, n_valid, 0, p.K, tid);
        stage_planes(smem);
    }
    __syncthreads();

    const int arow = wm * 64 + (lane & 31);
    const int brow = wn * 64 + (lane & 31);
    const int khalf = lane >> 5;

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * CBK;
            sa.load(A, p.lda, m0, m_valid, k0, p.K, tid);
            sb.load(B, p.ldb, n0, n_valid, k0, p.K, tid);
        }
        const uint8_t *st = smem + cur * CSTAGE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 2 * ks + khalf;
            u32x4 ar[2], ai[2], br[2], bi[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ar[i] = *reinterpret_cast<const u32x4 *>(st + coff(arow + 32 * i, c));
                ai[i] = *reinterpret_cast<const u32x4 *>(st + PLANE + coff(arow + 32 * i, c));
                br[i] = *reinterpret_cast<const u32x4 *>(st + 2 * PLANE + coff(brow + 32 * i, c));
                bi[i] = *reinterpret_cast<const u32x4 *>(st + 3 * PLANE + coff(brow + 32 * i, c));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x4 ain = negate_f16x8(ai[i]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // operands swapped (B first) so a lane holds 4 consecutive columns of a row
                    accr[i][j] = TF16::mma(br[j], ar[i], accr[i][j]);
                    if constexpr (!DUAL) accr[i][j] = TF16::mma(bi[j], ain, accr[i][j]);
                    acci[i][j] = TF16::mma(bi[j], ar[i], acci[i][j]);
                    acci[i][j] = TF16::mma(br[j], ai[i], acci[i][j]);
                }
            }
        }
        if (more) stage_planes(smem + (cur ^ 1) * CSTAGE);
        __syncthreads();
    }

    // epilogue: lane holds row 32i + l%32, columns 32j + 8g + 4(l/32) + e (e = 0..3) of each
    // part; D and C are interleaved (re, im) numbers of type T
    const int hi = lane >> 5, rl = lane & 31;
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + 32 * i + rl;
        if (m >= p.M) continue;
        const int64_t row = (int64_t)m * p.ldc;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 64 + 32 * j + 8 * g + 4 * hi;
                T out[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float tr = p.alpha * accr[i][j][4 * g + e];
                    float ti = p.alpha * acci[i][j][4 * g + e];
                    if (p.has_beta && n + e < p.N) {
                        tr += p.beta * (float)C[2 * (row + n + e)];
                        ti += p.beta * (float)C[2 * (row + n + e) + 1];
                    }
                    out[2 * e] = (T)tr;
                    out[2 * e + 1] = (T)ti;
                }
                if (n + 4 <= p.N) {
                    __builtin_memcpy(D + 2 * (row + n), out, sizeof(out));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) {
                            D[2 * (row + n + e)] = out[2 * e];
                            D[2 * (row + n + e) + 1] = out[2 * e + 1];
                        }
                }
            }
    }
}

template <class TO, bool DUAL, bool AT, bool BT>
hipError_t launch_complex(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_complex<TO, DUAL, AT, BT>), dim3(grid), dim3(CNT), 0, s, p);
    return hipGetLastError();
}

template <class TO, bool DUAL>
const KernelEntry *lookup_complex(int op_a, int op_b) {
    static const KernelEntry e[4] = {
        {launch_complex<TO, DUAL, false, false>, CBM, CBN, CBK, 2, 2, DUAL ? "gemm_dual_128x128" : "gemm_complex_128x128"},
        {launch_complex<TO, DUAL, false, true>, CBM, CBN, CBK, 2, 2, DUAL ? "gemm_dual_128x128" : "gemm_complex_128x128"},
        {launch_complex<TO, DUAL, true, false>, CBM, CBN, CBK, 2, 2, DUAL ? "gemm_dual_128x128" : "gemm_complex_128x128"},
        {launch_complex<TO, DUAL, true, true>, CBM, CBN, CBK, 2, 2, DUAL ? "gemm_dual_128x128" : "gemm_complex_128x128"},
    };
    if (op_a < 0 || op_a > 1 || op_b < 0 || op_b > 1) return nullptr;
    return &e[op_a * 2 + op_b];
}

}  // namespace

const KernelEntry *complex_cf16_cf32(int a, int b) { return lookup_complex<OF32, false>(a, b); }
const KernelEntry *complex_cf16_cf16(int a, int b) { return lookup_complex<OF16, false>(a, b); }
const KernelEntry *complex_df16_df32(int a, int b) { return lookup_complex<OF32, true>(a, b); }
const KernelEntry *complex_df16_df16(int a, int b) { return lookup_complex<OF16, true>(a, b); }

}  // namespace tge
