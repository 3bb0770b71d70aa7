// Hierarchical tiled GEMM with a fused register epilogue for gfx950 (MI355X, CDNA4).
//
// One workgroup computes one BM x BN tile of D; its waves each own a (BM/waves_m) x
// (BN/waves_n) sub-tile made of 32x32 MFMA tiles; K is walked in slabs of 128 bytes.  This is
// the recursive blocking of "Flexible Performant GEMM Kernels on GPUs" (section 3: global ->
// shared -> registers, matrix-multiply-accumulate per tile, one store of D) and the thread-block
// / warp hierarchy of "CUTLASS: Fast Linear Algebra in CUDA C++" ("Hierarchical GEMM
// Structure"), re-done for 64-wide waves, LDS and MFMA:
//
//  * tile scheduler: workgroup ids are re-mapped so that each of the 8 XCDs (each with its own
//    L2) works on a contiguous band of a grouped raster order of the output tiles;
//  * global -> LDS staging: 16-byte loads along each operand's contiguous dimension; operands
//    whose contiguous dimension is M or N (A stored transposed, B not transposed) are transposed
//    in registers as 16-byte blocks, so LDS always holds both operands K-contiguous ("layouts
//    handled while loading", Flexible GEMM paper section 5.1); rows are XOR-swizzled in
//    16-byte chunks so fragment reads and staging writes avoid bank conflicts (the paper's
//    section 5.1 pads shared memory for the same reason and names swizzling as the missing
//    piece);
//  * double-buffered LDS with the next slab's global loads in flight during the current slab's
//    MFMAs, one barrier per slab ("Software Pipelining" in the CUTLASS page);
//  * MFMA operands are fed swapped (op(B) as the instruction's A input, op(A) as its B input),
//    so each lane's accumulators hold 4 consecutive columns of one row of D: the epilogue
//    loads bias and C and stores D 4 elements at a time;
//  * the epilogue alpha*acc + beta*C + bias[j], max(0, .), convert, runs on the accumulator
//    registers before the single store ("Fusing Element-wise Operations" in the CUTLASS page);
//  * ragged M/N/K: tiles that reach past an edge take a guarded load path that zero-fills
//    out-of-range elements; stores are masked per element.
//
// Compiled once per (input type, output type) pair, selected with TGE_PAIR.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

// ---- small helpers ---------------------------------------------------------------------------

// Physical 16-byte chunk of logical chunk c in LDS row r (8 chunks of 16 bytes per row).
// (r ^ r>>3) & 7 differs for 8 consecutive rows (fragment reads walk rows) and for rows
// 8 apart (the transposing stage writes rows 8 apart from consecutive lanes).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) { return (row * 8 + (chunk ^ swz(row))) * 16; }

// ---- operand staging -------------------------------------------------------------------------
// Side view of one operand: rows are the M (for A) or N (for B) index, columns the K index.
// KCONTIG: element (row, k) at base[row*ld + k];  otherwise at base[k*ld + row].

template <int E, int BMN, int NT, bool KCONTIG>
struct Stager;

template <int E, int BMN, int NT>
struct Stager<E, BMN, NT, true> {
    static constexpr int VE = 16 / E;
    static constexpr int CH = BMN * 8 / NT;   // 16-byte chunks per thread per slab
    static_assert(BMN * 8 % NT == 0, "tile rows must cover the threads");
    u32x4 r[CH];

    __device__ __forceinline__ void load(const uint8_t *base, int ld, int row0, int rows_valid,
                                         int k0, int K, bool interior, int tid) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int q = tid + NT * i, row = q >> 3, c = q & 7;
            int k = k0 + c * VE;
            const uint8_t *p = base + ((int64_t)(row0 + row) * ld + k) * E;
            if (interior) {
                r[i] = ldg16(p);
            } else if (row < rows_valid && k + VE <= K) {
                r[i] = ldg16(p);
            } else if (row < rows_valid && k < K) {
                r[i] = ldg16_partial<E>(p, K - k);
            } else {
                r[i] = u32x4{0, 0, 0, 0};
            }
        }
    }
    // xf: the load transform (sign bit set -> +0) on the staged values
    __device__ __forceinline__ void store(uint8_t *lds, int tid, int xf) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int q = tid + NT * i, row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4 *>(lds + lds_off(row, c)) = zero_negative<E>(r[i], xf);
        }
    }
};

template <int E, int BMN, int NT>
struct Stager<E, BMN, NT, false> {
    static constexpr int VE = 16 / E;
    static constexpr int NCH = BMN / VE;            // 16-byte chunks along the row index
    static constexpr int NBLK = 8 * NCH;            // VE x VE blocks per slab (8 k groups)
    static constexpr int NB = (NBLK + NT - 1) / NT; // blocks per thread
    u32x4 r[NB][VE];

    __device__ __forceinline__ void load(const uint8_t *base, int ld, int row0, int rows_valid,
                                         int k0, int K, bool interior, int tid) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int b = tid + NT * i;
            if (NBLK % NT != 0 && b >= NBLK) break;
            int mc = b % NCH, kg = b / NCH;
            int rowl = mc * VE;
#pragma unroll
            for (int rr = 0; rr < VE; ++rr) {
                int k = k0 + kg * VE + rr;
                const uint8_t *p = base + ((int64_t)k * ld + row0 + rowl) * E;
                if (interior) {
                    r[i][rr] = ldg16(p);
                } else if (k < K && rowl + VE <= rows_valid) {
                    r[i][rr] = ldg16(p);
                } else if (k < K && rowl < rows_valid) {
                    r[i][rr] = ldg16_partial<E>(p, rows_valid - rowl);
                } else {
                    r[i][rr] = u32x4{0, 0, 0, 0};
                }
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t *lds, int tid, int xf) const {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int b = tid + NT * i;
            if (NBLK % NT != 0 && b >= NBLK) break;
            int mc = b % NCH, kg = b / NCH;
            u32x4 t[VE], x[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) x[e] = zero_negative<E>(r[i][e], xf);
            transpose_block<E>(x, t);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                *reinterpret_cast<u32x4 *>(lds + lds_off(mc * VE + e, kg)) = t[e];
        }
    }
};

// ---- the kernel ------------------------------------------------------------------------------

template <int BM, int BN, int WGM, int WGN, class TI, class TO, bool AT, bool BT>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void gemm_mfma(GemmParams p) {
    constexpr int NT = WGM * WGN * 64;
    constexpr int E = TI::E;
    constexpr int BK = 128 / E;            // K elements per slab (128 bytes)
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int STAGE = (BM + BN) * 128; // bytes of one LDS stage
    using accv_t = typename TI::accv_t;
    using acc_t = typename TI::acc_t;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    int tile_m, tile_n;
    const int tid_in = select_batch<TI::E, (int)sizeof(typename TO::T)>(
        p, xcd_remap(blockIdx.x, gridDim.x), p.tiles_m * p.tiles_n);
    raster(tid_in, p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int m_valid = p.M - m0, n_valid = p.N - n0;
    const bool mn_interior = m_valid >= BM && n_valid >= BN;

    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);

    Stager<E, BM, NT, !AT> sa;
    Stager<E, BN, NT, BT> sb;
    // load slab at K offset k0 into the stagers
    auto load = [&](int k0, bool interior) {
        sa.load(A, p.lda, m0, m_valid, k0, p.K, interior, tid);
        sb.load(B, p.ldb, n0, n_valid, k0, p.K, interior, tid);
    };

    accv_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = (p.K + BK - 1) / BK;   // K slabs
    if (nk > 0) {
        load(0, mn_interior && BK <= p.K);
        sa.store(smem, tid, p.xform_a);
        sb.store(smem + BM * 128, tid, p.xform_b);
    }
    __syncthreads();

    // fragment rows of this lane inside the stage
    const int arow = wm * WTM + (lane & 31);
    const int brow = wn * WTN + (lane & 31);
    const int khalf = lane >> 5;

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * BK;
            load(k0, mn_interior && k0 + BK <= p.K);
        }
        const uint8_t *la = smem + cur * STAGE;
        const uint8_t *lb = la + BM * 128;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 af[TM], bf[TN];
            const int c = 2 * ks + khalf;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(la + lds_off(arow + 32 * i, c));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const u32x4 *>(lb + lds_off(brow + 32 * j, c));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = TI::mma(bf[j], af[i], acc[i][j]);
        }
        if (more) {
            uint8_t *nxt = smem + (cur ^ 1) * STAGE;
            sa.store(nxt, tid, p.xform_a);
            sb.store(nxt + BM * 128, tid, p.xform_b);
        }
        __syncthreads();
    }

    store_tile<TO, acc_t>(p, m0 + wm * WTM, n0 + wn * WTN, lane, acc);
}

template <int BM, int BN, int WGM, int WGN, class TI, class TO, bool AT, bool BT>
hipError_t launch(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_mfma<BM, BN, WGM, WGN, TI, TO, AT, BT>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, s, p);
    return hipGetLastError();
}

#define TGE_STR2(x) #x
#define TGE_STR(x) TGE_STR2(x)

template <class TI, class TO, bool AT, bool BT>
struct Table {
    static constexpr int BKE = 128 / TI::E;
    static const KernelEntry *get(int cfg) {
        static const KernelEntry e[CFG_COUNT] = {
            {launch<256, 256, 2, 2, TI, TO, AT, BT>, 256, 256, BKE, 2, 2, "gemm_mfma_256x256"},
            {launch<128, 128, 2, 2, TI, TO, AT, BT>, 128, 128, BKE, 2, 2, "gemm_mfma_128x128"},
            {launch<64, 64, 2, 2, TI, TO, AT, BT>, 64, 64, BKE, 2, 2, "gemm_mfma_64x64"},
        };
        return (cfg >= 0 && cfg < CFG_COUNT) ? &e[cfg] : nullptr;
    }
};

template <class TI, class TO>
const KernelEntry *lookup(int op_a, int op_b, int cfg) {
    if (op_a == 0 && op_b == 0) return Table<TI, TO, false, false>::get(cfg);
    if (op_a == 0 && op_b == 1) return Table<TI, TO, false, true>::get(cfg);
    if (op_a == 1 && op_b == 0) return Table<TI, TO, true, false>::get(cfg);
    if (op_a == 1 && op_b == 1) return Table<TI, TO, true, true>::get(cfg);
    return nullptr;
}

}  // namespace

#if defined(TGE_PAIR_F32_F32)
const KernelEntry *kernels_f32_f32(int a, int b, int c) { return lookup<TF32, OF32>(a, b, c); }
#elif defined(TGE_PAIR_F16_F16)
const KernelEntry *kernels_f16_f16(int a, int b, int c) { return lookup<TF16, OF16>(a, b, c); }
#elif defined(TGE_PAIR_F16_F32)
const KernelEntry *kernels_f16_f32(int a, int b, int c) { return lookup<TF16, OF32>(a, b, c); }
#elif defined(TGE_PAIR_BF16_BF16)
const KernelEntry *kernels_bf16_bf16(int a, int b, int c) { return lookup<TBF16, OBF16>(a, b, c); }
#elif defined(TGE_PAIR_BF16_F32)
const KernelEntry *kernels_bf16_f32(int a, int b, int c) { return lookup<TBF16, OF32>(a, b, c); }
#elif defined(TGE_PAIR_I8_I32)
const KernelEntry *kernels_i8_i32(int a, int b, int c) { return lookup<TI8, OI32>(a, b, c); }
#else
#error "define one TGE_PAIR_* macro"
#endif

}  // namespace tge
