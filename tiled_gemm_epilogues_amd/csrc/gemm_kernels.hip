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

#include <type_traits>

#include "gemm_internal.h"

namespace tge {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- element types ---------------------------------------------------------------------------
// Every MFMA step consumes 16 bytes of K per lane for each operand: 8 fp16/bf16, 16 int8, or
// 4 fp32 (4 chained 32x32x2 instructions).

struct TF16 {
    static constexpr int E = 2;
    using acc_t = float;
    using accv_t = f32x16;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
struct TBF16 {
    static constexpr int E = 2;
    using acc_t = float;
    using accv_t = f32x16;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
struct TI8 {
    static constexpr int E = 1;
    using acc_t = int;
    using accv_t = i32x16;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};
struct TF32 {
    static constexpr int E = 4;
    using acc_t = float;
    using accv_t = f32x16;
    // lanes 0-31 and 32-63 each supply 4 consecutive k; instruction j takes element j of both,
    // so the 4 instructions together cover 8 distinct k exactly once.
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // copy the element out first: bit_cast of a vector-element lvalue reads element 0
            const uint32_t aj = a[j], bj = b[j];
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, aj),
                                                     __builtin_bit_cast(float, bj), c, 0, 0, 0);
        }
        return c;
    }
};

// output element types
struct OF16 { using T = _Float16; static constexpr int E = 2; };
struct OBF16 { using T = __bf16; static constexpr int E = 2; };
struct OF32 { using T = float; static constexpr int E = 4; };
struct OI32 { using T = int; static constexpr int E = 4; };

// ---- small helpers ---------------------------------------------------------------------------

// 16-byte global load with no alignment requirement (gfx950 serves unaligned dwordx4 loads).
__device__ __forceinline__ u32x4 ldg16(const uint8_t *p) {
    u32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// Element-wise 16-byte chunk load: elements with index e < nvalid are read, the rest are 0.
template <int E>
__device__ __forceinline__ u32x4 ldg16_partial(const uint8_t *p, int nvalid) {
    uint8_t tmp[16];
#pragma unroll
    for (int e = 0; e < 16 / E; ++e) {
        if (e < nvalid) {
#pragma unroll
            for (int b = 0; b < E; ++b) tmp[e * E + b] = p[e * E + b];
        } else {
#pragma unroll
            for (int b = 0; b < E; ++b) tmp[e * E + b] = 0;
        }
    }
    u32x4 v;
    __builtin_memcpy(&v, tmp, 16);
    return v;
}

// Physical 16-byte chunk of logical chunk c in LDS row r (8 chunks of 16 bytes per row).
// (r ^ r>>3) & 7 differs for 8 consecutive rows (fragment reads walk rows) and for rows
// 8 apart (the transposing stage writes rows 8 apart from consecutive lanes).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) { return (row * 8 + (chunk ^ swz(row))) * 16; }

// Transpose a VE x VE block of E-byte elements held as VE rows of 16 bytes.
template <int E>
__device__ __forceinline__ void transpose_block(const u32x4 *in, u32x4 *out);

template <>
__device__ __forceinline__ void transpose_block<2>(const u32x4 *in, u32x4 *out) {
    // out[e] word w = (in[2w] half e, in[2w+1] half e)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t lo = in[2 * w][e >> 1], hi = in[2 * w + 1][e >> 1];
            // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the first
            out[e][w] = __builtin_amdgcn_perm(hi, lo, (e & 1) ? 0x07060302u : 0x05040100u);
        }
}

template <>
__device__ __forceinline__ void transpose_block<4>(const u32x4 *in, u32x4 *out) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[e][r] = in[r][e];
}

template <>
__device__ __forceinline__ void transpose_block<1>(const u32x4 *in, u32x4 *out) {
    // out[e] byte r = in[r] byte e.  First gather 4 rows' byte e into one word with two
    // permutes per word.
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int wsel = e >> 2, bsel = e & 3;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t x0 = in[4 * w + 0][wsel], x1 = in[4 * w + 1][wsel];
            uint32_t x2 = in[4 * w + 2][wsel], x3 = in[4 * w + 3][wsel];
            // pick byte bsel of x0 (low) and x1 (next), then of x2, x3
            uint32_t s01 = __builtin_amdgcn_perm(x1, x0, (uint32_t)(bsel | ((bsel + 4) << 8)) | 0x0c0c0000u);
            uint32_t s23 = __builtin_amdgcn_perm(x3, x2, (uint32_t)(bsel | ((bsel + 4) << 8)) | 0x0c0c0000u);
            out[e][w] = (s01 & 0xffffu) | (s23 << 16);
        }
    }
}

// XCD-aware re-mapping: the hardware hands workgroup w to XCD w % 8.  Give each XCD a
// contiguous range of logical tile ids so the tiles resident on one XCD share its L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    constexpr int NX = 8;
    int q = nwg / NX, r = nwg % NX;
    int x = wg % NX, i = wg / NX;
    return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Grouped raster: consecutive ids walk down group_m tile rows, then move one tile column.
__device__ __forceinline__ void raster(int id, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
    int per_group = group_m * tiles_n;
    int g = id / per_group;
    int first = g * group_m;
    int gm = min(tiles_m - first, group_m);
    int in = id - g * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

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
    __device__ __forceinline__ void store(uint8_t *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int q = tid + NT * i, row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4 *>(lds + lds_off(row, c)) = r[i];
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
    __device__ __forceinline__ void store(uint8_t *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int b = tid + NT * i;
            if (NBLK % NT != 0 && b >= NBLK) break;
            int mc = b % NCH, kg = b / NCH;
            u32x4 t[VE];
            transpose_block<E>(r[i], t);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                *reinterpret_cast<u32x4 *>(lds + lds_off(mc * VE + e, kg)) = t[e];
        }
    }
};

// ---- epilogue --------------------------------------------------------------------------------

template <class O>
__device__ __forceinline__ float cd_to_f32(typename O::T v) { return (float)v; }

template <class O, class Acc>
__device__ __forceinline__ void epilogue4(const GemmParams &p, int m, int n, const Acc v[4]) {
    using T = typename O::T;
    const int N = p.N;
    const int64_t row = (int64_t)m * p.ldc;
    T out[4];
    if constexpr (std::is_same<Acc, int>::value) {
        // integer path: alpha == 1, beta in {0, 1}
        int t[4];
        const int *bias = static_cast<const int *>(p.bias);
        const T *C = static_cast<const T *>(p.C);
        if (n + 3 < N) {
            int cv[4] = {0, 0, 0, 0}, bv[4] = {0, 0, 0, 0};
            if (p.has_beta) __builtin_memcpy(cv, C + row + n, 16);
            if (p.has_bias) __builtin_memcpy(bv, bias + n, 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = v[e] + cv[e] + bv[e];
                if (p.relu) t[e] = max(t[e], 0);
                out[e] = t[e];
            }
            __builtin_memcpy(static_cast<T *>(p.D) + row + n, out, sizeof(out));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e >= N) break;
                int x = v[e];
                if (p.has_beta) x += C[row + n + e];
                if (p.has_bias) x += bias[n + e];
                if (p.relu) x = max(x, 0);
                static_cast<T *>(p.D)[row + n + e] = x;
            }
        }
    } else {
        const float *bias = static_cast<const float *>(p.bias);
        const T *C = static_cast<const T *>(p.C);
        if (n + 3 < N) {
            float t[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = p.alpha * v[e];
            if (p.has_beta) {
                T cv[4];
                __builtin_memcpy(cv, C + row + n, sizeof(cv));
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] += p.beta * cd_to_f32<O>(cv[e]);
            }
            if (p.has_bias) {
                float bv[4];
                __builtin_memcpy(bv, bias + n, 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] += bv[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (p.relu) t[e] = t[e] > 0.0f ? t[e] : 0.0f;
                out[e] = (T)t[e];
            }
            __builtin_memcpy(static_cast<T *>(p.D) + row + n, out, sizeof(out));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e >= N) break;
                float x = p.alpha * v[e];
                if (p.has_beta) x += p.beta * cd_to_f32<O>(C[row + n + e]);
                if (p.has_bias) x += bias[n + e];
                if (p.relu) x = x > 0.0f ? x : 0.0f;
                static_cast<T *>(p.D)[row + n + e] = (T)x;
            }
        }
    }
}

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
    raster(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int m_valid = p.M - m0, n_valid = p.N - n0;
    const bool mn_interior = m_valid >= BM && n_valid >= BN;

    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);

    Stager<E, BM, NT, !AT> sa;
    Stager<E, BN, NT, BT> sb;

    accv_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = (p.K + BK - 1) / BK;
    if (nk > 0) {
        bool interior = mn_interior && BK <= p.K;
        sa.load(A, p.lda, m0, m_valid, 0, p.K, interior, tid);
        sb.load(B, p.ldb, n0, n_valid, 0, p.K, interior, tid);
        sa.store(smem, tid);
        sb.store(smem + BM * 128, tid);
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
            int k0 = (kt + 1) * BK;
            bool interior = mn_interior && k0 + BK <= p.K;
            sa.load(A, p.lda, m0, m_valid, k0, p.K, interior, tid);
            sb.load(B, p.ldb, n0, n_valid, k0, p.K, interior, tid);
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
            sa.store(nxt, tid);
            sb.store(nxt + BM * 128, tid);
        }
        __syncthreads();
    }

    // epilogue: lane holds D[m][n .. n+3] for 4 column groups per MFMA tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WTM + 32 * i + (lane & 31);
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + 32 * j + 8 * g + 4 * khalf;
                acc_t v[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                              acc[i][j][4 * g + 3]};
                epilogue4<TO, acc_t>(p, m, n, v);
            }
    }
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
