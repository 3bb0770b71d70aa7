// Fast path for large fp16/bf16 GEMMs on gfx950: 256x256 output tile per workgroup, 4 waves of
// 128x128 (4x4 MFMA 32x32x16 tiles, accumulators in AGPRs), K walked in slabs of 64.
//
// The blocking follows "Flexible Performant GEMM Kernels on GPUs" (section 3: tiles copied up
// the memory hierarchy, global -> shared -> registers, then matrix-multiply-accumulate) and the
// software pipelining of "CUTLASS: Fast Linear Algebra in CUDA C++" ("Software Pipelining":
// loads for the next slab in flight while the current one is multiplied, one barrier per slab),
// re-done for the hardware:
//
//  * global -> LDS with direct-to-LDS 16-byte loads (global_load_lds_dwordx4): no staging
//    registers and no LDS write instructions.  One wave instruction fills 1 KiB of LDS, lane l
//    writing bytes [16l, 16l+16); the XOR swizzle is therefore applied on the global side by
//    choosing which 16-byte chunk each lane fetches.
//  * layouts are handled at load time without transposing through registers ("Flexible GEMM"
//    section 5.1 adapts its loaders to the N/T layout the same way): an operand whose contiguous
//    dimension is K is kept [mn][k] in LDS and read with ds_read_b128; an operand whose
//    contiguous dimension is M or N is kept [k][mn] and read with the gfx950 transposing LDS
//    read ds_read_b64_tr_b16, which hands each lane four consecutive-k values of one column.
//  * swizzles (bank-conflict avoidance, the role padding plays in "Flexible GEMM" section 5.1):
//    [mn][k] rows of 128 B hold logical 16-byte chunk c at c ^ ((r ^ r>>3) & 7); [k][mn] rows of
//    512 B hold chunk c at c ^ h(k & 3) with h = {0, 4, 10, 14}.  Both spread every group of
//    reads over distinct banks for 32- and 64-bank LDS organisations.
//  * pipeline per slab s (buffers X = s % 2, Y = the other): the fragments of k-slice j+1 are
//    read while the MFMAs of k-slice j run; after the last read of X the wave waits for its own
//    loads of slab s+1 and joins the barrier; then it issues the loads of slab s+2 into X and the
//    first fragment reads of Y while the last k-slice's MFMAs run.  The loop body holds two slabs
//    so that every stage index is a compile-time constant; the trips between the first and the
//    last ones carry no branches.
//  * M/N edges: source rows past the edge are clamped to the last valid row (their products
//    only reach output rows/columns that the masked epilogue drops); the K tail (K % slab) runs
//    one guarded register-staged slab with zero fill.
//  * epilogue (the epilogue building block of "Flexible GEMM" section 4, fused as in the bias and
//    ReLU functor of "CUTLASS", "Fusing Element-wise Operations"): alpha, beta*C, bias[j], ReLU
//    and the conversion run on the accumulators; the result goes through a per-wave LDS staging
//    buffer so that D is written in whole 128-byte lines.
//
// Preconditions (checked by the host): 16- or 8-bit inputs, A/B base pointers and leading
// dimensions 16-byte aligned, M (if A is stored transposed) and N (if B is not transposed)
// multiples of 16 bytes' worth of elements, K of at least one slab.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int BM = 256, BN = 256;                    // output tile
constexpr int SLAB_BYTES = 128;                      // K bytes per slab: 64 fp16/bf16 or 128 int8
constexpr int NT = 256;                              // 4 waves
constexpr int KC_BYTES = 256 * SLAB_BYTES;           // one operand slab: 32 KiB either layout
// LDS map: [A stage 0 | A stage 1 | B stage 0 | B stage 1], 32 KiB each, so that every fragment
// read is (base register) + (stage and k-slice offset as the instruction's 16-bit immediate)
constexpr int OPND = 2 * KC_BYTES;                   // byte offset of operand B's stages
// a slab's 16 direct loads go out one per DMA_STRIDE MFMA slots (see slab_step)
constexpr int DMA_STRIDE = 2;

// [mn][k] layout (K-contiguous operands): 256 rows of 128 B, 16-byte chunk c of row r at
// c ^ swz_kc(r); identical in bytes for 8- and 16-bit elements.
__device__ __forceinline__ int swz_kc(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int off_kc(int r, int c) { return r * 128 + ((c ^ swz_kc(r)) << 4); }

// [k][mn] layout (M/N-contiguous operands): 64 rows of 512 B (16-bit) or 128 rows of 256 B
// (8-bit).  The transposing reads touch, per group of lanes served together, 4 (16-bit) or 8
// (8-bit) consecutive rows at 2 adjacent 16-byte chunks; the swizzle gives those accesses
// distinct banks for 32- and 64-bank LDS.
template <int E>
__device__ __forceinline__ int swz_mc(int k) {
    if constexpr (E == 2) {
        const int q = k & 3;
        return 4 * q + 2 * (q >> 1);
    } else {
        const int q = k & 7;
        return 2 * q + (q >> 2);
    }
}
template <int E>
__device__ __forceinline__ int off_mc(int k, int c) { return k * 256 * E + ((c ^ swz_mc<E>(k)) << 4); }

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// One direct-to-LDS 16-byte load per lane: global address sbase + voff (bytes), LDS destination
// lds + 16 * lane.  Issued as inline assembly so that the compiler does not treat the LDS write
// as aliasing every later LDS read (it would wait for the load before each read); completion is
// awaited explicitly with s_waitcnt vmcnt before the barrier that publishes the slab.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
                 :: "s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}

// ---- per-operand direct-load plan -----------------------------------------------------------
// Each wave issues 8 instructions (1 KiB each) per operand per slab.  For lane l and instruction
// i the byte offset from the slab's base address is fixed for the whole kernel.

template <int E, bool KC>
struct Loader {
    static constexpr int VE = 16 / E;    // elements per 16-byte chunk
    uint32_t voff[8];

    // row0: first M (or N) index of the tile; ext: M (or N); ld: leading dimension.
    __device__ __forceinline__ void init(int wave, int lane, int row0, int ext, int ld) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = wave * 8 + i;                          // 1 KiB block of the slab
            if constexpr (KC) {
                const int r = blk * 8 + (lane >> 3);               // tile row (8 rows of 128 B)
                const int c = (lane & 7) ^ swz_kc(r);              // logical chunk this lane fetches
                const int gr = min(row0 + r, ext - 1);
                voff[i] = (uint32_t)(gr * ld + c * VE) * (uint32_t)E;
            } else {
                constexpr int CPR = 16 * E;                        // chunks per [k] row
                const int k = blk * (64 / CPR) + lane / CPR;       // slab row (k)
                const int c = (lane % CPR) ^ swz_mc<E>(k);
                const int col = min(row0 + c * VE, ext - VE);      // ext % VE == 0: whole chunks
                voff[i] = (uint32_t)(k * ld + col) * (uint32_t)E;
            }
        }
    }
    // base of the slab whose K starts at element k0
    __device__ __forceinline__ static const uint8_t *slab_base(const uint8_t *base, int ld, int k0) {
        return KC ? base + (size_t)k0 * E : base + (size_t)k0 * ld * E;
    }
    // instruction i of this wave: LDS block (wave*8 + i) of the operand slab at `dst`
    __device__ __forceinline__ void issue(const uint8_t *sb, uint32_t dst, int wave, int i) const {
        dma16(sb, voff[i], dst + (uint32_t)(wave * 8 + i) * 1024u);
    }
};

// Guarded staging of a partial slab (k0 .. K-1, zero beyond) into the same LDS layout.
template <int E, bool KC>
__device__ __forceinline__ void stage_tail(const uint8_t *base, int ld, int row0, int ext, int k0, int K, uint8_t *dst,
                           int tid) {
    constexpr int VE = 16 / E;
    // 2048 chunks of 16 bytes per operand slab, 8 per thread
#pragma unroll 1
    for (int i = 0; i < 8; ++i) {
        const int q = tid + NT * i;
        uint8_t v[16];
        if constexpr (KC) {
            const int r = q >> 3, c = q & 7;
            const int gr = min(row0 + r, ext - 1);
            const uint8_t *p = base + ((size_t)gr * ld + k0 + c * VE) * E;
#pragma unroll
            for (int e = 0; e < VE; ++e)
#pragma unroll
                for (int b = 0; b < E; ++b) v[e * E + b] = (k0 + c * VE + e < K) ? p[e * E + b] : (uint8_t)0;
            __builtin_memcpy(dst + off_kc(r, c), v, 16);
        } else {
            constexpr int CPR = 16 * E;
            const int k = q / CPR, c = q % CPR;
            const int col = min(row0 + c * VE, ext - VE);
            if (k0 + k < K) {
                const uint8_t *p = base + ((size_t)(k0 + k) * ld + col) * E;
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = p[e];
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = 0;
            }
            __builtin_memcpy(dst + off_mc<E>(k, c), v, 16);
        }
    }
}

// ---- fragment reads ---------------------------------------------------------------------------
// Fragment (sub-tile t, k-slice j): lane l holds 16 bytes of consecutive k (8 fp16/bf16 or 16
// int8 values, k = j*KS + (l/32)*KS/2 + ..., KS = 32 bytes of K per k-slice) of tile row (or
// column) 32t + l%32.  A K-contiguous operand needs one ds_read_b128 per fragment, an
// M/N-contiguous one two transposing reads.

template <int E, bool KC>
struct Frag {
    static constexpr int NI = KC ? 1 : 2;   // LDS instructions per fragment
    // byte address (LDS) of this lane's fragment in stage 0: per sub-tile and k-slice for a
    // K-contiguous operand (the XOR swizzle is not additive), per sub-tile otherwise
    uint32_t addr[4][KC ? 4 : 1];

    __device__ __forceinline__ void init(int lane, int wrow, uint32_t opbase) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (KC) {
                const int r = wrow + 32 * t + (lane & 31);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    addr[t][j] = opbase + (uint32_t)off_kc(r, 2 * j + (lane >> 5));
            } else if constexpr (E == 2) {
                // ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i % 4
                // of the 8-byte chunks addressed by lanes i/4 + 4e, e = 0..3.  Lane a of the
                // group therefore addresses k row a/4 and columns 4*(a%4) .. +3.
                const int q = (lane & 15) >> 2;
                const int k = 8 * (lane >> 5) + q;
                const int col = wrow + 32 * t + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                addr[t][0] = opbase + (uint32_t)(k * 512 + (((col >> 3) ^ swz_mc<2>(k)) << 4) + (col & 7) * 2);
            } else {
                // ds_read_b64_tr_b8: in each group of 16 lanes, lane i receives byte i % 8 of
                // the 8-byte chunks addressed by lanes i/8 + 2e, e = 0..7.  Lane a of the group
                // therefore addresses k row a/2 and columns 8*(a%2) .. +7.
                const int a = lane & 15;
                const int k = 16 * (lane >> 5) + (a >> 1);
                const int col = wrow + 32 * t + 16 * ((lane >> 4) & 1) + 8 * (a & 1);
                addr[t][0] = opbase + (uint32_t)(k * 256 + (((col >> 4) ^ swz_mc<1>(k)) << 4) + (col & 15));
            }
        }
    }
    // instruction h (< NI) of fragment (t, j) of `stage` into dst
    __device__ __forceinline__ void read(int stage, int t, int j, int h, u32x4 &dst) const {
        if constexpr (KC) {
            dst = *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)(addr[t][j] + stage * KC_BYTES);
        } else if constexpr (E == 2) {
            // rows 16j + 4h + (0..3): the swizzle depends only on k & 3
            const uint32_t a = addr[t][0] + stage * KC_BYTES + (16 * j + 4 * h) * 512;
            s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a);
            dst[2 * h] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v, v, 0, 1));
            dst[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v, v, 2, 3));
        } else {
            // rows 32j + 8h + (0..7): the swizzle depends only on k & 7
            const uint32_t a = addr[t][0] + stage * KC_BYTES + (32 * j + 8 * h) * 256;
            i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(uintptr_t)a);
            dst[2 * h] = (uint32_t)v[0];
            dst[2 * h + 1] = (uint32_t)v[1];
        }
    }
};

// ---- epilogue through LDS -------------------------------------------------------------------
// One wave's 128x128 sub-tile, 32 rows at a time: values are computed in the accumulator layout
// (alpha, beta*C, bias[j], ReLU, convert; lane l holds row 32i + l%32, columns 32j + 8g +
// 4(l/32) + e), written row-major into the wave's private staging buffer (16-byte chunk c of
// staged row r at c ^ (r % chunks-per-row)) and read back as 16-byte row pieces, so every store
// instruction writes whole 128-byte lines of D instead of 16-byte pieces of 32 rows.
//
// Vector-memory operations complete in issue order, so a load issued after a store can only be
// awaited together with that store.  Every load is therefore issued before the stores it would
// otherwise wait behind: the bias once before the first block, the C values of block i+1 before
// the stores of block i.
template <class O>
__device__ __forceinline__ constexpr int stg_bytes() { return 32 * 128 * (int)sizeof(typename O::T); }

template <class O, class Acc, bool BETA, bool FULL, class AccV>
__device__ __forceinline__ void store_tile_staged(const GemmParams &p, int mbase, int nbase, int lane,
                                                  AccV (&acc)[4][4], uint8_t *stg) {
    using T = typename O::T;
    constexpr bool INT = std::is_same<Acc, int>::value;
    using Bt = typename std::conditional<INT, int, float>::type;
    constexpr int ES = sizeof(T);
    constexpr int RB = 128 * ES;           // staged row bytes
    constexpr int CPR = RB / 16;           // 16-byte chunks per row
    constexpr int VE = 16 / ES;            // elements per chunk
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
    const int hi = lane >> 5, rl = lane & 31;
    const int M = p.M, N = p.N;
    const Bt *bias = static_cast<const Bt *>(p.bias);
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);

    // bias of this lane's 64 columns, shared by the four row blocks
    Bt bv[4][4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = nbase + 32 * j + 8 * g + 4 * hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[j][g][e] = 0;
            if (p.has_bias) {
                if constexpr (FULL) {
                    __builtin_memcpy(bv[j][g], bias + n, sizeof(bv[j][g]));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) bv[j][g][e] = bias[n + e];
                }
            }
        }
    // C values of row block i for this lane
    T cv[4][4][4];
    auto load_c = [&](int i) {
        const int m = mbase + 32 * i + rl;
        const int64_t row = (int64_t)(FULL ? m : min(m, M - 1)) * p.ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nbase + 32 * j + 8 * g + 4 * hi;
                if constexpr (FULL) {
                    __builtin_memcpy(cv[j][g], C + row + n, sizeof(cv[j][g]));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) cv[j][g][e] = n + e < N ? C[row + n + e] : (T)0;
                }
            }
    };
    if constexpr (BETA) load_c(0);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                T out[4];
                if constexpr (INT) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        int t = acc[i][j][4 * g + e] + bv[j][g][e];
                        if constexpr (BETA) t += (int)cv[j][g][e];
                        if (p.relu) t = max(t, 0);
                        out[e] = (T)t;
                    }
                } else {
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        t[e] = __builtin_fmaf(p.alpha, acc[i][j][4 * g + e], bv[j][g][e]);
                        if constexpr (BETA) t[e] = __builtin_fmaf(p.beta, (float)cv[j][g][e], t[e]);
                        if (p.relu) t[e] = __builtin_fmaxf(t[e], 0.0f);
                    }
                    if constexpr (ES == 2) {
                        // two-at-a-time conversion (round to nearest even)
                        const t2 lo = __builtin_convertvector((f32x2){t[0], t[1]}, t2);
                        const t2 hi2 = __builtin_convertvector((f32x2){t[2], t[3]}, t2);
                        out[0] = lo[0]; out[1] = lo[1]; out[2] = hi2[0]; out[3] = hi2[1];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = (T)t[e];
                    }
                }
                const int byte = (32 * j + 8 * g + 4 * hi) * ES;
                const int c = byte >> 4;
                __builtin_memcpy(stg + rl * RB + ((c ^ (rl % CPR)) << 4) + (byte & 15), out, 4 * ES);
            }
        if constexpr (BETA) {
            if (i < 3) load_c(i + 1);
        }
        // read back (the wave's LDS operations execute in order): 32 rows x CPR chunks, 16 bytes
        // per lane per round
#pragma unroll
        for (int q = 0; q < 32 * CPR / 64; ++q) {
            const int idx = q * 64 + lane;
            const int rr = idx / CPR, c = idx % CPR;
            u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rr * RB + ((c ^ (rr % CPR)) << 4));
            const int mg = mbase + 32 * i + rr;
            const int ng = nbase + c * VE;
            T *dst = D + (int64_t)mg * p.ldc + ng;
            if constexpr (FULL) {
                __builtin_memcpy(dst, &v, 16);
            } else if (mg < M) {
                if (ng + VE <= N) {
                    __builtin_memcpy(dst, &v, 16);
                } else {
                    T tv[VE];
                    __builtin_memcpy(tv, &v, 16);
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        if (ng + e < N) dst[e] = tv[e];
                }
            }
        }
    }
}

template <class O, class Acc, class AccV>
__device__ __forceinline__ void epilogue(const GemmParams &p, int mbase, int nbase, int lane,
                                         AccV (&acc)[4][4], uint8_t *stg) {
    // interior wave tiles (the common case) take a path with no edge checks
    const bool full = mbase + 128 <= p.M && nbase + 128 <= p.N;
    if (full) {
        if (p.has_beta) store_tile_staged<O, Acc, true, true>(p, mbase, nbase, lane, acc, stg);
        else store_tile_staged<O, Acc, false, true>(p, mbase, nbase, lane, acc, stg);
    } else {
        if (p.has_beta) store_tile_staged<O, Acc, true, false>(p, mbase, nbase, lane, acc, stg);
        else store_tile_staged<O, Acc, false, false>(p, mbase, nbase, lane, acc, stg);
    }
}

template <class TI, class TO, bool AK, bool BK>
__global__ __launch_bounds__(NT, 1) void gemm_fast(GemmParams p) {
    using accv_t = typename TI::accv_t;
    using acc_t = typename TI::acc_t;
    constexpr int E = TI::E;
    constexpr int BKE = SLAB_BYTES / E;       // K elements per slab
    using FA = Frag<E, AK>;
    using FB = Frag<E, BK>;
    // LDS instructions per k-slice, issued in the order the next k-slice's MFMAs consume them:
    // A0, B0, B1, B2, B3, A1, A2, A3 (each fragment 1 or 2 instructions)
    constexpr int NRD = 4 * FA::NI + 4 * FB::NI;
    // two pipeline stages of both operands; after the main loop the stage-1 halves of A and B
    // (never used by the K tail) hold the four waves' epilogue staging buffers
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * OPND];
    constexpr int STG = stg_bytes<TO>();
    static_assert(2 * STG <= KC_BYTES, "two staging buffers fit in one operand stage");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);   // this workgroup's raster id

    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const uint32_t lds0 = lds_addr(smem);
    uint8_t *const stg = smem + (wave < 2 ? 0 : OPND) + KC_BYTES + (wave & 1) * STG;

    FA fa;
    FB fb;
    Loader<E, AK> la;
    Loader<E, BK> lb;
    int m0 = 0, n0 = 0;
    auto set_tile = [&](int id) {
        int tm, tn;
        raster(id, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
        la.init(wave, lane, m0, p.M, p.lda);
        lb.init(wave, lane, n0, p.N, p.ldb);
    };

    const int nfull = p.K / BKE;
    accv_t acc[4][4];
    u32x4 af[2][4], bf[2][4];

    // read instruction q (0 .. NRD-1) of k-slice j of `stage` into fragment buffer `buf`
    auto rd = [&](int stage, int j, int buf, int q) {
        // fragment order A0, B0, B1, B2, B3, A1, A2, A3
        int idx = 0;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const bool isA = f == 0 || f >= 5;
            const int t = f == 0 ? 0 : (f <= 4 ? f - 1 : f - 4);
            const int ni = isA ? FA::NI : FB::NI;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h < ni) {
                    if (idx == q) {
                        if (isA) fa.read(stage, t, j, h, af[buf][t]);
                        else fb.read(stage, t, j, h, bf[buf][t]);
                    }
                    ++idx;
                }
            }
        }
    };
    // MFMA number t (0..15) of a k-slice: A fragment t/4 times B fragment t%4
    auto mma = [&](int buf, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = TI::mma(bf[buf][j], af[buf][i], acc[i][j]);
    };
    // LDS addresses of operand slabs in a stage
    auto dstA = [&](int st) { return lds0 + (uint32_t)(st * KC_BYTES); };
    auto dstB = [&](int st) { return lds0 + (uint32_t)(OPND + st * KC_BYTES); };
    auto issue_slab = [&](int s, int st) {
        const uint8_t *sa = Loader<E, AK>::slab_base(A, p.lda, s * BKE);
        const uint8_t *sb = Loader<E, BK>::slab_base(B, p.ldb, s * BKE);
#pragma unroll
        for (int i = 0; i < 8; ++i) la.issue(sa, dstA(st), wave, i);
#pragma unroll
        for (int i = 0; i < 8; ++i) lb.issue(sb, dstB(st), wave, i);
    };
    auto prologue = [&]() {
        if (nfull > 0) issue_slab(0, 0);
        if (nfull > 1) issue_slab(1, 1);
    };

    // Slab s reads stage X; slab s+1 lives in Y.  The 16 loads of a slab are spread one per
    // three MFMA slots over 47 slots: loads 0-4 of slab s+2 go out in k-slice 3 of slab s (after
    // the barrier has freed X), loads 5-15 of slab s+1 in k-slices 0 and 1 of slab s; k-slice 2
    // issues none, leaving time for the last ones to land before the barrier.  Bursting all 16
    // at once fills the vector-memory queue and stalls the wave's in-order issue (MFMAs too).
    //   dma_next:  issue loads 5-15 of slab s+1 into Y (its loads 0-4 went out in slab s-1)
    //   dma_next2: issue loads 0-4 of slab s+2 into X
    //   has_next:  slab s+1 exists (wait for it, read its k-slice 0)
    auto slab_step = [&](int s, int X, int Y, bool dma_next, bool dma_next2, bool has_next) {
        const uint8_t *na = Loader<E, AK>::slab_base(A, p.lda, (s + 1) * BKE);
        const uint8_t *nb = Loader<E, BK>::slab_base(B, p.ldb, (s + 1) * BKE);
        const uint8_t *n2a = Loader<E, AK>::slab_base(A, p.lda, (s + 2) * BKE);
        const uint8_t *n2b = Loader<E, BK>::slab_base(B, p.ldb, (s + 2) * BKE);
        auto dma = [&](const uint8_t *sa, const uint8_t *sb, int st, int d) {
            if (d < 8) la.issue(sa, dstA(st), wave, d);
            else lb.issue(sb, dstB(st), wave, d - 8);
        };
        // k-slices 0..2: MFMAs of slice j interleaved with the reads of slice j+1
#pragma unroll
        for (int j = 0; j < 3; ++j) {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(j & 1, t);
                if (t < NRD) rd(X, j + 1, (j + 1) & 1, t);
                if (dma_next) {
                    const int q = 15 + 16 * j + t;               // load slot 15..62
                    if (q % DMA_STRIDE == 0 && q / DMA_STRIDE < 16) dma(na, nb, Y, q / DMA_STRIDE);
                }
                fence();
            }
        }
        // k-slice 3: every read of X has been issued.  Finish them and our loads of slab s+1,
        // meet at the barrier (after one MFMA, so the matrix core is busy meanwhile), then
        // start refilling X with slab s+2 and read slice 0 of Y while the remaining MFMAs run.
        wait_lgkmcnt0();
        if (has_next) wait_vmcnt0();
        fence();
        mma(1, 0);
        fence();
        __syncthreads();
        fence();
#pragma unroll
        for (int t = 1; t < 16; ++t) {
            mma(1, t);
            if (dma_next2) {
                const int q = t - 1;                             // load slot 0..14
                if (q % DMA_STRIDE == 0) dma(n2a, n2b, X, q / DMA_STRIDE);
            }
            if (has_next) {
                if (t - 1 < NRD) rd(Y, 0, 0, t - 1);
                if (t == 15 && NRD == 16) rd(Y, 0, 0, 15);
            }
            fence();
        }
    };

    set_tile(lid);
    fa.init(lane, wm * 128, lds0);
    fb.init(lane, wn * 128, lds0 + OPND);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    if (nfull > 0) {
        prologue();
        // slab 0 landed, slab 1 may still fly
        if (nfull > 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else wait_vmcnt0();
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NRD; ++q) rd(0, 0, 0, q);
    }

    // two slabs per trip so the stage of every read and load is a compile-time constant.  The
    // first trip and the last ones take the flags as uniform branches (slab 1 was loaded whole by
    // the prologue); the trips in between have every flag set and no branches.
    auto trip = [&](int s) {
        [[clang::always_inline]] slab_step(s, 0, 1, s >= 1 && s + 1 < nfull, s + 2 < nfull, s + 1 < nfull);
        if (s + 1 < nfull)
            [[clang::always_inline]] slab_step(s + 1, 1, 0, s + 2 < nfull, s + 3 < nfull, s + 2 < nfull);
    };
    int s = 0;
    if (nfull > 0) {
        [[clang::always_inline]] trip(0);
        s = 2;
    }
#pragma unroll 1
    for (; s + 3 < nfull; s += 2) {
        [[clang::always_inline]] slab_step(s, 0, 1, true, true, true);
        [[clang::always_inline]] slab_step(s + 1, 1, 0, true, true, true);
    }
#pragma unroll 1
    for (; s < nfull; s += 2) [[clang::always_inline]] trip(s);

    // K tail: one guarded slab through registers (zero fill past K), in stage 0
    const int k0 = nfull * BKE;
    if (k0 < p.K) {
        __syncthreads();
        stage_tail<E, AK>(A, p.lda, m0, p.M, k0, p.K, smem, tid);
        stage_tail<E, BK>(B, p.ldb, n0, p.N, k0, p.K, smem + OPND, tid);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // the 4 k-slices of the slab
#pragma unroll
            for (int q = 0; q < NRD; ++q) rd(0, j, 0, q);
#pragma unroll
            for (int t = 0; t < 16; ++t) mma(0, t);
        }
    }

    // every wave's reads of the stage-1 buffers ended before the last slab's barrier
    epilogue<TO, acc_t>(p, m0 + wm * 128, n0 + wn * 128, lane, acc, stg);
}

template <class TI, class TO, bool AT, bool BT>
hipError_t launch_fast(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_fast<TI, TO, !AT, BT>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO>
const KernelEntry *lookup_fast(int op_a, int op_b) {
    constexpr int BKE = SLAB_BYTES / TI::E;
    static const KernelEntry e[4] = {
        {launch_fast<TI, TO, false, false>, BM, BN, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, false, true>, BM, BN, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, true, false>, BM, BN, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, true, true>, BM, BN, BKE, 2, 2, "gemm_fast_256x256"},
    };
    if (op_a < 0 || op_a > 1 || op_b < 0 || op_b > 1) return nullptr;
    return &e[op_a * 2 + op_b];
}

}  // namespace

#if defined(TGE_PAIR_F16_F16)
const KernelEntry *fast_f16_f16(int a, int b) { return lookup_fast<TF16, OF16>(a, b); }
#elif defined(TGE_PAIR_F16_F32)
const KernelEntry *fast_f16_f32(int a, int b) { return lookup_fast<TF16, OF32>(a, b); }
#elif defined(TGE_PAIR_BF16_BF16)
const KernelEntry *fast_bf16_bf16(int a, int b) { return lookup_fast<TBF16, OBF16>(a, b); }
#elif defined(TGE_PAIR_BF16_F32)
const KernelEntry *fast_bf16_f32(int a, int b) { return lookup_fast<TBF16, OF32>(a, b); }
#elif defined(TGE_PAIR_I8_I32)
const KernelEntry *fast_i8_i32(int a, int b) { return lookup_fast<TI8, OI32>(a, b); }
#else
#error "define one TGE_PAIR_* macro with a 16- or 8-bit input type"
#endif

}  // namespace tge
