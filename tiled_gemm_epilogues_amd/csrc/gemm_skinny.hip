// Memory-bound path for short-and-wide GEMMs on gfx950 (M <= 64, e.g. a fully-connected layer
// applied to a small batch): every byte of B is read once from HBM, so the kernel is built to
// keep enough loads in flight to stream B at full bandwidth rather than to maximise reuse.
// "CUTLASS: Fast Linear Algebra in CUDA C++" ("CUTLASS GEMM Strategies") specialises its tiling
// for tall and narrow shapes the same way; the shape here is the transposed case.
//
//  * one workgroup (one per CU: its LDS is the whole ring) per 64 output columns and k split:
//    a row of a non-transposed B is read as whole 128-byte lines; K is split S ways over
//    workgroups when the column blocks alone are too few to fill the chip (S chosen by the
//    plan), and over the 4 waves of a workgroup.  A transposed B (rows along K) can be read
//    16 output columns per workgroup instead, each of its rows still in whole lines: with
//    enough such blocks to fill the chip the plan takes that narrow variant and no k split;
//  * each wave streams its K range through a private ring of LDS slots with direct-to-LDS
//    loads (no barriers inside the loop: a wave only waits for its own loads): per k chunk of
//    64 bytes (32 k of 16-bit inputs, 64 of int8), 4 KiB of B (64 columns) and 1 KiB of A per
//    16 rows;
//  * fragments: A (K-contiguous) and a transposed B with ds_read_b128, a non-transposed B with
//    the transposing read ds_read_b64_tr_b16; MFMA 16x16x32 with fp32 accumulation (int8:
//    16x16x64 with int32 accumulation, the same 16 bytes of k per lane and operand);
//  * the four waves' partial sums are added through LDS; then either the fused epilogue
//    (alpha, beta*C, bias[j], ReLU, convert) and the store, or, with S > 1, the workgroup's
//    sums go to a workspace and a second small kernel adds the S splits in split order and
//    applies the epilogue (the kernel boundary orders the two; no device-wide fences, which
//    cost more than the whole product here).
//
// Preconditions (checked by the host): 16-bit inputs, or int8 inputs with B transposed; op(A) =
// A (not transposed), M <= 64, K a whole number of 64-byte chunks, A/B pointers and leading
// dimensions 16-byte aligned, N % 8 == 0 when B is not transposed; with S > 1 a workspace of
// S * M * N floats (int32 for int8) per product of the batch (one product for int8).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "gemm_internal.h"

namespace tge {
namespace {

using namespace dev;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int NT = 256;
constexpr int NB = 64;         // output columns per workgroup: whole 128-byte lines of a row of B
constexpr int NB_NARROW = 16;  // output columns per workgroup of the narrow variant (B transposed)
// k per chunk (one MFMA step): 64 bytes of every row of A and of a transposed B
template <class TI>
constexpr int kch() { return 64 / TI::E; }

// accumulators of one 16x16 MFMA tile: fp32, int32 for int8
template <class TI>
struct SkAcc { using type = f32x4; };
template <>
struct SkAcc<TI8> { using type = i32x4; };

template <class TI>
__device__ __forceinline__ typename SkAcc<TI>::type mma16(u32x4 a, u32x4 b, typename SkAcc<TI>::type c);
template <>
__device__ __forceinline__ f32x4 mma16<TF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma16<TBF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ i32x4 mma16<TI8>(u32x4 a, u32x4 b, i32x4 c) {
    return TI8::mma16(a, b, c);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}

// direct-to-LDS 16-byte load per lane (LDS destination lds + 16 * lane), see gemm_fast.hip
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
                 :: "s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// s_waitcnt vmcnt(n) for a run-time n (immediates only): rounds n down to a supported value,
// which only waits longer.
__device__ __forceinline__ void wait_vm_atmost(int n) {
    if (n >= 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
    else if (n >= 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    else if (n >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n >= 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// MT: 16-row tiles of A (M <= 16 * MT); BT: B is stored transposed (N x K); CB: output
// columns per workgroup (64, or 16 with B transposed).
// Grid: (k split, column block) pairs of every product: p.tiles_m holds the number of k splits
// S, p.tiles_n the number of CB-column blocks.
template <class TI, class TO, int MT, bool BT, int CB>
__global__ __launch_bounds__(NT, 1) void gemm_skinny(GemmParams p) {
    static_assert(CB == NB || (CB == NB_NARROW && BT), "narrow blocks need rows of B along K");
    static_assert(TI::E == 2 || BT, "int8: B transposed only (no transposing byte reads here)");
    constexpr int ES = TI::E;                           // input element bytes
    constexpr int KCH = kch<TI>();
    constexpr bool INT = ES == 1;
    using AV = typename SkAcc<TI>::type;
    constexpr int G = CB / 16;                          // 16-column groups (MFMA N tiles)
    constexpr int BCH = G;                              // 1 KiB loads per chunk of B (CB x 32 k)
    constexpr int DPC = BCH + MT;                       // load instructions per chunk
    constexpr int SLOT = DPC * 1024;                    // B chunk, then MT A chunks
    // ring depth per wave: as deep as the CU's 160 KiB of LDS and the vmcnt range allow
    constexpr int DEPTH = CB == NB ? (MT == 1 ? 8 : MT == 2 ? 6 : 5)
                                   : (MT == 1 ? 16 : MT == 2 ? 12 : MT == 3 ? 9 : 7);
    constexpr int STEADY = (DEPTH - 1) * DPC;           // loads in flight when waiting for one chunk
    constexpr int RING_BYTES = 4 * DEPTH * SLOT;
    static_assert(RING_BYTES <= 160 * 1024 && STEADY <= 63, "LDS budget, vmcnt range");
    static_assert(4 * MT * G * 64 * 16 <= RING_BYTES, "reduction area");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[RING_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per = p.tiles_m * p.tiles_n;
    const int prod = blockIdx.x / per;                  // product of the batch
    const int lid = select_batch<ES, (int)sizeof(typename TO::T)>(p, blockIdx.x, per);
    const int S = p.tiles_m;
    const int split = lid / p.tiles_n, cb = lid - split * p.tiles_n;
    const int n0 = cb * CB;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);

    // chunks [c0, c1) of this wave: the split's share of K, divided over the four waves
    const int nch_all = p.K / KCH;
    const int s0 = (int)((int64_t)nch_all * split / S), s1 = (int)((int64_t)nch_all * (split + 1) / S);
    const int c0 = s0 + (s1 - s0) * wave / 4, c1 = s0 + (s1 - s0) * (wave + 1) / 4;
    const int nch = c1 - c0;

    uint8_t *ring = smem + wave * DEPTH * SLOT;
    const uint32_t lring = lds_addr(ring);

    // per-lane load offsets (bytes) inside one chunk, relative to the chunk's base pointer.  A
    // lane's LDS destination is fixed (16 bytes at 16 * lane of the instruction's KiB), so the
    // XOR swizzles that keep the fragment reads free of bank conflicts are applied by choosing
    // which 16-byte piece of its row each lane fetches: a row of 64 B (A, a transposed B) keeps
    // piece q at q ^ ((row / 4) % 4) of 4; a row of 128 B (B stored K x N) keeps piece q at
    // q ^ (2 ((row / 2) % 2) + 4 ((row / 8) % 2)) of 8 (row: within the chunk).  Rows that share
    // banks then hold the pieces one fragment read needs in different banks.
    uint32_t voffB[BCH], voffA[MT];
    const int sw64 = (lane >> 4) & 3;                   // row lane/4: (row / 4) % 4
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        if constexpr (BT) {
            // B stored N x K: CB rows (n) of 64 B; instruction i -> rows 16i + lane/4
            const int n = min(n0 + 16 * i + (lane >> 2), p.N - 1);
            voffB[i] = (uint32_t)(n * p.ldb * ES + ((lane & 3) ^ sw64) * 16);
        } else {
            // B stored K x N: 32 rows (k) of 128 B (whole lines); instruction i -> rows 8i + lane/8,
            // 8 columns per piece (columns past N read the last 8 valid ones: never stored)
            const int sw128 = (((lane >> 4) & 1) << 1) | ((i & 1) << 2);   // row 8i + lane/8
            const int col = min(n0 + 8 * ((lane & 7) ^ sw128), p.N - 8);
            voffB[i] = (uint32_t)((8 * i + (lane >> 3)) * p.ldb + col) * 2u;
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        // A rows 16t + lane/4 (clamped) of the 64 B k chunk
        const int m = min(16 * t + (lane >> 2), p.M - 1);
        voffA[t] = (uint32_t)(m * p.lda * ES + ((lane & 3) ^ sw64) * 16);
    }
    auto issue = [&](int c, int slot) {
        const int k0 = c * KCH;
        const uint8_t *bb = BT ? B + k0 * ES : B + (size_t)k0 * p.ldb * ES;
        const uint32_t dst = lring + (uint32_t)(slot * SLOT);
#pragma unroll
        for (int i = 0; i < BCH; ++i) dma16(bb, voffB[i], dst + 1024u * i);
#pragma unroll
        for (int t = 0; t < MT; ++t) dma16(A + k0 * ES, voffA[t], dst + 1024u * (BCH + t));
    };

    // fragment read offsets inside a slot.  A chunk (16 rows x 64 B, row r at 64 r): lane l
    // needs row l%16, k 8*(l/16) .. +7, i.e. piece l/16 (swizzled).  B, transposed layout: rows n
    // at 64 B, column group g (16 columns) at 1024 g, same lane map as A.  B, K x N layout: rows
    // k of 128 B, read with the transposing read: lane a of each 16-lane group addresses row
    // r = a/4 + 8*(l/16) (+ 4h, which leaves the swizzle unchanged) and columns 16g + 4*(a%4)
    // .. +3, i.e. 8 bytes of piece 2g + (a%4)/2 (swizzled).
    const int ra = lane & 15;
    const uint32_t offA = (uint32_t)(ra * 64 + (((lane >> 4) ^ ((ra >> 2) & 3)) * 16));
    const int rb = 8 * (lane >> 4) + ((lane & 15) >> 2);
    const int swb = (((rb >> 1) & 1) << 1) | (((rb >> 3) & 1) << 2);
    uint32_t offB[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        offB[g] = BT ? offA + 1024u * g
                     : (uint32_t)(rb * 128 + (((2 * g + ((lane & 3) >> 1)) ^ swb) * 16) + (lane & 1) * 8);

    AV acc[MT][G];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[t][g] = AV{0, 0, 0, 0};

    const int npro = min(DEPTH, nch);
    for (int c = 0; c < npro; ++c) issue(c0 + c, c);

#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int slot = c % DEPTH;
        // loads of later chunks still allowed in flight
        if (nch - 1 - c >= DEPTH - 1) wait_vm<STEADY>();
        else wait_vm_atmost((nch - 1 - c) * DPC);
        const uint32_t sl = lring + (uint32_t)(slot * SLOT);
        u32x4 bf[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if constexpr (BT) {
                bf[g] = *(const lds_u32x4 *)(uintptr_t)(sl + offB[g]);
            } else {
                const uint32_t a = sl + offB[g];
                s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a);
                s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(a + 4 * 128));
                bf[g][0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
                bf[g][1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
                bf[g][2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
                bf[g][3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
            }
        }
        u32x4 af[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) af[t] = *(const lds_u32x4 *)(uintptr_t)(sl + 1024u * (BCH + t) + offA);
        // load transforms (no-ops when disabled)
#pragma unroll
        for (int g = 0; g < G; ++g) bf[g] = zero_negative<ES>(bf[g], p.xform_b);
#pragma unroll
        for (int t = 0; t < MT; ++t) af[t] = zero_negative<ES>(af[t], p.xform_a);
        // the slot is refilled below: its reads must have returned first
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[t][g] = mma16<TI>(af[t], bf[g], acc[t][g]);
        if (c + DEPTH < nch) issue(c0 + c + DEPTH, slot);
    }

    // add the four waves' partial sums (every wave has waited for all of its loads): all park
    // theirs in LDS, then wave w adds up column group w in wave order (the narrow variant has
    // one group: wave 0 adds it, the others are done)
    __syncthreads();
    AV *part = reinterpret_cast<AV *>(smem);          // [wave][MT][group][64 lanes]
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g) part[((wave * MT + t) * G + g) * 64 + lane] = acc[t][g];
    __syncthreads();
    if (wave >= G) return;
    AV sum[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        sum[t] = part[((0 * MT + t) * G + wave) * 64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum[t] += part[((w * MT + t) * G + wave) * 64 + lane];
    }

    // lane holds rows 16t + 4*(lane/16) + r of column n
    const int n = n0 + 16 * wave + (lane & 15);
    if (S > 1) {
        // split K: this split's sums to the workspace, for the finishing kernel
        if (n >= p.N) return;
        using W = typename std::conditional<INT, int, float>::type;
        W *ws = reinterpret_cast<W *>(p.ws) + ((int64_t)prod * S + split) * p.M * p.N;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * t + 4 * (lane >> 4) + r;
                if (m < p.M) ws[(int64_t)m * p.N + n] = sum[t][r];
            }
        return;
    }

    // epilogue
    using T = typename TO::T;
    if (n >= p.N) return;
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);
    if constexpr (INT) {
        // int32: acc + C (beta 0 or 1) + bias[n], wrapping as two's complement; then ReLU
        const uint32_t bi = p.has_bias ? (uint32_t)static_cast<const int *>(p.bias)[n] : 0u;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * t + 4 * (lane >> 4) + r;
                if (m >= p.M) continue;
                const int64_t idx = (int64_t)m * p.ldc + n;
                uint32_t x = (uint32_t)sum[t][r];
                if (p.has_beta) x += (uint32_t)c_in_i((int)C[idx], p.xform_c);
                x += bi;
                int y = (int)x;
                if (p.relu) y = y > 0 ? y : 0;
                D[idx] = (T)y;
            }
        return;
    }
    const float bv = p.has_bias ? static_cast<const float *>(p.bias)[n] : 0.0f;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * t + 4 * (lane >> 4) + r;
            if (m >= p.M) continue;
            const int64_t idx = (int64_t)m * p.ldc + n;
            float x = p.alpha * sum[t][r];
            if (p.has_beta) x += p.beta * c_in_f(C[idx], p.xform_c);
            x += bv;
            if (p.relu) x = x > 0.0f ? x : 0.0f;
            D[idx] = (T)x;
        }
}

// Split K, second step: D[m][n] = epilogue(sum of the S splits' partial sums, in split order).
// One thread per FCOLS consecutive output columns (FCOLS = 4: 16-byte loads of the partial sums
// when N is a multiple of 4, for large outputs; 1 for small ones, which then get more
// workgroups); the split loop is unrolled so that several loads are in flight; workgroup =
// 256 * FCOLS consecutive columns of one row of a product.
template <class TO, int FCOLS>
__global__ __launch_bounds__(NT) void skinny_finish(GemmParams p) {
    using T = typename TO::T;
    constexpr int SPAN = NT * FCOLS;
    const int tiles = (p.N + SPAN - 1) / SPAN;
    const int per = tiles * p.M;
    const int prod = blockIdx.x / per;
    const int lid = select_batch<2, (int)sizeof(T)>(p, blockIdx.x, per);
    const int m = lid / tiles;
    const int n0 = (lid - m * tiles) * SPAN + (int)threadIdx.x * FCOLS;
    if (n0 >= p.N) return;
    const int S = p.tiles_m;
    const int64_t plane = (int64_t)p.M * p.N;
    const float *ws = p.ws + (int64_t)prod * S * plane + (int64_t)m * p.N + n0;
    float v[FCOLS];
#pragma unroll
    for (int e = 0; e < FCOLS; ++e) v[e] = 0.0f;
    if (FCOLS == 1) {
#pragma unroll 4
        for (int q = 0; q < S; ++q) v[0] += ws[q * plane];
    } else if (p.N % FCOLS == 0) {
        // whole, 16-byte aligned groups (the workspace rows are N floats)
#pragma unroll 4
        for (int q = 0; q < S; ++q) {
            const f32x4 w = *reinterpret_cast<const f32x4 *>(ws + q * plane);
#pragma unroll
            for (int e = 0; e < FCOLS; ++e) v[e] += w[e & 3];
        }
    } else {
#pragma unroll
        for (int e = 0; e < FCOLS; ++e)
            if (n0 + e < p.N)
                for (int q = 0; q < S; ++q) v[e] += ws[q * plane + e];
    }
#pragma unroll
    for (int e = 0; e < FCOLS; ++e) {
        const int n = n0 + e;
        if (n >= p.N) break;
        const int64_t idx = (int64_t)m * p.ldc + n;
        float x = p.alpha * v[e];
        if (p.has_beta) x += p.beta * c_in_f(static_cast<const T *>(p.C)[idx], p.xform_c);
        if (p.has_bias) x += static_cast<const float *>(p.bias)[n];
        if (p.relu) x = x > 0.0f ? x : 0.0f;
        static_cast<T *>(p.D)[idx] = (T)x;
    }
}

// The finishing kernel (also used on its own by the fast kernel's K split, which writes the same
// workspace layout): 4 columns per thread from 2^20 output elements per product, else 1.
template <class TO>
hipError_t launch_finish(const GemmParams &p, hipStream_t s) {
    const bool wide = (int64_t)p.M * p.N >= ((int64_t)1 << 20);
    const int span = NT * (wide ? 4 : 1);
    const unsigned g = (unsigned)((int64_t)((p.N + span - 1) / span) * p.M * p.batch);
    if (wide) hipLaunchKernelGGL((skinny_finish<TO, 4>), dim3(g), dim3(NT), 0, s, p);
    else hipLaunchKernelGGL((skinny_finish<TO, 1>), dim3(g), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO, int MT, bool BT, int CB = NB>
hipError_t launch_skinny(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_skinny<TI, TO, MT, BT, CB>), dim3(grid), dim3(NT), 0, s, p);
    if (p.tiles_m > 1) {
        if constexpr (TI::E == 1) return finish_i8_i32(p, s);   // int32 partial sums
        else return launch_finish<TO>(p, s);
    }
    return hipGetLastError();
}


// narrow = 1: the 16-column variant (B transposed only)
template <class TI, class TO>
const KernelEntry *lookup_skinny(int op_b, int mt, int narrow) {
    constexpr int KC = kch<TI>();
    static const KernelEntry nar[4] = {
        {launch_skinny<TI, TO, 1, true, NB_NARROW>, 16, NB_NARROW, KC, 1, 4, "gemm_skinny_m16_n16"},
        {launch_skinny<TI, TO, 2, true, NB_NARROW>, 32, NB_NARROW, KC, 1, 4, "gemm_skinny_m32_n16"},
        {launch_skinny<TI, TO, 3, true, NB_NARROW>, 48, NB_NARROW, KC, 1, 4, "gemm_skinny_m48_n16"},
        {launch_skinny<TI, TO, 4, true, NB_NARROW>, 64, NB_NARROW, KC, 1, 4, "gemm_skinny_m64_n16"}};
    if (narrow) return (op_b == 1 && mt >= 1 && mt <= 4) ? &nar[mt - 1] : nullptr;
    if (op_b < 0 || op_b > 1 || mt < 1 || mt > 4) return nullptr;
    static const KernelEntry t[4] = {
        {launch_skinny<TI, TO, 1, true>, 16, NB, KC, 1, 4, "gemm_skinny_m16"},
        {launch_skinny<TI, TO, 2, true>, 32, NB, KC, 1, 4, "gemm_skinny_m32"},
        {launch_skinny<TI, TO, 3, true>, 48, NB, KC, 1, 4, "gemm_skinny_m48"},
        {launch_skinny<TI, TO, 4, true>, 64, NB, KC, 1, 4, "gemm_skinny_m64"}};
    if (op_b == 1) return &t[mt - 1];
    if constexpr (TI::E == 1) {
        return nullptr;   // int8 with B not transposed: not this kernel
    } else {
        static const KernelEntry n[4] = {
            {launch_skinny<TI, TO, 1, false>, 16, NB, KC, 1, 4, "gemm_skinny_m16"},
            {launch_skinny<TI, TO, 2, false>, 32, NB, KC, 1, 4, "gemm_skinny_m32"},
            {launch_skinny<TI, TO, 3, false>, 48, NB, KC, 1, 4, "gemm_skinny_m48"},
            {launch_skinny<TI, TO, 4, false>, 64, NB, KC, 1, 4, "gemm_skinny_m64"}};
        return &n[mt - 1];
    }
}

}  // namespace

#if defined(TGE_PAIR_F16_F16)
const KernelEntry *skinny_f16_f16(int b, int mt, int nw) { return lookup_skinny<TF16, OF16>(b, mt, nw); }
hipError_t finish_f16_f16(const GemmParams &p, hipStream_t s) { return launch_finish<OF16>(p, s); }
#elif defined(TGE_PAIR_F16_F32)
const KernelEntry *skinny_f16_f32(int b, int mt, int nw) { return lookup_skinny<TF16, OF32>(b, mt, nw); }
hipError_t finish_f16_f32(const GemmParams &p, hipStream_t s) { return launch_finish<OF32>(p, s); }
#elif defined(TGE_PAIR_BF16_BF16)
const KernelEntry *skinny_bf16_bf16(int b, int mt, int nw) { return lookup_skinny<TBF16, OBF16>(b, mt, nw); }
hipError_t finish_bf16_bf16(const GemmParams &p, hipStream_t s) { return launch_finish<OBF16>(p, s); }
#elif defined(TGE_PAIR_BF16_F32)
const KernelEntry *skinny_bf16_f32(int b, int mt, int nw) { return lookup_skinny<TBF16, OF32>(b, mt, nw); }
hipError_t finish_bf16_f32(const GemmParams &p, hipStream_t s) { return launch_finish<OF32>(p, s); }
#elif defined(TGE_PAIR_I8_I32)
// (B transposed only; the finishing step is finish_i8_i32)
const KernelEntry *skinny_i8_i32(int b, int mt, int nw) { return lookup_skinny<TI8, OI32>(b, mt, nw); }
#else
#error "define one TGE_PAIR_* macro"
#endif

}  // namespace tge
