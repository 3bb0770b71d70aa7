// Memory-bound path for short-and-wide GEMMs on gfx950 (M <= 64, e.g. a fully-connected layer
// applied to a small batch): every byte of B is read once from HBM, so the kernel is built to
// keep enough loads in flight to stream B at full bandwidth rather than to maximise reuse.
// "CUTLASS: Fast Linear Algebra in CUDA C++" ("CUTLASS GEMM Strategies") specialises its tiling
// for tall and narrow shapes the same way; the shape here is the transposed case.
//
//  * one workgroup per 16 output columns (N / 16 workgroups, 256 for N = 4096), K split evenly
//    over its 4 waves; neighbouring column blocks are placed on the same XCD so that the 128-byte
//    lines they share are fetched into one L2;
//  * each wave streams its own K range through a private ring of 16 LDS slots with direct-to-LDS
//    loads (no barriers inside the loop: a wave only waits for its own loads): per 32-wide k
//    chunk, 1 KiB of B (32 k x 16 columns) and 1 KiB of A per 16 rows;
//  * fragments: A (K-contiguous) and a transposed B with ds_read_b128, a non-transposed B with
//    the transposing read ds_read_b64_tr_b16; MFMA 16x16x32 with fp32 accumulation;
//  * the four waves' partial sums are added through LDS and the first wave applies the fused
//    epilogue (alpha, beta*C, bias[j], ReLU, convert) and stores.
//
// Preconditions (checked by the host): 16-bit inputs, op(A) = A (not transposed), M <= 64,
// K % 32 == 0, A/B pointers and leading dimensions 16-byte aligned, N % 8 == 0 when B is not
// transposed.

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
constexpr int NB = 16;         // output columns per workgroup
constexpr int KCH = 32;        // k per chunk
constexpr int RING = 16;       // LDS slots per wave

template <class TI>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mma16<TF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma16<TBF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}

// direct-to-LDS 16-byte load per lane (LDS destination lds + 16 * lane), see gemm_fast.hip
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
                 :: "s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
}

constexpr int min_c(int a, int b) { return a < b ? a : b; }

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

// MT: 16-row tiles of A (M <= 16 * MT); BT: B is stored transposed (N x K)
template <class TI, class TO, int MT, bool BT>
__global__ __launch_bounds__(NT, 1) void gemm_skinny(GemmParams p) {
    constexpr int SLOT = (1 + MT) * 1024;   // B chunk, then MT A chunks
    constexpr int DPC = 1 + MT;              // load instructions per chunk
    // ring depth: at most RING, within 40 KiB of LDS per wave, and few enough loads in flight
    // for the 6-bit vmcnt to count
    constexpr int DEPTH = min_c(min_c(RING, 40 / DPC), 63 / DPC);
    constexpr int STEADY = (DEPTH - 1) * DPC;  // loads allowed in flight when waiting for one chunk
    static_assert(4 * DEPTH * SLOT <= 160 * 1024 && 3 * MT * 1024 <= 4 * DEPTH * SLOT, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * DEPTH * SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // consecutive column blocks share 128-byte lines of a non-transposed B: keep them on one
    // XCD (one L2) with the same re-mapping the tiled kernels use
    const int n0 = select_batch<2, (int)sizeof(typename TO::T)>(p, xcd_remap(blockIdx.x, gridDim.x), p.tiles_n) * NB;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    // K range of this wave, in chunks
    const int nch_all = p.K / KCH;
    const int per = (nch_all + 3) / 4;
    const int c0 = min(wave * per, nch_all), c1 = min(c0 + per, nch_all);
    const int nch = c1 - c0;

    uint8_t *ring = smem + wave * DEPTH * SLOT;
    const uint32_t lring = lds_addr(ring);

    // per-lane load offsets (bytes) inside one chunk, relative to the chunk's base pointer
    uint32_t voffB, voffA[MT];
    if constexpr (BT) {
        // B stored N x K: 16 rows (n) of 64 B; lane -> row lane/4, 16 B piece lane%4
        const int n = min(n0 + (lane >> 2), p.N - 1);
        voffB = (uint32_t)(n * p.ldb + (lane & 3) * 8) * 2u;
    } else {
        // B stored K x N: 32 rows (k) of 32 B; lane -> row lane/2, columns 8*(lane%2) .. +7
        const int col = min(n0 + 8 * (lane & 1), p.N - 8);
        voffB = (uint32_t)((lane >> 1) * p.ldb + col) * 2u;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        // A rows 16t + lane/4 (clamped), 16 B piece lane%4 of the 64 B k chunk
        const int m = min(16 * t + (lane >> 2), p.M - 1);
        voffA[t] = (uint32_t)(m * p.lda + (lane & 3) * 8) * 2u;
    }
    auto issue = [&](int c, int slot) {
        const int k0 = (c0 + c) * KCH;
        const uint16_t *bb = BT ? B + k0 : B + (size_t)k0 * p.ldb;
        const uint32_t dst = lring + (uint32_t)(slot * SLOT);
        dma16(bb, voffB, dst);
#pragma unroll
        for (int t = 0; t < MT; ++t) dma16(A + k0, voffA[t], dst + 1024u * (1 + t));
    };

    // fragment read offsets inside a slot
    // A chunk (16 rows x 64 B, row r at 64 r): lane l needs row l%16, k 8*(l/16) .. +7
    const uint32_t offA = (uint32_t)((lane & 15) * 64 + (lane >> 4) * 16);
    // B: transposed layout = same shape as A (rows n); otherwise rows k of 32 B read with the
    // transposing read: lane a of each 16-lane group addresses row a/4 (+ 8*(l/16) + 4h) and
    // columns 4*(a%4) .. +3
    const uint32_t offB = BT ? offA
                             : (uint32_t)((8 * (lane >> 4) + ((lane & 15) >> 2)) * 32 + (lane & 3) * 8);

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npro = min(DEPTH, nch);
    for (int c = 0; c < npro; ++c) issue(c, c);

#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int slot = c % DEPTH;
        // loads of later chunks still allowed in flight
        if (nch - 1 - c >= DEPTH - 1) wait_vm<STEADY>();
        else wait_vm_atmost((nch - 1 - c) * DPC);
        const uint8_t *sl = ring + slot * SLOT;
        u32x4 bf;
        if constexpr (BT) {
            bf = *(const lds_u32x4 *)(uintptr_t)(lds_addr(sl) + offB);
        } else {
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(lds_addr(sl) + offB));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(lds_addr(sl) + offB + 4 * 32));
            bf[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
            bf[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
            bf[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
            bf[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
        }
        u32x4 af[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t)
            af[t] = *(const lds_u32x4 *)(uintptr_t)(lds_addr(sl) + 1024u * (1 + t) + offA);
        // load transforms (no-ops when disabled)
        bf = zero_negative<2>(bf, p.xform_b);
#pragma unroll
        for (int t = 0; t < MT; ++t) af[t] = zero_negative<2>(af[t], p.xform_a);
        // the slot is refilled below: its reads must have returned first
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = mma16<TI>(af[t], bf, acc[t]);
        if (c + DEPTH < nch) issue(c + DEPTH, slot);
    }

    // add the four waves' partial sums: waves 1..3 park theirs in LDS
    __syncthreads();
    float *part = reinterpret_cast<float *>(smem);   // [wave 1..3][MT][64 lanes][4]
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[(((wave - 1) * MT + t) * 64 + lane) * 4 + r] = acc[t][r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] += part[((w * MT + t) * 64 + lane) * 4 + r];

    // epilogue: lane holds D[16t + 4*(lane/16) + r][n0 + lane%16]
    using T = typename TO::T;
    const int n = n0 + (lane & 15);
    if (n >= p.N) return;
    const float bv = p.has_bias ? static_cast<const float *>(p.bias)[n] : 0.0f;
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * t + 4 * (lane >> 4) + r;
            if (m >= p.M) continue;
            const int64_t idx = (int64_t)m * p.ldc + n;
            float x = p.alpha * acc[t][r];
            if (p.has_beta) x += p.beta * c_in_f(C[idx], p.xform_c);
            x += bv;
            if (p.relu) x = x > 0.0f ? x : 0.0f;
            D[idx] = (T)x;
        }
}

template <class TI, class TO, int MT, bool BT>
hipError_t launch_skinny(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_skinny<TI, TO, MT, BT>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO>
const KernelEntry *lookup_skinny(int op_b, int mt) {
    static const KernelEntry e[2][4] = {
        {{launch_skinny<TI, TO, 1, false>, 16, NB, KCH, 1, 4, "gemm_skinny_m16"},
         {launch_skinny<TI, TO, 2, false>, 32, NB, KCH, 1, 4, "gemm_skinny_m32"},
         {launch_skinny<TI, TO, 3, false>, 48, NB, KCH, 1, 4, "gemm_skinny_m48"},
         {launch_skinny<TI, TO, 4, false>, 64, NB, KCH, 1, 4, "gemm_skinny_m64"}},
        {{launch_skinny<TI, TO, 1, true>, 16, NB, KCH, 1, 4, "gemm_skinny_m16"},
         {launch_skinny<TI, TO, 2, true>, 32, NB, KCH, 1, 4, "gemm_skinny_m32"},
         {launch_skinny<TI, TO, 3, true>, 48, NB, KCH, 1, 4, "gemm_skinny_m48"},
         {launch_skinny<TI, TO, 4, true>, 64, NB, KCH, 1, 4, "gemm_skinny_m64"}},
    };
    if (op_b < 0 || op_b > 1 || mt < 1 || mt > 4) return nullptr;
    return &e[op_b][mt - 1];
}

}  // namespace

#if defined(TGE_PAIR_F16_F16)
const KernelEntry *skinny_f16_f16(int b, int mt) { return lookup_skinny<TF16, OF16>(b, mt); }
#elif defined(TGE_PAIR_F16_F32)
const KernelEntry *skinny_f16_f32(int b, int mt) { return lookup_skinny<TF16, OF32>(b, mt); }
#elif defined(TGE_PAIR_BF16_BF16)
const KernelEntry *skinny_bf16_bf16(int b, int mt) { return lookup_skinny<TBF16, OBF16>(b, mt); }
#elif defined(TGE_PAIR_BF16_F32)
const KernelEntry *skinny_bf16_f32(int b, int mt) { return lookup_skinny<TBF16, OF32>(b, mt); }
#else
#error "define one 16-bit TGE_PAIR_* macro"
#endif

}  // namespace tge
