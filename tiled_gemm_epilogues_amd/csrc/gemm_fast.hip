// Fast path for large fp16/bf16/int8 GEMMs on gfx950: 256x256 output tile per workgroup, 4 waves
// of 128x128 (8x8 MFMA 16x16 tiles, or 4x4 32x32 tiles; 256 accumulators per lane in AGPRs), K
// walked in slabs of 128 bytes (64 fp16/bf16, 128 int8).  A 128x128 instance (4 waves of 64x64,
// two workgroups per CU; direct loads, 16x16 shape) serves mid-size products.
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
//    choosing which 16-byte chunk each lane fetches.  Operands the direct loads cannot take
//    (unaligned pointers, leading dimensions or strides; M/N extents off the 16-byte grid) are
//    copied into aligned, zero-padded rows first (gemm_repack.hip), or, when no copy workspace
//    exists, read by a register-staged variant that moves the same chunks through registers to
//    the same places.
//  * layouts are handled at load time without transposing through registers ("Flexible GEMM"
//    section 5.1 adapts its loaders to the N/T layout the same way): an operand whose contiguous
//    dimension is K is kept [mn][k] in LDS and read with ds_read_b128; an operand whose
//    contiguous dimension is M or N is kept [k][mn] and read with the gfx950 transposing LDS
//    read ds_read_b64_tr_b16, which hands each lane four consecutive-k values of one column.
//  * swizzles (bank-conflict avoidance, the role padding plays in "Flexible GEMM" section 5.1):
//    [mn][k] rows of 128 B hold logical 16-byte chunk c at c ^ ((r ^ r>>3) & 7); [k][mn] rows of
//    512 B hold chunk c at c ^ h(k & 3) with h = {0, 4, 10, 14} (16x16 shape: also ^ 2 in rows
//    16-31 of each 32).  With the k-group order of kgrp() they give every group of lanes the LDS
//    serves together distinct banks (the LDS bank-conflict counter reads ~0 in the loop).
//  * pipeline per slab s (buffers X = s % 2, Y = the other): the fragments of k-slice j+1 are
//    read while the MFMAs of k-slice j run; after the last read of X the wave waits for its own
//    loads of slab s+1 and joins the barrier; then it issues the loads of slab s+2 into X and the
//    first fragment reads of Y while the last k-slice's MFMAs run.  The loop body holds two slabs
//    so that every stage index is a compile-time constant; the trips between the first and the
//    last ones carry no branches.
//  * M/N edges: source rows past the edge are clamped to the last valid row (their products
//    only reach output rows/columns that the masked epilogue drops); the K tail (K % slab) runs
//    one guarded register-staged slab with zero fill.
//  * MFMA shape: 16x16x32 (16x16x64 int8) for NN, NT and TT; 32x32 for TN read in place, for
//    the load transforms and for the register-staged variant, whose extra live registers the
//    16x16 schedule cannot hold without shuffling accumulators (the host copies a TN layout's
//    A transposed, into K-contiguous rows, when that pays, and runs the NN kernel on it).
//  * epilogue (the epilogue building block of "Flexible GEMM" section 4, fused as in the bias and
//    ReLU functor of "CUTLASS", "Fusing Element-wise Operations"): alpha, beta*C, bias[j], ReLU
//    and the conversion run on the accumulators; the result goes through a per-wave LDS staging
//    buffer so that D is written in whole 128-byte lines.
//
// Preconditions (checked by the host): 16- or 8-bit inputs and K of at least one slab; for the
// direct loads also A/B base pointers, leading dimensions and batch strides 16-byte aligned and
// M (if A is stored transposed) and N (if B is not transposed) multiples of 16 bytes' worth of
// elements, or stored rows zero-padded to whole chunks (the copies); for the register-staged
// variant an M/N-contiguous extent of at least one chunk.

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

constexpr int SLAB_BYTES = 128;                      // K bytes per slab: 64 fp16/bf16 or 128 int8
constexpr int NT = 256;                              // 4 waves

// Tile geometry: TL x TL output tile (256, or 128 for mid-size products), 4 waves of TL/2 x TL/2.
// One operand slab is TL * 128 bytes in either layout (32 KiB at TL = 256).  LDS map: [A stage
// 0 | A stage 1 | B stage 0 | B stage 1], so that every fragment read is (base register) +
// (stage and k-slice offset as the instruction's 16-bit immediate).
template <int TL>
struct Geo {
    static constexpr int KC = TL * SLAB_BYTES;       // bytes of one operand slab
    static constexpr int OPND = 2 * KC;              // byte offset of operand B's stages
    static constexpr int NL = KC / 1024 / 4;         // direct loads per wave, operand and slab
    static constexpr int WT = TL / 2;                // wave tile
};

// [mn][k] layout (K-contiguous operands): TL rows of 128 B, 16-byte chunk c of row r at
// c ^ swz_kc(r); identical in bytes for 8- and 16-bit elements.
__device__ __forceinline__ int swz_kc(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int off_kc(int r, int c) { return r * 128 + ((c ^ swz_kc(r)) << 4); }

// [k][mn] layout (M/N-contiguous operands): 64 rows of TL 16-bit elements (512 B at TL = 256, 256 B
// at TL = 128) or 128 rows of 256 B (8-bit, TL = 256 only).  A transposing read (8 bytes per lane) is served 32 lanes at a time; the 16 lanes of
// one k group touch 4 (16-bit) or 8 (8-bit) consecutive rows at 2 adjacent 16-byte chunks, and
// the swizzle gives those accesses distinct banks.  With the 16x16 MFMA shape the two k groups
// served together (lanes 0-15 and 16-31) lie 16 (16-bit) or 32 (8-bit) rows apart: one more
// row bit of the swizzle moves the second group to the other half of the banks (the 32x32
// shape keeps the k groups of a pass in one row block, and adds whole k-slices to a base
// address, which must not change the swizzle).
template <int E, int MF, int TL = 256>
__device__ __forceinline__ int swz_mc(int k) {
    if constexpr (E == 1 && TL == 128) {
        // 8-bit rows of 128 B (8 chunks; a row spans half the banks, rows k and k+2 the same
        // half): the 16 lanes of a k group read 8 consecutive rows at one chunk, so rows of one
        // half (k, k+2, k+4, k+6) take 4 different chunks; the k group served with it, 32 rows
        // on, takes the other 4.  Invariant under adding 8 or 64 to a fragment's base row (the
        // second transposing read, the k-slice offset).
        static_assert(MF == 16, "16x16 shape");
        return ((k >> 1) & 3) ^ (((k >> 5) & 1) << 2);
    } else if constexpr (E == 2) {
        const int q = k & 3;
        return (4 * q + 2 * (q >> 1)) ^ (MF == 16 ? ((k >> 4) & 1) << 1 : 0);
    } else {
        const int q = k & 7;
        return (2 * q + (q >> 2)) ^ (MF == 16 ? (k >> 5) & 1 : 0);
    }
}
template <int E, int MF, int TL>
__device__ __forceinline__ int off_mc(int k, int c) { return k * TL * E + ((c ^ swz_mc<E, MF, TL>(k)) << 4); }

// k group of the 16 lanes l/16 = g of a 16x16 MFMA fragment.  A 16-byte read (ds_read_b128)
// is served as lanes l and l+32 together, so the groups g and g+2 must read chunks of opposite
// parity (a bank-disjoint pair under the [mn][k] swizzle): group g takes the k range
// 8*grp(g) .. +7 of the k-slice (16 for 8-bit), the same for both operands, which only
// relabels the products' summation order.  The 32x32 shape keeps the natural order.
template <int MF>
__device__ __forceinline__ int kgrp(int g) { return MF == 16 ? ((g & 1) << 1) | (g >> 1) : g; }

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

// RS: register-staged variant for operands the direct loads cannot take (a pointer or leading
// dimension off 16-byte alignment, or an M/N-contiguous extent that is not a whole number of
// chunks): the same chunk of the same slab goes global -> registers (unaligned 16-byte loads are
// legal) -> LDS, so the LDS image is identical.  An M/N-contiguous chunk that starts inside the
// row and crosses its end reads on into the next stored row (at most 15 bytes, inside the
// matrix as long as a next row exists: the last row of K always goes through the guarded tail);
// a chunk that starts past the end reads the row's last element onwards.  Those extra elements
// only reach output rows or columns past the edge, which are never stored.  Needs an extent of
// at least one chunk.
template <int E, bool KC, int MF, bool RS = false, int TL = 256>
struct Loader {
    static constexpr int VE = 16 / E;    // elements per 16-byte chunk
    static constexpr int NL = Geo<TL>::NL;
    uint32_t voff[NL];

    // row0: first M (or N) index of the tile; ext: M (or N); ld: leading dimension.
    __device__ __forceinline__ void init(int wave, int lane, int row0, int ext, int ld) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int blk = wave * NL + i;                         // 1 KiB block of the slab
            if constexpr (KC) {
                const int r = blk * 8 + (lane >> 3);               // tile row (8 rows of 128 B)
                const int c = (lane & 7) ^ swz_kc(r);              // logical chunk this lane fetches
                const int gr = min(row0 + r, ext - 1);
                voff[i] = (uint32_t)(gr * ld + c * VE) * (uint32_t)E;
            } else {
                constexpr int CPR = TL * E / 16;                   // chunks per [k] row
                const int k = blk * (64 / CPR) + lane / CPR;       // slab row (k)
                const int c = (lane % CPR) ^ swz_mc<E, MF, TL>(k);
                if constexpr (RS) {
                    const int col = min(row0 + c * VE, ext - 1);   // starts inside the row
                    voff[i] = (uint32_t)(k * ld + col) * (uint32_t)E;
                } else {
                    // the last chunk starts at the last multiple of VE below ext: whole chunks
                    // when ext % VE == 0, else it runs into the zero padding of a repacked row
                    const int col = min(row0 + c * VE, (ext - 1) / VE * VE);
                    voff[i] = (uint32_t)(k * ld + col) * (uint32_t)E;
                }
            }
        }
    }
    // base of the slab whose K starts at element k0
    __device__ __forceinline__ static const uint8_t *slab_base(const uint8_t *base, int ld, int k0) {
        return KC ? base + (size_t)k0 * E : base + (size_t)k0 * ld * E;
    }
    // instruction i of this wave: LDS block (wave*NL + i) of the operand slab at `dst`
    __device__ __forceinline__ void issue(const uint8_t *sb, uint32_t dst, int wave, int i) const {
        dma16(sb, voff[i], dst + (uint32_t)(wave * NL + i) * 1024u);
    }
    // RS: chunk i of this lane from the slab at sb, into registers (raw; nothing may touch the
    // registers before put, so the load has a slab's time to land)
    __device__ __forceinline__ u32x4 fetch(const uint8_t *sb, int i) const { return ldg16(sb + voff[i]); }
    // RS: chunk i fetched into v, with the load transform applied (xf), to its LDS place in the
    // slab (the one a direct load would fill)
    __device__ __forceinline__ static void put(uint8_t *slab, int wave, int i, int lane, u32x4 v, int xf) {
        v = zero_negative<E>(v, xf);
        *reinterpret_cast<u32x4 *>(slab + (wave * NL + i) * 1024 + 16 * lane) = v;
    }
};

// Guarded staging of a partial slab (k0 .. K-1, zero beyond) into the same LDS layout, with the
// load transform xf applied (register-staged kernels; the others transform their fragments).
// fetch() issues all of this thread's loads (8 chunks of 16 bytes; both operands' fetches go
// out before the barrier that frees the stage), put() writes them to LDS.
template <int E, bool KC, int MF, int TL = 256>
struct TailStage {
    static constexpr int VE = 16 / E;
    static constexpr int CPR = TL * E / 16;   // chunks per [k] row of an M/N-contiguous slab
    static constexpr int NC = TL * 8 / NT;    // chunks per thread
    u32x4 v[NC];

    __device__ __forceinline__ void fetch(const uint8_t *base, int ld, int row0, int ext, int k0, int K, int tid) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int q = tid + NT * i;
            const uint8_t *p;
            int nval;          // leading elements of the chunk inside the operand (0 .. VE)
            if constexpr (KC) {
                const int r = q >> 3, c = q & 7;
                p = base + ((size_t)min(row0 + r, ext - 1) * ld + k0 + c * VE) * E;
                nval = K - (k0 + c * VE);
            } else {
                const int k = q / CPR, c = q % CPR;
                const int col = row0 + c * VE;
                p = base + ((size_t)(k0 + k) * ld + col) * E;
                // elements past the M/N edge are zero (their products are never stored)
                nval = k0 + k < K ? ext - col : 0;
            }
            v[i] = u32x4{0, 0, 0, 0};
            if (nval >= VE) v[i] = ldg16(p);
            else if (nval > 0) v[i] = ldg16_partial<E>(p, nval);
        }
    }
    __device__ __forceinline__ void put(uint8_t *dst, int tid, int xf) const {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int q = tid + NT * i;
            const uint32_t off = KC ? off_kc(q >> 3, q & 7) : off_mc<E, MF, TL>(q / CPR, q % CPR);
            const u32x4 w = zero_negative<E>(v[i], xf);
            __builtin_memcpy(dst + off, &w, 16);
        }
    }
};

// ---- fragment reads ---------------------------------------------------------------------------
// MF = 32 (MFMA 32x32, k-slice of 32 bytes of K): fragment (sub-tile t, k-slice j) gives lane l
// 16 bytes of consecutive k (k = j*KS + (l/32)*KS/2 + ..., KS = 32 bytes) of tile row (or
// column) 32t + l%32.  MF = 16 (MFMA 16x16, k-slice of 64 bytes): lane l gets 16 bytes of
// consecutive k (k = j*KS + (l/16)*KS/4 + ..., KS = 64 bytes) of row 16t + l%16.  A K-contiguous
// operand needs one ds_read_b128 per fragment, an M/N-contiguous one two transposing reads,
// issued together and assembled as one vector (assembling the halves in separate steps makes
// the register allocator shuffle accumulators).

template <int MF, int TL = 256>
struct Shape {
    static constexpr int NF = TL / 2 / MF;          // fragments per operand and k-slice
    static constexpr int NS = MF == 32 ? 4 : 2;     // k-slices per slab
    static constexpr int NMS = NF * NF;             // MFMAs per k-slice
    static constexpr int KSB = SLAB_BYTES / NS;     // bytes of K per k-slice
};

template <int E, bool KC, int MF, int TL = 256>
struct Frag {
    using S = Shape<MF, TL>;
    static constexpr int KCB = Geo<TL>::KC;         // bytes of one operand stage
    static constexpr int ROWB = TL * E;             // bytes of an [k][mn] row
    static constexpr int NF = S::NF;
    // byte address (LDS) of this lane's fragment in stage 0: per sub-tile and k-slice for a
    // K-contiguous operand (the XOR swizzle is not additive), per sub-tile otherwise
    uint32_t addr[NF][KC ? S::NS : 1];

    __device__ __forceinline__ void init(int lane, int wrow, uint32_t opbase) {
        constexpr int LR = MF;                       // lanes per row group
        const int lr = lane & (LR - 1), lg = lane / LR;
#pragma unroll
        for (int t = 0; t < NF; ++t) {
            if constexpr (KC) {
                const int r = wrow + MF * t + lr;
#pragma unroll
                for (int j = 0; j < S::NS; ++j)
                    addr[t][j] = opbase + (uint32_t)off_kc(r, (S::KSB / 16) * j + kgrp<MF>(lg));
            } else if constexpr (E == 2) {
                // ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i % 4
                // of the 8-byte chunks addressed by lanes i/4 + 4e, e = 0..3.  Lane a of the
                // group therefore addresses k row a/4 and columns 4*(a%4) .. +3; lane group g
                // (of 64/MF... groups of 16) covers k 8 kgrp(g).. (MF 16) or 8(l/32).. (MF 32).
                const int q = (lane & 15) >> 2;
                const int k = 8 * kgrp<MF>(lg) + q;
                const int col = wrow + MF * t + (MF == 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
                addr[t][0] = opbase + (uint32_t)(k * ROWB + (((col >> 3) ^ swz_mc<2, MF, TL>(k)) << 4) + (col & 7) * 2);
            } else {
                // ds_read_b64_tr_b8: in each group of 16 lanes, lane i receives byte i % 8 of
                // the 8-byte chunks addressed by lanes i/8 + 2e, e = 0..7.  Lane a of the group
                // therefore addresses k row a/2 and columns 8*(a%2) .. +7.
                const int a = lane & 15;
                const int k = 16 * kgrp<MF>(lg) + (a >> 1);
                const int col = wrow + MF * t + (MF == 32 ? 16 * ((lane >> 4) & 1) : 0) + 8 * (a & 1);
                addr[t][0] = opbase + (uint32_t)(k * ROWB + (((col >> 4) ^ swz_mc<1, MF, TL>(k)) << 4) + (col & 15));
            }
        }
    }
    // fragment (t, j) of `stage` into dst
    __device__ __forceinline__ void read(int stage, int t, int j, u32x4 &dst) const {
        if constexpr (KC) {
            dst = *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)(addr[t][j] + stage * KCB);
        } else if constexpr (E == 2) {
            // k rows j*KS/2 + (0..3) and + (4..7) past the lane's base: the swizzle depends on
            // k & 3 and (16x16 shape) k bit 4, which these offsets leave unchanged
            const uint32_t a = addr[t][0] + stage * KCB + ((S::KSB / 2) * j) * ROWB;
            s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a);
            s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(a + 4 * ROWB));
            dst = __builtin_bit_cast(u32x4, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            // k rows j*KS + (0..7) and + (8..15) past the lane's base: the swizzle depends on
            // k & 7 and (16x16 shape) k bit 5, which these offsets leave unchanged
            const uint32_t a = addr[t][0] + stage * KCB + (S::KSB * j) * ROWB;
            i32x2 v0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(uintptr_t)a);
            i32x2 v1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(uintptr_t)(a + 8 * ROWB));
            dst = __builtin_bit_cast(u32x4, __builtin_shufflevector(v0, v1, 0, 1, 2, 3));
        }
    }
};

// ---- epilogue through LDS -------------------------------------------------------------------
// One wave's 128x128 sub-tile, in four blocks of 32 rows: values are computed in the
// accumulator layout (alpha, beta*C, bias[j], ReLU, convert), written row-major into the wave's
// private staging buffer (16-byte chunk c of staged row r at c ^ (r % chunks-per-row)) and read
// back as 16-byte row pieces, so every store instruction writes whole 128-byte lines of D
// instead of 16-byte pieces of 32 rows.
//
// In both MFMA shapes a lane holds, per block, 16 groups of 4 consecutive columns of one row:
//   MF 32: group q = 4j + g of block b is acc[b][j][4g..4g+3], row l%32, columns 32j + 8g + 4(l/32)
//   MF 16: group q = 8i + j of block b is acc[2b+i][j][0..3], row 16i + l%16, columns 16j + 4(l/16)
//
// Vector-memory operations complete in issue order, so a load issued after a store can only be
// awaited together with that store.  Every load is therefore issued before the stores it would
// otherwise wait behind: the bias once before the first block, the C values of block i+1 before
// the stores of block i.
template <class O, int WT>
__device__ __forceinline__ constexpr int stg_bytes() { return 32 * WT * (int)sizeof(typename O::T); }

// WT: the wave tile (128, or 64 for the 128 x 128 workgroup tile, 16x16 shape only)
template <int MF, int WT>
struct EpiMap {
    static_assert(MF == 16 || WT == 128, "the 32x32 shape runs 128-wide wave tiles");
    static constexpr int NBG = MF == 32 ? 16 : WT / 16;   // distinct column groups per lane
    static constexpr int QB = MF == 32 ? 16 : 2 * NBG;    // groups of 4 values per 32-row block
    __device__ static int row(int q, int lane) { return MF == 32 ? (lane & 31) : 16 * (q / NBG) + (lane & 15); }
    __device__ static int col(int q, int lane) {
        return MF == 32 ? 32 * (q >> 2) + 8 * (q & 3) + 4 * (lane >> 5) : 16 * (q % NBG) + 4 * (lane >> 4);
    }
    __device__ static int bgroup(int q) { return MF == 32 ? q : (q % NBG); }
};

template <class O, class Acc, int MF, bool BETA, bool FULL, class AccV, int NF>
__device__ __forceinline__ void store_tile_staged(const GemmParams &p, int mbase, int nbase, int lane,
                                                  AccV (&acc)[NF][NF], uint8_t *stg) {
    using T = typename O::T;
    constexpr int WT = NF * MF;            // wave tile
    using Map = EpiMap<MF, WT>;
    constexpr int QB = Map::QB;
    constexpr int NB = WT / 32;            // 32-row blocks
    constexpr bool INT = std::is_same<Acc, int>::value;
    using Bt = typename std::conditional<INT, int, float>::type;
    constexpr int ES = sizeof(T);
    constexpr int RB = WT * ES;            // staged row bytes
    constexpr int CPR = RB / 16;           // 16-byte chunks per row
    constexpr int VE = 16 / ES;            // elements per chunk
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
    const int M = p.M, N = p.N;
    const Bt *bias = static_cast<const Bt *>(p.bias);
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);
    // D is written once and not read again here: when more rounds of tiles follow (more
    // workgroups than CUs), streaming stores keep the L2 and the infinity cache for the A and B
    // panels those rounds read (measured with the 16x16 shape: 3-8 % faster at 8192^3); in a
    // single round, and with the 32x32 shape, the plain stores measured faster
    const bool stream_d = MF == 16 && (int64_t)p.tiles_m * p.tiles_n * p.batch > (WT == 128 ? 256 : 512);
    typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(1)));
    // accumulator value e of group q in block b
    auto accv = [&](int b, int q, int e) -> Acc {
        if constexpr (MF == 32) return acc[b][q >> 2][4 * (q & 3) + e];
        else return acc[2 * b + (q / Map::NBG)][q % Map::NBG][e];
    };

    // bias of this lane's columns, shared by the row blocks
    Bt bv[Map::NBG][4];
#pragma unroll
    for (int q = 0; q < Map::NBG; ++q) {
        const int n = nbase + Map::col(q, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[q][e] = 0;
        if (p.has_bias) {
            if constexpr (FULL) {
                __builtin_memcpy(bv[q], bias + n, sizeof(bv[q]));
            } else {
                // columns past N read the last valid one (those outputs are never stored)
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[q][e] = bias[min(n + e, N - 1)];
            }
        }
    }
    // C values of row block b for this lane
    T cv[QB][4];
    auto load_c = [&](int b) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const int m = mbase + 32 * b + Map::row(q, lane);
            const int64_t row = (int64_t)(FULL ? m : min(m, M - 1)) * p.ldc;
            const int n = nbase + Map::col(q, lane);
            if constexpr (FULL) {
                __builtin_memcpy(cv[q], C + row + n, sizeof(cv[q]));
            } else {
                // unconditional loads: columns past N read the row's last valid element (those
                // outputs are never stored).  The former per-element conditional 16-bit loads
                // came out wrong for element 0 in one build of the 32x32-shape kernel.
#pragma unroll
                for (int e = 0; e < 4; ++e) cv[q][e] = C[row + min(n + e, N - 1)];
            }
        }
    };
    if constexpr (BETA) load_c(0);

#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const Bt *bq = bv[Map::bgroup(q)];
            T out[4];
            if constexpr (INT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int t = accv(b, q, e) + bq[e];
                    if constexpr (BETA) t += c_in_i((int)cv[q][e], p.xform_c);
                    if (p.relu) t = max(t, 0);
                    out[e] = (T)t;
                }
            } else {
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t[e] = __builtin_fmaf(p.alpha, accv(b, q, e), bq[e]);
                    if constexpr (BETA) t[e] = __builtin_fmaf(p.beta, c_in_f(cv[q][e], p.xform_c), t[e]);
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
            const int rl = Map::row(q, lane);
            const int byte = Map::col(q, lane) * ES;
            const int c = byte >> 4;
            __builtin_memcpy(stg + rl * RB + ((c ^ (rl % CPR)) << 4) + (byte & 15), out, 4 * ES);
        }
        if constexpr (BETA) {
            if (b < NB - 1) load_c(b + 1);
        }
        // read back (the wave's LDS operations execute in order): 32 rows x CPR chunks, 16 bytes
        // per lane per round
#pragma unroll
        for (int q = 0; q < 32 * CPR / 64; ++q) {
            const int idx = q * 64 + lane;
            const int rr = idx / CPR, c = idx % CPR;
            u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rr * RB + ((c ^ (rr % CPR)) << 4));
            const int mg = mbase + 32 * b + rr;
            const int ng = nbase + c * VE;
            T *dst = D + (int64_t)mg * p.ldc + ng;
            if constexpr (FULL) {
                if (stream_d) __builtin_nontemporal_store((u32x4u)v, reinterpret_cast<u32x4u *>(dst));
                else __builtin_memcpy(dst, &v, 16);
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

template <class O, class Acc, int MF, class AccV, int NF>
__device__ __forceinline__ void epilogue(const GemmParams &p, int mbase, int nbase, int lane,
                                         AccV (&acc)[NF][NF], uint8_t *stg) {
    // interior wave tiles (the common case) take a path with no edge checks
    constexpr int WT = NF * MF;
    const bool full = mbase + WT <= p.M && nbase + WT <= p.N;
    if (full) {
        if (p.has_beta) store_tile_staged<O, Acc, MF, true, true>(p, mbase, nbase, lane, acc, stg);
        else store_tile_staged<O, Acc, MF, false, true>(p, mbase, nbase, lane, acc, stg);
    } else {
        if (p.has_beta) store_tile_staged<O, Acc, MF, true, false>(p, mbase, nbase, lane, acc, stg);
        else store_tile_staged<O, Acc, MF, false, false>(p, mbase, nbase, lane, acc, stg);
    }
}

// Per-shape schedule: BAR_AT MFMAs of a slab's last k-slice run before its barrier; the slab's 16
// direct loads go out one per DS MFMA slots (N3 of them after the barrier, in the last k-slice
// of the previous slab, the rest from the start of the slab).
template <int MF, int TL = 256>
struct Sched {
    static constexpr int NLD = 2 * Geo<TL>::NL;          // loads per slab and wave
    static constexpr int BAR_AT = MF == 32 ? 4 : 8;
    static constexpr int DS = MF == 32 || TL == 128 ? 2 : 4;
    static constexpr int REM = Shape<MF, TL>::NMS - BAR_AT;   // MFMA slots after the barrier
    static constexpr int N3 = (REM + DS - 1) / DS;       // loads of slab s+2 in them
    static_assert(N3 <= NLD, "loads after the barrier");
    // every load of a slab finds a slot: N3 after the barrier, the rest in the first k-slices
    static_assert(N3 + ((Shape<MF, TL>::NS - 1) * Shape<MF, TL>::NMS + DS - 1) / DS >= NLD, "load slots");
};

// XF: the launch has a load transform on op(A) or op(B), applied to every fragment after its LDS
// read (the direct loads put raw operand bytes in LDS).  RS: operands go through registers
// (global -> VGPR -> LDS, same LDS image) for layouts the direct loads cannot take; the load
// transforms are then applied once per element on the way to LDS (XF stays off).  TL: the
// workgroup tile (256; 128 for mid-size products: two workgroups per CU, 16x16 shape, direct
// loads, no load transforms).
template <class TI, class TO, bool AK, bool BK, int MF, bool XF, bool RS = false, int TL = 256>
__global__ __launch_bounds__(NT, TL == 256 ? 1 : 2) void gemm_fast(GemmParams p) {
    static_assert(TL == 256 || (TL == 128 && MF == 16 && !XF && !RS), "tile variants");
    using acc_t = typename TI::acc_t;
    using accv_t = typename std::conditional<MF == 32, typename TI::accv_t, typename TI::accv16_t>::type;
    using SH = Shape<MF, TL>;
    using SC = Sched<MF, TL>;
    using G = Geo<TL>;
    constexpr int NF = SH::NF, NS = SH::NS, NMS = SH::NMS;
    constexpr int NL = G::NL;
    constexpr int E = TI::E;
    constexpr int BKE = SLAB_BYTES / E;       // K elements per slab
    using FA = Frag<E, AK, MF, TL>;
    using FB = Frag<E, BK, MF, TL>;
    // fragment reads per k-slice, issued in the order the next k-slice's MFMAs consume them:
    // A0, B0 .. B(NF-1), A1 .. A(NF-1)
    constexpr int NRD = 2 * NF;
    // two pipeline stages of both operands; after the main loop the stage-1 halves of A and B
    // (never used by the K tail) hold the four waves' epilogue staging buffers
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * G::OPND];
    constexpr int STG = stg_bytes<TO, G::WT>();
    static_assert(2 * STG <= G::KC, "two staging buffers fit in one operand stage");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // this workgroup's product and raster id inside it
    const int lid = select_batch<TI::E, (int)sizeof(typename TO::T)>(p, xcd_remap(blockIdx.x, gridDim.x),
                                                                    p.tiles_m * p.tiles_n);

    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const uint32_t lds0 = lds_addr(smem);
    uint8_t *const stg = smem + (wave < 2 ? 0 : G::OPND) + G::KC + (wave & 1) * STG;

    FA fa;
    FB fb;
    Loader<E, AK, MF, RS, TL> la;
    Loader<E, BK, MF, RS, TL> lb;
    // RS: one slab of this wave's chunks in flight between global memory and LDS
    u32x4 ra[RS ? NL : 1], rb[RS ? NL : 1];
    int m0 = 0, n0 = 0;
    auto set_tile = [&](int id) {
        int tm, tn;
        raster(id, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        m0 = tm * TL;
        n0 = tn * TL;
        la.init(wave, lane, m0, p.M, p.lda);
        lb.init(wave, lane, n0, p.N, p.ldb);
    };

    // full slabs through the pipeline; a register-staged M/N-contiguous operand leaves the slab
    // holding the last row of K to the guarded tail
    const int nfull = (RS && (!AK || !BK)) ? (p.K - 1) / BKE : p.K / BKE;
    accv_t acc[NF][NF];
    u32x4 af[2][NF], bf[2][NF];

    // fragment read q (0 .. NRD-1) of k-slice j of `stage` into fragment buffer `buf`, in the
    // order A0, B0 .. B(NF-1), A1 .. A(NF-1)
    auto rd = [&](int stage, int j, int buf, int q) {
        if (q == 0) fa.read(stage, 0, j, af[buf][0]);
        else if (q <= NF) fb.read(stage, q - 1, j, bf[buf][q - 1]);
        else fa.read(stage, q - NF, j, af[buf][q - NF]);
        if constexpr (XF) {
            // load transform on the fragment just read (a disabled one is a no-op)
            if (q == 0) af[buf][0] = zero_negative<E>(af[buf][0], p.xform_a);
            else if (q <= NF) bf[buf][q - 1] = zero_negative<E>(bf[buf][q - 1], p.xform_b);
            else af[buf][q - NF] = zero_negative<E>(af[buf][q - NF], p.xform_a);
        }
    };
    // reads issued with MFMA slot t of a k-slice (slots 0 .. NMS-1 spread NRD reads)
    auto rd_slot = [&](int stage, int j, int buf, int t, int slots) {
        if constexpr (MF == 32) {
            if (slots == NMS) {
                if (t < NRD) rd(stage, j, buf, t);
                return;
            }
        }
#pragma unroll
        for (int q = (t * NRD) / slots; q < ((t + 1) * NRD) / slots; ++q) rd(stage, j, buf, q);
    };
    // MFMA number t (0 .. NMS-1) of a k-slice: A fragment t/NF times B fragment t%NF
    auto mma = [&](int buf, int t) {
        const int i = t / NF, j = t % NF;

        if constexpr (MF == 32) acc[i][j] = TI::mma(bf[buf][j], af[buf][i], acc[i][j]);
        else acc[i][j] = TI::mma16(bf[buf][j], af[buf][i], acc[i][j]);
    };
    // LDS addresses of operand slabs in a stage
    auto dstA = [&](int st) { return lds0 + (uint32_t)(st * G::KC); };
    auto dstB = [&](int st) { return lds0 + (uint32_t)(G::OPND + st * G::KC); };
    auto issue_slab = [&](int s, int st) {
        const uint8_t *sa = Loader<E, AK, MF, RS, TL>::slab_base(A, p.lda, s * BKE);
        const uint8_t *sb = Loader<E, BK, MF, RS, TL>::slab_base(B, p.ldb, s * BKE);
#pragma unroll
        for (int i = 0; i < NL; ++i) la.issue(sa, dstA(st), wave, i);
#pragma unroll
        for (int i = 0; i < NL; ++i) lb.issue(sb, dstB(st), wave, i);
    };
    auto prologue = [&]() {
        if (nfull > 0) issue_slab(0, 0);
        if (nfull > 1) issue_slab(1, 1);
    };
    // RS: chunk d (0 .. NL-1 A, NL .. 2NL-1 B) of slab s into registers; register chunk d into
    // stage st
    auto rs_fetch = [&](int s, int d) {
        if (d < NL) ra[d] = la.fetch(Loader<E, AK, MF, RS, TL>::slab_base(A, p.lda, s * BKE), d);
        else rb[d - NL] = lb.fetch(Loader<E, BK, MF, RS, TL>::slab_base(B, p.ldb, s * BKE), d - NL);
    };
    auto rs_put = [&](int st, int d) {
        if (d < NL) la.put(smem + st * G::KC, wave, d, lane, ra[d], p.xform_a);
        else lb.put(smem + G::OPND + st * G::KC, wave, d - NL, lane, rb[d - NL], p.xform_b);
    };

    // Slab s reads stage X; slab s+1 lives in Y.  The NLD (16; 8 at TL = 128) loads of a slab are
    // spread one per DS MFMA slots: the first N3 go out in the last k-slice of slab s-2 (after
    // its barrier freed the stage), the rest from the start of slab s-1.  Bursting them all at
    // once fills the vector-memory queue and stalls the wave's in-order issue (MFMAs too).
    //   dma_next:  issue loads N3..NLD-1 of slab s+1 into Y (its first loads went out in slab s-1)
    //   dma_next2: issue loads 0..N3-1 of slab s+2 into X
    //   has_next:  slab s+1 exists (wait for it, read its k-slice 0)
    //   RS: in the first k-slices, chunk by chunk, the registers (slab s+1) go to Y and are
    //   refilled with slab s+2 (has_next, dma_next2); the barrier then waits for LDS only
    auto slab_step = [&](int s, int X, int Y, bool dma_next, bool dma_next2, bool has_next) {
        const uint8_t *na = Loader<E, AK, MF, RS, TL>::slab_base(A, p.lda, (s + 1) * BKE);
        const uint8_t *nb = Loader<E, BK, MF, RS, TL>::slab_base(B, p.ldb, (s + 1) * BKE);
        const uint8_t *n2a = Loader<E, AK, MF, RS, TL>::slab_base(A, p.lda, (s + 2) * BKE);
        const uint8_t *n2b = Loader<E, BK, MF, RS, TL>::slab_base(B, p.ldb, (s + 2) * BKE);
        auto dma = [&](const uint8_t *sa, const uint8_t *sb, int st, int d) {
            if (d < NL) la.issue(sa, dstA(st), wave, d);
            else lb.issue(sb, dstB(st), wave, d - NL);
        };
        // k-slices 0 .. NS-2: MFMAs of slice j interleaved with the reads of slice j+1
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) {
#pragma unroll
            for (int t = 0; t < NMS; ++t) {
                mma(j & 1, t);
                rd_slot(X, j + 1, (j + 1) & 1, t, NMS);
                const int q = NMS * j + t;                       // load slot in the slab
                if constexpr (RS) {
                    if (q % 2 == 0 && q / 2 < SC::NLD) {
                        if (has_next) rs_put(Y, q / 2);
                        if (dma_next2) rs_fetch(s + 2, q / 2);
                    }
                } else if (dma_next) {
                    if (q % SC::DS == 0 && SC::N3 + q / SC::DS < SC::NLD) dma(na, nb, Y, SC::N3 + q / SC::DS);
                }
                fence();
            }
        }
        // last k-slice: every read of X has been issued.  The first BAR_AT MFMAs run while those
        // reads land; then the wave finishes them and its loads of slab s+1 and meets the others
        // at the barrier; then it starts refilling X with slab s+2 and reads slice 0 of Y while
        // the remaining MFMAs run.
        constexpr int LB = (NS - 1) & 1;                         // fragment buffer of the slice
#pragma unroll
        for (int t = 0; t < SC::BAR_AT; ++t) {
            mma(LB, t);
            fence();
        }
        wait_lgkmcnt0();
        if (has_next && !RS) wait_vmcnt0();
        fence();
        __syncthreads();
        fence();
#pragma unroll
        for (int t = SC::BAR_AT; t < NMS; ++t) {
            mma(LB, t);
            const int u = t - SC::BAR_AT;                        // slot after the barrier
            if (!RS && dma_next2 && u % SC::DS == 0) dma(n2a, n2b, X, u / SC::DS);
            if (has_next) rd_slot(Y, 0, 0, u, SC::REM);
            fence();
        }
    };

    set_tile(lid);
    fa.init(lane, wm * G::WT, lds0);
    fb.init(lane, wn * G::WT, lds0 + G::OPND);
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int r = 0; r < (MF == 32 ? 16 : 4); ++r) acc[i][j][r] = 0;

    if (nfull > 0) {
        if constexpr (RS) {
            // slab 0 to stage 0 through the registers; slab 1 stays in them
#pragma unroll
            for (int d = 0; d < 2 * NL; ++d) rs_fetch(0, d);
#pragma unroll
            for (int d = 0; d < 2 * NL; ++d) rs_put(0, d);
            if (nfull > 1)
#pragma unroll
                for (int d = 0; d < 2 * NL; ++d) rs_fetch(1, d);
        } else {
            prologue();
            // slab 0 landed, slab 1 (its 2 NL loads) may still fly
            if (nfull > 1) {
                if constexpr (NL == 8) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            } else {
                wait_vmcnt0();
            }
        }
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
        TailStage<E, AK, MF, TL> ta;
        TailStage<E, BK, MF, TL> tb;
        ta.fetch(A, p.lda, m0, p.M, k0, p.K, tid);
        tb.fetch(B, p.ldb, n0, p.N, k0, p.K, tid);
        __syncthreads();
        ta.put(smem, tid, RS ? p.xform_a : 0);
        tb.put(smem + G::OPND, tid, RS ? p.xform_b : 0);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NS; ++j) {   // the k-slices of the slab
#pragma unroll
            for (int q = 0; q < NRD; ++q) rd(0, j, 0, q);
#pragma unroll
            for (int t = 0; t < NMS; ++t) mma(0, t);
        }
    }

    // every wave's reads of the stage-1 buffers ended before the last slab's barrier
    epilogue<TO, acc_t, MF>(p, m0 + wm * G::WT, n0 + wn * G::WT, lane, acc, stg);
}

// MFMA shape of the fast path.  Both shapes give the same results (fp32/int32 accumulation of
// the same products); the 16x16 one (K = 32 fp16/bf16 or 64 int8 per instruction) moves half
// as much accumulator data per multiply-add, which on this power-limited part keeps the clock
// higher: ~10% more throughput at 8192^3 than the 32x32 shape.  With both operands M/N-
// contiguous (A transposed, B not) the 16x16 schedule needs more registers than the allocator
// finds without shuffling accumulators, so that layout keeps the 32x32 shape when it is read in
// place.
template <bool AT, bool BT>
constexpr int fast_mf() { return (AT && !BT) ? 32 : 16; }

template <class TI, class TO, bool AT, bool BT>
hipError_t launch_fast(const GemmParams &p, unsigned grid, hipStream_t s) {
    // load transforms on op(A)/op(B) run on the fragments; with the 16x16 schedule the extra
    // VALU work on fragment registers makes the allocator shuffle accumulators, the 32x32 one
    // stays clean
    if (p.xform_a || p.xform_b)
        hipLaunchKernelGGL((gemm_fast<TI, TO, !AT, BT, 32, true>), dim3(grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_fast<TI, TO, !AT, BT, fast_mf<AT, BT>(), false>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// Register-staged launch: every operand pointer, leading dimension and extent.  Always with the
// 32x32 shape (its register budget leaves room for the staging registers); the load transforms
// run in the staging step.
template <class TI, class TO, bool AT, bool BT>
hipError_t launch_fast_rs(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_fast<TI, TO, !AT, BT, 32, false, true>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO>
const KernelEntry *lookup_fast(int op_a, int op_b, int rs) {
    constexpr int BKE = SLAB_BYTES / TI::E;
    static const KernelEntry e[8] = {
        {launch_fast<TI, TO, false, false>, 256, 256, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, false, true>, 256, 256, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, true, false>, 256, 256, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast<TI, TO, true, true>, 256, 256, BKE, 2, 2, "gemm_fast_256x256"},
        {launch_fast_rs<TI, TO, false, false>, 256, 256, BKE, 2, 2, "gemm_fast_256x256_rs"},
        {launch_fast_rs<TI, TO, false, true>, 256, 256, BKE, 2, 2, "gemm_fast_256x256_rs"},
        {launch_fast_rs<TI, TO, true, false>, 256, 256, BKE, 2, 2, "gemm_fast_256x256_rs"},
        {launch_fast_rs<TI, TO, true, true>, 256, 256, BKE, 2, 2, "gemm_fast_256x256_rs"},
    };
    if (op_a < 0 || op_a > 1 || op_b < 0 || op_b > 1) return nullptr;
    return &e[(rs ? 4 : 0) + op_a * 2 + op_b];
}

// 128 x 128 tiles for mid-size products (direct loads, no load transforms): 4
// waves of 64 x 64 and two workgroups per CU, so that a product with a few hundred 128-wide
// tiles fills the chip that its few dozen 256-wide tiles would leave mostly idle.
template <class TI, class TO, bool AT, bool BT>
hipError_t launch_fast128(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_fast<TI, TO, !AT, BT, 16, false, false, 128>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO>
const KernelEntry *lookup_fast128(int op_a, int op_b) {
    constexpr int BKE = SLAB_BYTES / TI::E;
    static const KernelEntry e[4] = {
        {launch_fast128<TI, TO, false, false>, 128, 128, BKE, 2, 2, "gemm_fast_128x128"},
        {launch_fast128<TI, TO, false, true>, 128, 128, BKE, 2, 2, "gemm_fast_128x128"},
        {launch_fast128<TI, TO, true, false>, 128, 128, BKE, 2, 2, "gemm_fast_128x128"},
        {launch_fast128<TI, TO, true, true>, 128, 128, BKE, 2, 2, "gemm_fast_128x128"},
    };
    if (op_a < 0 || op_a > 1 || op_b < 0 || op_b > 1) return nullptr;
    return &e[op_a * 2 + op_b];
}

}  // namespace

#if defined(TGE_PAIR_F16_F16)
const KernelEntry *fast_f16_f16(int a, int b, int rs) { return lookup_fast<TF16, OF16>(a, b, rs); }
const KernelEntry *fast128_f16_f16(int a, int b) { return lookup_fast128<TF16, OF16>(a, b); }
#elif defined(TGE_PAIR_F16_F32)
const KernelEntry *fast_f16_f32(int a, int b, int rs) { return lookup_fast<TF16, OF32>(a, b, rs); }
const KernelEntry *fast128_f16_f32(int a, int b) { return lookup_fast128<TF16, OF32>(a, b); }
#elif defined(TGE_PAIR_BF16_BF16)
const KernelEntry *fast_bf16_bf16(int a, int b, int rs) { return lookup_fast<TBF16, OBF16>(a, b, rs); }
const KernelEntry *fast128_bf16_bf16(int a, int b) { return lookup_fast128<TBF16, OBF16>(a, b); }
#elif defined(TGE_PAIR_BF16_F32)
const KernelEntry *fast_bf16_f32(int a, int b, int rs) { return lookup_fast<TBF16, OF32>(a, b, rs); }
const KernelEntry *fast128_bf16_f32(int a, int b) { return lookup_fast128<TBF16, OF32>(a, b); }
#elif defined(TGE_PAIR_I8_I32)
const KernelEntry *fast_i8_i32(int a, int b, int rs) { return lookup_fast<TI8, OI32>(a, b, rs); }
const KernelEntry *fast128_i8_i32(int a, int b) { return lookup_fast128<TI8, OI32>(a, b); }
#else
#error "define one TGE_PAIR_* macro with a 16- or 8-bit input type"
#endif

}  // namespace tge
