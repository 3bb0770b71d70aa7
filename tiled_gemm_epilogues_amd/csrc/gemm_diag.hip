// Products with a diagonal operand ("Flexible Performant GEMM Kernels on GPUs", section 5.2 and
// Table 1): D = epilogue(alpha * diag(a) op(B) + beta * C), epilogue(alpha * op(A) diag(b) + ...)
// or epilogue(alpha * diag(a) diag(b) + ...), the diagonal operand given as its vector.
//
// A diagonal matrix has one nonzero per row and column, so every output element takes exactly
// one product: a[m] * op(B)[m][n], op(A)[m][n] * b[n], or a[m] * b[m] on the diagonal.  The
// work is a scaled copy of the dense operand fused with the epilogue, bounded by HBM bandwidth
// (read the dense operand and C once, write D once), not a contraction: it is streamed with
// 16-byte loads and stores instead of running the MFMA pipeline over the one nonzero band.
//   * dense operand stored like D (row-major in m, n): each lane owns one 16-byte chunk of a row,
//     eight rows per wave, so every load and store instruction of a wave covers whole lines;
//   * dense operand stored transposed (op T): 64 x 64 tiles go through LDS, read along the
//     stored rows and written along the rows of D.
// The products are exact in fp32 for fp16/bf16 inputs (and in int32 for int8), so the results
// equal those of a GEMM kernel that multiplies the stored zeros; the zeros are never formed.
#include "device_common.hpp"

namespace tge {
namespace {

using namespace dev;

template <class TI>
struct Elt;
template <>
struct Elt<TF16> { using T = _Float16; using A = float; };
template <>
struct Elt<TBF16> { using T = __bf16; using A = float; };
template <>
struct Elt<TF32> { using T = float; using A = float; };
template <>
struct Elt<TI8> { using T = int8_t; using A = int; };

constexpr int NT = 256;

// 16 bytes with no alignment requirement, for non-temporal (streaming) stores of D
typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(1)));

// One element of a vector or matrix of E-byte elements, in the accumulation type, with the load
// transform (sign bit set -> +0) applied when `xf` is set.
template <class TI>
__device__ __forceinline__ typename Elt<TI>::A load_elt(const uint8_t *base, int64_t i, int xf) {
    using T = typename Elt<TI>::T;
    T v;
    __builtin_memcpy(&v, base + i * (int64_t)sizeof(T), sizeof(T));
    u32x4 w = {0, 0, 0, 0};
    __builtin_memcpy(&w, &v, sizeof(T));
    w = zero_negative<(int)sizeof(T)>(w, xf);
    __builtin_memcpy(&v, &w, sizeof(T));
    return (typename Elt<TI>::A)v;
}

// Elements i0 .. i0+n-1 (n <= VE, VE elements per 16-byte chunk of the vector's type) of a
// vector in the accumulation type, with the load transform; whole chunks in one load.
template <class TI, int VE>
__device__ __forceinline__ void load_run(const uint8_t *base, int64_t i0, int n, int xf,
                                         typename Elt<TI>::A (&out)[VE]) {
    using T = typename Elt<TI>::T;
    constexpr int E = (int)sizeof(T);
    static_assert(VE * E % 16 == 0, "whole chunks");
    T v[VE];
    if (n == VE) {
#pragma unroll
        for (int q = 0; q < VE * E / 16; ++q) {
            u32x4 w = zero_negative<E>(ldg16(base + (i0 * E + q * 16)), xf);
            __builtin_memcpy(reinterpret_cast<uint8_t *>(v) + q * 16, &w, 16);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) out[e] = (typename Elt<TI>::A)v[e];
    } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) out[e] = e < n ? load_elt<TI>(base, i0 + e, xf) : (typename Elt<TI>::A)0;
    }
}

// bias[n0 .. n0+n-1] (n <= VE), zero when absent
template <class Acc, int VE>
__device__ __forceinline__ void load_bias(const GemmParams &p, int n0, int n, Acc (&out)[VE]) {
    const Acc *b = static_cast<const Acc *>(p.bias) + n0;
    if (p.has_bias && n == VE) {
        __builtin_memcpy(out, b, sizeof(out));
    } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) out[e] = p.has_bias && e < n ? b[e] : (Acc)0;
    }
}

// The epilogue of one output element (the same arithmetic as the tiled kernels' epilogues).
template <class TO, class Acc>
__device__ __forceinline__ typename TO::T epi_one(const GemmParams &p, Acc acc, typename TO::T c, Acc bias) {
    using T = typename TO::T;
    if constexpr (std::is_same<Acc, int>::value) {
        int t = acc + bias;
        if (p.has_beta) t += c_in_i((int)c, p.xform_c);
        if (p.relu) t = t > 0 ? t : 0;
        return (T)t;
    } else {
        float t = p.alpha * acc;
        if (p.has_beta) t = __builtin_fmaf(p.beta, c_in_f(c, p.xform_c), t);
        t += bias;
        if (p.relu) t = t > 0.0f ? t : 0.0f;
        return (T)t;
    }
}

// D[n0 .. n0+n-1] of one row (n <= VE): whole runs as 16-byte stores, non-temporal when NTS
// (measured: faster for the row kernel's whole-line stream, slower for the tile kernel), else
// element by element
template <bool NTS, class T, int VE>
__device__ __forceinline__ void store_run(T *row, int n0, int n, const T (&out)[VE]) {
    static_assert(sizeof(out) % 16 == 0, "whole chunks");
    T *dst = row + n0;
    if (n == VE) {
        u32x4 o[sizeof(out) / 16];
        __builtin_memcpy(o, out, sizeof(out));
#pragma unroll
        for (int q = 0; q < (int)(sizeof(out) / 16); ++q) {
            uint8_t *d = reinterpret_cast<uint8_t *>(dst) + 16 * q;
            if constexpr (NTS) __builtin_nontemporal_store((u32x4u)o[q], reinterpret_cast<u32x4u *>(d));
            else __builtin_memcpy(d, &o[q], 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (e < n) dst[e] = out[e];
    }
}

// Row-major output tile: RT rows x (64 * VE) columns; wave w owns rows RPW*w .. RPW*w+RPW-1,
// lane l the VE columns starting at 64-lane chunk l.  DG: 1 = A diagonal, 2 = B diagonal, 3 = both (then
// there is no dense operand).  The dense operand of DG 1 / 2 is stored like D here.
constexpr int RPW = 8;   // rows per wave
constexpr int RT = 4 * RPW;

template <class TI, class TO, int DG>
__global__ __launch_bounds__(NT) void diag_rows(GemmParams p) {
    using X = typename Elt<TI>::T;
    using Acc = typename Elt<TI>::A;
    using T = typename TO::T;
    constexpr int E = (int)sizeof(X);
    constexpr int VE = 16 / E;
    const int id = select_batch<E, (int)sizeof(T)>(p, blockIdx.x, p.tiles_m * p.tiles_n);
    const int tm = id / p.tiles_n, tn = id - tm * p.tiles_n;
    // the wave index is uniform: the row factors below are then one broadcast load per wave
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = tn * (64 * VE) + lane * VE;
    const int m0 = tm * RT + wave * RPW;
    if (n >= p.N || m0 >= p.M) return;   // no barriers below
    const int nv = min(VE, p.N - n);      // valid columns of the lane's chunk

    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    // the dense operand and its leading dimension / transform
    const uint8_t *Xp = DG == 1 ? B : A;
    const int ldx = DG == 1 ? p.ldb : p.lda;
    const int xfx = DG == 1 ? p.xform_b : p.xform_a;

    // column factors (B diagonal) and bias: once per lane
    Acc colf[VE], bias[VE];
    if constexpr ((DG & 2) != 0) load_run<TI, VE>(B, n, nv, p.xform_b, colf);
    load_bias<Acc, VE>(p, n, nv, bias);

    // row factors (A diagonal): the wave's RPW consecutive elements of the vector at once
    Acc rowf[RPW];
    if constexpr ((DG & 1) != 0) {
        if (m0 + RPW <= p.M) {
            X v[RPW];
            __builtin_memcpy(v, A + (int64_t)m0 * E, sizeof(v));
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                u32x4 w = {0, 0, 0, 0};
                __builtin_memcpy(&w, &v[r], E);
                w = zero_negative<E>(w, p.xform_a);
                __builtin_memcpy(&v[r], &w, E);
                rowf[r] = (Acc)v[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < RPW; ++r) rowf[r] = m0 + r < p.M ? load_elt<TI>(A, m0 + r, p.xform_a) : (Acc)0;
        }
    }

    // loads of all rows first (dense chunks and C), then the arithmetic and the stores
    X xv[RPW][VE];
    T cv[RPW][VE];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int m = m0 + r;
        const bool ok = m < p.M;
        if constexpr (DG != 3) {
            u32x4 w = {0, 0, 0, 0};
            const uint8_t *src = Xp + ((int64_t)m * ldx + n) * E;
            if (ok && nv == VE) w = ldg16(src);
            else if (ok) w = ldg16_partial<E>(src, nv);
            w = zero_negative<E>(w, xfx);
            __builtin_memcpy(xv[r], &w, 16);
        }
        if (p.has_beta) {
            const T *src = static_cast<const T *>(p.C) + (int64_t)m * p.ldc + n;
            if (ok && nv == VE) {
                __builtin_memcpy(cv[r], src, sizeof(cv[r]));
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) cv[r][e] = ok && e < nv ? src[e] : (T)0;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int m = m0 + r;
        if (m >= p.M) break;
        T out[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            Acc acc;
            if constexpr (DG == 1) acc = rowf[r] * (Acc)xv[r][e];
            else if constexpr (DG == 2) acc = (Acc)xv[r][e] * colf[e];
            else acc = (m == n + e) ? rowf[r] * colf[e] : (Acc)0;
            out[e] = epi_one<TO, Acc>(p, acc, p.has_beta ? cv[r][e] : (T)0, bias[e]);
        }
        store_run<true, T, VE>(static_cast<T *>(p.D) + (int64_t)m * p.ldc, n, nv, out);
    }
}

// Dense operand stored transposed: X[m][n] at Xs[n * ldx + m].  A 64 x 64 output tile: the 64
// stored rows n0 .. n0+63 (64 contiguous m each) are loaded in 16-byte chunks into LDS, then
// thread t writes row m0 + t/4, columns n0 + 16(t%4) .. +15 of D.
constexpr int TT = 64;

template <class TI, class TO, int DG>
__global__ __launch_bounds__(NT) void diag_cols(GemmParams p) {
    using X = typename Elt<TI>::T;
    using Acc = typename Elt<TI>::A;
    using T = typename TO::T;
    constexpr int E = (int)sizeof(X);
    constexpr int VE = 16 / E;
    constexpr int CPR = TT / VE;                 // chunks per stored row of the tile
    constexpr int PITCH = TT * E + 4;            // LDS row pitch in bytes (4-byte aligned, skewed)
    __shared__ __attribute__((aligned(16))) uint8_t tile[TT * PITCH];

    const int id = select_batch<E, (int)sizeof(T)>(p, blockIdx.x, p.tiles_m * p.tiles_n);
    const int tm = id / p.tiles_n, tn = id - tm * p.tiles_n;
    const int m0 = tm * TT, n0 = tn * TT;
    const int tid = threadIdx.x;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const uint8_t *Xp = DG == 1 ? B : A;
    const int ldx = DG == 1 ? p.ldb : p.lda;
    const int xfx = DG == 1 ? p.xform_b : p.xform_a;

    // this thread's outputs: row m0 + ml, columns nbase .. nbase + nv - 1
    const int ml = tid >> 2, nb = (tid & 3) * 16;
    const int m = m0 + ml;
    const int nbase = n0 + nb;
    const int nv = min(16, p.N - nbase);
    const bool live = m < p.M && nv > 0;

    // every load first: the tile's chunks of the dense operand, then C, the scale factors and
    // the bias of this thread's outputs
    constexpr int NCH = TT * CPR / NT;
    u32x4 w[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = tid + NT * i;
        const int r = q / CPR, c = q % CPR;     // stored row n0 + r, elements m0 + c*VE ..
        const int nn = n0 + r, mm = m0 + c * VE;
        const int mv = p.M - mm;
        const uint8_t *src = Xp + ((int64_t)nn * ldx + mm) * E;
        w[i] = u32x4{0, 0, 0, 0};
        if (nn < p.N && mv >= VE) w[i] = ldg16(src);
        else if (nn < p.N && mv > 0) w[i] = ldg16_partial<E>(src, mv);
    }
    T cv[16];
    Acc rowf = 0, colf[16], bias[16];
    if (live) {
        if (p.has_beta) {
            const T *src = static_cast<const T *>(p.C) + (int64_t)m * p.ldc + nbase;
            if (nv == 16) {
                __builtin_memcpy(cv, src, sizeof(cv));
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) cv[j] = j < nv ? src[j] : (T)0;
            }
        }
        if constexpr ((DG & 1) != 0) rowf = load_elt<TI>(A, m, p.xform_a);
        if constexpr ((DG & 2) != 0) load_run<TI, 16>(B, nbase, nv, p.xform_b, colf);
        load_bias<Acc, 16>(p, nbase, nv, bias);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = tid + NT * i;
        const int r = q / CPR, c = q % CPR;
        const u32x4 v = zero_negative<E>(w[i], xfx);
        uint32_t *d = reinterpret_cast<uint32_t *>(tile + r * PITCH + c * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) d[k] = v[k];
    }
    __syncthreads();
    if (!live) return;   // after the only barrier

    T out[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        X x;
        __builtin_memcpy(&x, tile + (nb + j) * PITCH + ml * E, E);
        const Acc acc = DG == 1 ? rowf * (Acc)x : (Acc)x * colf[j];
        out[j] = epi_one<TO, Acc>(p, acc, p.has_beta ? cv[j] : (T)0, bias[j]);
    }
    store_run<false, T, 16>(static_cast<T *>(p.D) + (int64_t)m * p.ldc, nbase, nv, out);
}

template <class TI, class TO, int DG>
hipError_t launch_rows(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((diag_rows<TI, TO, DG>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <class TI, class TO, int DG>
hipError_t launch_cols(const GemmParams &p, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((diag_cols<TI, TO, DG>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// dg: bit 0 = A diagonal, bit 1 = B diagonal.  The layout of the dense operand picks the kernel
// (that of a diagonal one does not matter: it is a vector).
template <class TI, class TO>
const KernelEntry *lookup(int op_a, int op_b, int dg) {
    constexpr int CT = 64 * 16 / (int)sizeof(typename Elt<TI>::T);
    static const KernelEntry e[5] = {
        {launch_rows<TI, TO, 1>, RT, CT, 1, 4, 1, "gemm_diag_rows"},
        {launch_cols<TI, TO, 1>, TT, TT, 1, 4, 1, "gemm_diag_cols"},
        {launch_rows<TI, TO, 2>, RT, CT, 1, 4, 1, "gemm_diag_rows"},
        {launch_cols<TI, TO, 2>, TT, TT, 1, 4, 1, "gemm_diag_cols"},
        {launch_rows<TI, TO, 3>, RT, CT, 1, 4, 1, "gemm_diag_rows"},
    };
    if (dg == 1) return &e[op_b ? 1 : 0];
    if (dg == 2) return &e[op_a ? 3 : 2];
    if (dg == 3) return &e[4];
    return nullptr;
}

}  // namespace

const KernelEntry *diag_f32_f32(int a, int b, int dg) { return lookup<TF32, OF32>(a, b, dg); }
const KernelEntry *diag_f16_f16(int a, int b, int dg) { return lookup<TF16, OF16>(a, b, dg); }
const KernelEntry *diag_f16_f32(int a, int b, int dg) { return lookup<TF16, OF32>(a, b, dg); }
const KernelEntry *diag_bf16_bf16(int a, int b, int dg) { return lookup<TBF16, OBF16>(a, b, dg); }
const KernelEntry *diag_bf16_f32(int a, int b, int dg) { return lookup<TBF16, OF32>(a, b, dg); }
const KernelEntry *diag_i8_i32(int a, int b, int dg) { return lookup<TI8, OI32>(a, b, dg); }

}  // namespace tge
