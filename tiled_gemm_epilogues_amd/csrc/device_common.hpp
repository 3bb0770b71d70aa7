// Device-side building blocks shared by the GEMM kernels (gfx950): element-type traits with
// their MFMA step, unaligned 16-byte loads, the XCD-aware tile scheduler and the fused
// register epilogue.  Included only by the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_internal.h"

namespace tge {
namespace dev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
    using accv16_t = f32x4;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // 16x16 output, K = 32 per step (8 values per lane and operand, as above)
    __device__ static accv16_t mma16(u32x4 a, u32x4 b, accv16_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
struct TBF16 {
    static constexpr int E = 2;
    using acc_t = float;
    using accv_t = f32x16;
    using accv16_t = f32x4;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static accv16_t mma16(u32x4 a, u32x4 b, accv16_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
struct TI8 {
    static constexpr int E = 1;
    using acc_t = int;
    using accv_t = i32x16;
    using accv16_t = i32x4;
    __device__ static accv_t mma(u32x4 a, u32x4 b, accv_t c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
    // 16x16 output, K = 64 per step (16 values per lane and operand)
    __device__ static accv16_t mma16(u32x4 a, u32x4 b, accv16_t c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
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

// Load transform GEMM_TRANSFORM_RELU on a 16-byte chunk of E-byte elements: every element whose
// sign bit is set becomes +0 (max(x, 0) for every non-NaN x; the same rule for fp16, bf16 and
// int8 as 16- or 8-bit two's-complement sign tests, and for fp32 / int32 as 32-bit ones).
// Branch-free with the enable `on` (uniform 0/1), so it can sit inside a software pipeline.
template <int E>
__device__ __forceinline__ u32x4 zero_negative(u32x4 v, int on) {
    if constexpr (E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (on && (int)v[i] < 0) ? 0u : v[i];
    } else if constexpr (E == 2) {
        typedef short s2 __attribute__((ext_vector_type(2)));
        const short fl = on ? (short)0 : (short)-32768;   // max(x, -32768) leaves x unchanged
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = v[i];   // bit_cast of a vector-element lvalue would read element 0
            const s2 h = __builtin_bit_cast(s2, w);
            v[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(h, (s2){fl, fl}));
        }
    } else {
        // sign bits m (0x80 per negative byte) -> whole-byte masks m | (m - m/128); no byte
        // borrows from its neighbour because each byte of m is >= the same byte of m >> 7
        const uint32_t sel = on ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t m = v[i] & sel;
            v[i] &= ~(m | (m - (m >> 7)));
        }
    }
    return v;
}

// A C element as the epilogue uses it: in the accumulation type, with the load transform
// (relu_in: sign bit set -> +0) applied.
template <class T>
__device__ __forceinline__ float c_in_f(T c, int relu_in) {
    const float f = (float)c;
    return (relu_in && __builtin_bit_cast(int, f) < 0) ? 0.0f : f;
}
__device__ __forceinline__ int c_in_i(int c, int relu_in) { return (relu_in && c < 0) ? 0 : c; }

// Strided batch: workgroup id -> (product b, id inside the product, `per` ids per product); the
// operand pointers of `p` are moved to product b.  Consecutive ids share a product, so the
// XCD-contiguous id ranges of xcd_remap keep each product on few XCDs.  With two batch modes
// product b is (b1, b2) = (b / batch2, b % batch2), moved by b1 * stride + b2 * stride2: the
// index map of a tensor contraction whose batch index has two modes with their own strides.
template <int EAB, int ECD>
__device__ __forceinline__ int select_batch(GemmParams &p, int id, int per) {
    const int b = __builtin_amdgcn_readfirstlane(id / per);   // uniform: keeps pointers scalar
    if (b > 0) {
        const int b1 = __builtin_amdgcn_readfirstlane(b / p.batch2);
        const int b2 = b - b1 * p.batch2;
        const int64_t oa = b1 * p.stride_a + b2 * p.stride2_a, ob = b1 * p.stride_b + b2 * p.stride2_b;
        const int64_t oc = b1 * p.stride_c + b2 * p.stride2_c, obias = b1 * p.stride_bias + b2 * p.stride2_bias;
        p.A = static_cast<const uint8_t *>(p.A) + oa * EAB;
        p.B = static_cast<const uint8_t *>(p.B) + ob * EAB;
        if (p.C) p.C = static_cast<const uint8_t *>(p.C) + oc * ECD;
        p.D = static_cast<uint8_t *>(p.D) + oc * ECD;
        if (p.bias) p.bias = static_cast<const uint8_t *>(p.bias) + obias * 4;
    }
    return __builtin_amdgcn_readfirstlane(id - b * per);
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

// ---- epilogue --------------------------------------------------------------------------------

// Epilogue of a wave's MFMA tiles.  Lane l holds, for 32x32 tile (i, j), accumulator register
// 4g+e = D[mbase + 32i + l%32][nbase + 32j + 8g + 4(l/32) + e].  The bias values of the wave's
// columns are loaded once, the C values of one 32-row block are loaded together before any of
// its stores (C == D is allowed: every element is read before the same lane writes it), so the
// loads overlap instead of each waiting for the store before it.
template <class O, class Acc, class AccV, int TM, int TN>
__device__ __forceinline__ void store_tile(const GemmParams &p, int mbase, int nbase, int lane,
                                           AccV (&acc)[TM][TN]) {
    using T = typename O::T;
    constexpr bool INT = std::is_same<Acc, int>::value;
    using B = typename std::conditional<INT, int, float>::type;
    const int hi = lane >> 5, rl = lane & 31;
    const int N = p.N;
    const bool full_n = nbase + 32 * TN <= N;
    const B *bias = static_cast<const B *>(p.bias);
    const T *C = static_cast<const T *>(p.C);
    T *D = static_cast<T *>(p.D);

    B bv[TN][4][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = nbase + 32 * j + 8 * g + 4 * hi;
            if (p.has_bias && full_n) {
                __builtin_memcpy(bv[j][g], bias + n, sizeof(bv[j][g]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[j][g][e] = (p.has_bias && n + e < N) ? bias[n + e] : (B)0;
            }
        }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = mbase + 32 * i + rl;
        if (m >= p.M) continue;
        const int64_t row = (int64_t)m * p.ldc;
        T cv[TN][4][4];
        if (p.has_beta) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nbase + 32 * j + 8 * g + 4 * hi;
                    if (full_n) {
                        __builtin_memcpy(cv[j][g], C + row + n, sizeof(cv[j][g]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) cv[j][g][e] = (n + e < N) ? C[row + n + e] : (T)0;
                    }
                }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nbase + 32 * j + 8 * g + 4 * hi;
                T out[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (INT) {
                        // integer path: alpha == 1, beta in {0, 1}
                        int t = acc[i][j][4 * g + e] + bv[j][g][e];
                        if (p.has_beta) t += c_in_i((int)cv[j][g][e], p.xform_c);
                        if (p.relu) t = t > 0 ? t : 0;
                        out[e] = (T)t;
                    } else {
                        float t = p.alpha * acc[i][j][4 * g + e];
                        if (p.has_beta) t += p.beta * c_in_f(cv[j][g][e], p.xform_c);
                        t += bv[j][g][e];
                        if (p.relu) t = t > 0.0f ? t : 0.0f;
                        out[e] = (T)t;
                    }
                }
                if (full_n) {
                    __builtin_memcpy(D + row + n, out, sizeof(out));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) D[row + n + e] = out[e];
                }
            }
    }
}

}  // namespace dev
}  // namespace tge
