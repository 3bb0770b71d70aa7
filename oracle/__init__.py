"""CPU oracle for D = act(alpha * op(A) * op(B) + beta * C + bias): TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its binding) never does, and shares no code
with it.  The arithmetic lives in oracle.c (plain C, fp64 / int64); this module only marshals
numpy arrays.

What it computes (cited by page title and section):
  * "CUTLASS: Fast Linear Algebra in CUDA C++", "Efficient Matrix Multiplication on GPUs":
    C = alpha*A*B + beta*C, summed by the naive, k-outermost or tiled loop nest (order 0/1/2),
    all with ascending k per element.
  * same page, "Fusing Element-wise Operations": alpha*acc + bias + beta*c, then max(0, .).
  * "Flexible Performant GEMM Kernels on GPUs", section 5.3: the bias vector is added to every
    row (bias[j] for output column j).
Readings where the pages are silent (all matrices row-major, op T = the stored array is the
transpose, beta == 0 means C is not read, RNE to the output type) are stated in oracle.c.

Raw operand formats (the exact bits a kernel receives): f32 -> numpy float32, f16 and bf16 ->
numpy uint16 bit patterns, i8 -> int8, i32 -> int32; complex / dual numbers (cf16, df16, cf32,
df32) -> interleaved pairs of their part type.  Matrices are flat or 2-D C-contiguous
arrays with an explicit leading dimension.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB lets the mutation tests load a deliberately broken build of oracle.c
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "f64": 5}
RAW_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "i32": np.int32,
          "f64": np.float64}
ORDERS = {"ijk": 0, "kij": 1, "tiled": 2}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, dbl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        L.oracle_decode_f64.argtypes = [ci, vp, i64, vp]
        L.oracle_decode_i64.argtypes = [ci, vp, i64, vp]
        L.oracle_round_to.argtypes = [ci, vp, i64, vp]
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = dbl
        L.oracle_f64_to_f16.argtypes = [dbl]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [dbl]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_gather_f64.argtypes = [ci, i64, i64, vp, i64, vp]
        L.oracle_gather_i64.argtypes = [ci, i64, i64, vp, i64, vp]
        L.oracle_matmul_f64.argtypes = [ci, i64, i64, i64, vp, vp, vp, i64, i64, ci]
        L.oracle_matmul_i64.argtypes = [ci, i64, i64, i64, vp, vp, vp, i64, i64, ci]
        L.oracle_epilogue_f64.argtypes = [i64, i64, vp, dbl, vp, dbl, vp, ci, vp]
        L.oracle_epilogue_i64.argtypes = [i64, i64, vp, i64, vp, i64, vp, ci, vp]
        L.oracle_epilogue_i64.restype = ci
        for name, acc in (("oracle_points_f64", dbl), ("oracle_points_i64", i64)):
            getattr(L, name).argtypes = [i64, vp, vp, i64, ci, ci, ci, vp, i64, vp, i64, ci, vp, i64,
                                         ci, vp, acc, acc, ci, vp]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _raw_store(transform, ab, a):
    """Flat raw storage of an operand in its stored type (the source type of a conversion)."""
    return _raw(CONVERT_FROM.get(transform, ab), a)


def _raw(dtype, a):
    a = np.ascontiguousarray(a)
    want = RAW_NP[dtype]
    if a.dtype != want:
        if dtype in ("f16", "bf16") and a.dtype.itemsize == 2:
            a = a.view(np.uint16)
        else:
            raise TypeError(f"raw {dtype} data must be {np.dtype(want)}, got {a.dtype}")
    return a.reshape(-1)


def is_int(dtype):
    return dtype in ("i8", "i32")


def decode(dtype, a):
    """Exact value of every element: float64 for float types, int64 for integer types."""
    shape = np.shape(a)
    r = _raw(dtype, a)
    if is_int(dtype):
        out = np.empty(r.size, np.int64)
        rc = lib().oracle_decode_i64(DT[dtype], _ptr(r), r.size, _ptr(out))
    else:
        out = np.empty(r.size, np.float64)
        rc = lib().oracle_decode_f64(DT[dtype], _ptr(r), r.size, _ptr(out))
    assert rc == 0
    return out.reshape(shape)


def round_to(dtype, x):
    """Round exact float64 values to `dtype` (RNE); returns the raw array (uint16 bits for
    f16/bf16, float32 for f32)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, RAW_NP[dtype])
    assert lib().oracle_round_to(DT[dtype], _ptr(x), x.size, _ptr(out)) == 0
    return out


def _dense_op(op, rows, cols, X, ldx, integer):
    """Dense rows x cols copy of op(X) from a decoded stored array X (flat, leading dim ldx)."""
    out = np.empty(rows * cols, np.int64 if integer else np.float64)
    if rows and cols:
        f = lib().oracle_gather_i64 if integer else lib().oracle_gather_f64
        f(1 if op == "T" else 0, rows, cols, _ptr(X), ldx, _ptr(out))
    return out


def _span(op, rows, cols, ld):
    """Number of stored elements that op(X) (rows x cols) touches."""
    if rows == 0 or cols == 0:
        return 0
    return (cols - 1) * ld + rows if op == "T" else (rows - 1) * ld + cols


def zero_negative(x):
    """The load transform ReLU on decoded values: every element whose sign bit is set becomes
    +0, i.e. max(x, 0) for every non-NaN x ("Flexible Performant GEMM Kernels on GPUs",
    section 4: a transform applies a function such as an activation to every element after it
    is loaded; the ReLU itself is max(0, x), as in "CUTLASS: Fast Linear Algebra in CUDA C++",
    "Fusing Element-wise Operations").  Reading where the pages are silent: -0 -> +0, and a NaN
    is kept unless its sign bit is set."""
    x = np.asarray(x)
    return np.where(np.signbit(x), x.dtype.type(0), x)


# load transforms that convert the stored type to the input type: transform name -> stored type
CONVERT_FROM = {"from_f32": "f32", "from_i8": "i8"}


def convert_to(ab, x):
    """The type-converting load transform on decoded stored values: each value becomes the
    nearest `ab` value, ties to even ("Flexible Performant GEMM Kernels on GPUs", section 4: a
    transform applied to every element after it is loaded may convert its type).  Reading where
    the pages are silent: round to nearest even, as the output conversion; int8 values convert
    exactly to fp16 and bf16."""
    x = np.ascontiguousarray(x, np.float64)
    return decode(ab, round_to(ab, x))


def _operand(ab, transform, raw, span_start, span_len, integer):
    """Decoded stored elements [span_start, span_start + span_len) of an operand, converted to
    the input type `ab` when its transform is a type conversion."""
    st = CONVERT_FROM.get(transform)
    if st is None:
        return decode(ab, raw[span_start: span_start + span_len])
    vals = decode(st, _raw(st, raw)[span_start: span_start + span_len]).astype(np.float64)
    return convert_to(ab, vals)


def gemm(M, N, K, op_a, op_b, A, lda, B, ldb, ab, C=None, ldc=None, cd=None, bias=None,
         bias_dt=None, alpha=1.0, beta=0.0, relu=False, order="tiled", rows=None, threads=None,
         transform_a="none", transform_b="none", transform_c="none", kind_a="dense",
         kind_b="dense"):
    """Exact (unrounded) result rows x N of act(alpha*tA(op(A)) tB(op(B)) + beta*tC(C) + bias).

    ab: input dtype; cd: C/D dtype; bias_dt: bias dtype (default f32, i32 for i8 inputs).
    rows: optional (r0, r1) to compute only those output rows.  transform_*: "none" or "relu"
    (zero_negative) on the loaded op(A), op(B) and C; for A and B also "from_f32" / "from_i8"
    (the operand is stored as fp32 / int8, its array and leading dimension in that type, and
    every element is converted to `ab` as it is loaded: convert_to).  kind_*: "dense" or "diagonal" (the
    operand is the square diagonal matrix of the vector given, its op and ld ignored:
    "Flexible Performant GEMM Kernels on GPUs", section 5.2).  Returns float64, or int64 when
    the inputs are int8."""
    integer = is_int(ab)
    r0, r1 = (0, M) if rows is None else rows
    mr = r1 - r0
    threads = threads or os.cpu_count() or 1
    Ar = _raw(CONVERT_FROM.get(transform_a, ab), A)
    Br = _raw(CONVERT_FROM.get(transform_b, ab), B)
    if kind_a == "diagonal":
        # rows r0..r1 of diag(a): element (i, k) = a[r0 + i] if k == r0 + i else 0
        assert K == M
        Aop = np.zeros((mr, K), np.int64 if integer else np.float64)
        Aop[np.arange(mr), r0 + np.arange(mr)] = _operand(ab, transform_a, Ar, r0, mr, integer)
        Aop = Aop.reshape(-1)
    else:
        # decode only the stored rows that op(A)[r0:r1] touches
        if op_a == "N":
            Asub = _operand(ab, transform_a, Ar, r0 * lda, _span("N", mr, K, lda), integer)
        else:
            Asub = _operand(ab, transform_a, Ar, r0, _span("T", mr, K, lda), integer)
        Aop = _dense_op(op_a, mr, K, Asub, lda, integer)
    if kind_b == "diagonal":
        assert K == N
        Bop = np.diag(_operand(ab, transform_b, Br, 0, N, integer)).astype(
            np.int64 if integer else np.float64).reshape(-1)
    else:
        Bop = _dense_op(op_b, K, N, _operand(ab, transform_b, Br, 0, _span(op_b, K, N, ldb), integer),
                        ldb, integer)
    if transform_a == "relu":
        Aop = np.ascontiguousarray(zero_negative(Aop))
    if transform_b == "relu":
        Bop = np.ascontiguousarray(zero_negative(Bop))
    acc = np.zeros(mr * N, np.int64 if integer else np.float64)
    if mr and N and K:
        f = lib().oracle_matmul_i64 if integer else lib().oracle_matmul_f64
        assert f(ORDERS[order], mr, N, K, _ptr(Aop), _ptr(Bop), _ptr(acc), 0, mr, threads) == 0
    Cd = None
    if beta != 0:
        Cr = _raw(cd, C)
        Cd = np.empty(mr * N, np.int64 if integer else np.float64)
        for i in range(mr):
            Cd[i * N:(i + 1) * N] = decode(cd, Cr[(r0 + i) * ldc:(r0 + i) * ldc + N])
        if transform_c == "relu":
            Cd = np.ascontiguousarray(zero_negative(Cd))
    bd = None
    if bias is not None:
        bias_dt = bias_dt or ("i32" if integer else "f32")
        bd = decode(bias_dt, _raw(bias_dt, bias)[:N])
    out = np.empty(mr * N, np.int64 if integer else np.float64)
    if integer:
        assert float(alpha) == int(alpha) and float(beta) == int(beta)
        lib().oracle_epilogue_i64(mr, N, _ptr(acc), int(alpha), _ptr(Cd), int(beta), _ptr(bd),
                                  1 if relu else 0, _ptr(out))
    else:
        lib().oracle_epilogue_f64(mr, N, _ptr(acc), float(alpha), _ptr(Cd), float(beta),
                                  _ptr(bd), 1 if relu else 0, _ptr(out))
    return out.reshape(mr, N)


PART = {"cf16": "f16", "df16": "f16", "cf32": "f32", "df32": "f32"}


def gemm_pair(M, N, K, op_a, op_b, A, lda, B, ldb, ab, C=None, ldc=None, cd=None, alpha=1.0,
              beta=0.0, rows=None, threads=None):
    """Exact result (rows x N x 2: first and second parts) of D = alpha*op(A)op(B) + beta*C on
    complex ("cf16") or dual ("df16") numbers stored interleaved (two parts per number, ld in
    numbers), with real alpha and beta.  "Flexible Performant GEMM Kernels on GPUs", section 5.4:
    the product of a tile is four real products of the parts, combined as
      complex: re = Are*Bre - Aim*Bim,  im = Are*Bim + Aim*Bre   (i^2 = -1)
      dual:    re = Are*Bre,            im = Are*Bim + Aim*Bre   (eps^2 = 0)
    each real product being the plain definition above (fp64, ascending k)."""
    part = PART[ab]
    Ar = _raw(part, A).reshape(-1, 2)
    Br = _raw(part, B).reshape(-1, 2)
    prod = {}
    for (x, y) in [(0, 0), (1, 1), (0, 1), (1, 0)]:
        if ab.startswith("d") and (x, y) == (1, 1):
            continue
        prod[(x, y)] = gemm(M, N, K, op_a, op_b, np.ascontiguousarray(Ar[:, x]), lda,
                            np.ascontiguousarray(Br[:, y]), ldb, part, rows=rows, threads=threads)
    re = prod[(0, 0)] - prod[(1, 1)] if ab.startswith("c") else prod[(0, 0)]
    im = prod[(0, 1)] + prod[(1, 0)]
    out = np.stack([re, im], axis=-1) * float(alpha)
    if beta != 0:
        r0, r1 = (0, M) if rows is None else rows
        Cr = _raw(PART[cd], C).reshape(-1, 2)
        Cd = np.empty((r1 - r0, N, 2))
        for i in range(r1 - r0):
            Cd[i] = decode(PART[cd], Cr[(r0 + i) * ldc:(r0 + i) * ldc + N])
        out = out + float(beta) * Cd
    return out


def gemm_batched(M, N, K, op_a, op_b, A, lda, B, ldb, ab, C=None, ldc=None, cd=None, bias=None,
                 bias_dt=None, alpha=1.0, beta=0.0, relu=False, batch=1, stride_a=0, stride_b=0,
                 stride_c=0, stride_bias=0, threads=None, transform_a="none", transform_b="none",
                 transform_c="none", kind_a="dense", kind_b="dense", batch2=1, stride2_a=0,
                 stride2_b=0, stride2_c=0, stride2_bias=0):
    """Exact results of a strided batch: product b uses the stored operands starting b * stride
    elements after those of product 0 (C and D share stride_c; a zero stride shares the
    operand).  With batch2 > 1 the batch has two modes: product (b1, b2), b1 < batch,
    b2 < batch2, starts b1 * stride + b2 * stride2 elements after product (0, 0), and the
    result is batch x batch2 x M x N (a zero stride in one mode broadcasts the operand along
    it).  The logical-index-to-offset mapping of a batched operand is the layout idea of
    "Flexible Performant GEMM Kernels on GPUs", section 4 (tensor contractions computed as GEMMs
    whose loads reorganise indices); each product is the plain definition above."""
    if batch2 != 1:
        out = [gemm_batched(M, N, K, op_a, op_b, _raw_store(transform_a, ab, A)[b2 * stride2_a:], lda,
                            _raw_store(transform_b, ab, B)[b2 * stride2_b:], ldb, ab,
                            C=_raw(cd, C)[b2 * stride2_c:] if (C is not None and beta != 0) else None,
                            ldc=ldc, cd=cd,
                            bias=_raw(bias_dt or ("i32" if is_int(ab) else "f32"), bias)[b2 * stride2_bias:]
                            if bias is not None else None, bias_dt=bias_dt, alpha=alpha, beta=beta,
                            relu=relu, batch=batch, stride_a=stride_a, stride_b=stride_b,
                            stride_c=stride_c, stride_bias=stride_bias, threads=threads,
                            transform_a=transform_a, transform_b=transform_b, transform_c=transform_c,
                            kind_a=kind_a, kind_b=kind_b)
               for b2 in range(batch2)]
        return np.stack(out, axis=1) if batch2 > 0 else np.empty(
            (batch, 0, M, N), np.int64 if is_int(ab) else np.float64)
    integer = is_int(ab)
    out = np.empty((batch, M, N), np.int64 if integer else np.float64)
    Ar = _raw(CONVERT_FROM.get(transform_a, ab), A)
    Br = _raw(CONVERT_FROM.get(transform_b, ab), B)
    Cr = _raw(cd, C) if (C is not None and beta != 0) else None
    bias_dt = bias_dt or ("i32" if integer else "f32")
    br = _raw(bias_dt, bias) if bias is not None else None
    for b in range(batch):
        out[b] = gemm(M, N, K, op_a, op_b, Ar[b * stride_a:], lda, Br[b * stride_b:], ldb, ab,
                      C=Cr[b * stride_c:] if Cr is not None else None, ldc=ldc, cd=cd,
                      bias=br[b * stride_bias:] if br is not None else None, bias_dt=bias_dt,
                      alpha=alpha, beta=beta, relu=relu, threads=threads,
                      transform_a=transform_a, transform_b=transform_b, transform_c=transform_c,
                      kind_a=kind_a, kind_b=kind_b)
    return out


def points(ii, jj, K, op_a, op_b, A, lda, B, ldb, ab, C=None, ldc=0, cd="f32", bias=None,
           bias_dt=None, alpha=1.0, beta=0.0, relu=False):
    """Exact result at the output points (ii[p], jj[p]), straight from the raw stored operands
    (naive ascending-k sum per point)."""
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    integer = is_int(ab)
    Ar, Br = _raw(ab, A), _raw(ab, B)
    Cr = _raw(cd, C) if (C is not None and beta != 0) else None
    bias_dt = bias_dt or ("i32" if integer else "f32")
    br = _raw(bias_dt, bias) if bias is not None else None
    out = np.empty(ii.size, np.int64 if integer else np.float64)
    f = lib().oracle_points_i64 if integer else lib().oracle_points_f64
    conv = int if integer else float
    f(ii.size, _ptr(ii), _ptr(jj), K, 1 if op_a == "T" else 0, 1 if op_b == "T" else 0, DT[ab],
      _ptr(Ar), lda, _ptr(Br), ldb, DT[cd], _ptr(Cr), ldc, DT[bias_dt], _ptr(br), conv(alpha),
      conv(beta), 1 if relu else 0, _ptr(out))
    return out


def max_abs_op(dtype, X, op, rows, cols, ld, transform="none"):
    """max |op(X)| over the decoded elements op(X) uses (the tolerance's normaliser); with a
    type-converting transform, over the converted values."""
    if rows == 0 or cols == 0:
        return 0.0
    st = CONVERT_FROM.get(transform)
    if st is None:
        d = decode(dtype, _raw(dtype, X)[: _span(op, rows, cols, ld)])
    else:
        d = convert_to(dtype, decode(st, _raw(st, X)[: _span(op, rows, cols, ld)]))
    if op == "N":
        idx_ok = (np.arange(d.size) % ld) < cols
    else:
        idx_ok = (np.arange(d.size) % ld) < rows
    return float(np.max(np.abs(d[idx_ok]))) if idx_ok.any() else 0.0
