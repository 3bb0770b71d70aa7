"""Python binding of libtge.so, the MI355X tiled GEMM with a fused register epilogue:

    D = act(alpha * op(A) * op(B) + beta * C + bias[j])

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C
ABI (include/gemm.h).  The low-level functions carry the C names (gemm_plan_create, gemm_run,
gemm_plan_create_batched, gemm_plan_create_desc, gemm_plan_destroy, gemm_status_string,
gemm_plan_describe); `Plan` wraps them for torch tensors, whose device memory and streams are the
only things taken from PyTorch.

There is no fallback: importing this package fails if the HIP library has not been built
(python -m tiled_gemm_epilogues_amd.build, or __graft_entry__.build()).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtge.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python -m tiled_gemm_epilogues_amd.build)")

# torch ships its own HIP runtime (same soname as ROCm's).  Load it first so that libtge.so binds
# to that one runtime: device memory and streams come from torch, and a second runtime in the
# process would own neither.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

OP = {"N": 0, "T": 1}
DTYPE = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "cf16": 5, "cf32": 6, "df16": 7,
         "df32": 8}
EPILOGUE = {"none": 0, "relu": 1, "bias": 2, "bias_relu": 3}
TRANSFORM = {"none": 0, "relu": 1}
KIND = {"dense": 0, "diagonal": 1}
STATUS_SUCCESS, STATUS_INVALID_VALUE, STATUS_NOT_SUPPORTED, STATUS_HIP_ERROR, STATUS_ALLOC_FAILED = range(5)

_i64, _vp, _ci, _f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_lib.gemm_plan_create.argtypes = [ctypes.POINTER(_vp), _i64, _i64, _i64, _ci, _ci, _i64, _i64, _i64,
                                  _ci, _ci, _ci]
_lib.gemm_plan_create.restype = _ci
_lib.gemm_plan_create_batched.argtypes = [ctypes.POINTER(_vp), _i64, _i64, _i64, _ci, _ci, _i64, _i64,
                                          _i64, _ci, _ci, _ci, _i64, _i64, _i64, _i64, _i64]
_lib.gemm_plan_create_batched.restype = _ci


class GemmDesc(ctypes.Structure):
    """gemm_desc_t of include/gemm.h (field order and types as declared there)."""
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("op_a", _ci), ("op_b", _ci),
                ("lda", _i64), ("ldb", _i64), ("ldc", _i64), ("ab_type", _ci), ("cd_type", _ci),
                ("epilogue", _ci), ("batch", _i64), ("stride_a", _i64), ("stride_b", _i64),
                ("stride_c", _i64), ("stride_bias", _i64), ("transform_a", _ci),
                ("transform_b", _ci), ("transform_c", _ci), ("kind_a", _ci), ("kind_b", _ci)]


_lib.gemm_plan_create_desc.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(GemmDesc)]
_lib.gemm_plan_create_desc.restype = _ci
_lib.gemm_run.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _vp]
_lib.gemm_run.restype = _ci
_lib.gemm_plan_destroy.argtypes = [_vp]
_lib.gemm_plan_destroy.restype = _ci
_lib.gemm_status_string.argtypes = [_ci]
_lib.gemm_status_string.restype = ctypes.c_char_p
_lib.gemm_plan_describe.argtypes = [_vp, ctypes.c_char_p, ctypes.c_size_t]
_lib.gemm_plan_describe.restype = _ci

EXPORTED = ("gemm_plan_create", "gemm_plan_create_batched", "gemm_plan_create_desc", "gemm_run",
            "gemm_plan_destroy", "gemm_status_string", "gemm_plan_describe")


class GemmError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {gemm_status_string(status)}")


def gemm_status_string(status):
    return _lib.gemm_status_string(int(status)).decode()


def gemm_plan_create(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue):
    """Returns (status, handle); enum arguments may be names ('N', 'f16', 'bias_relu') or ints."""
    h = _vp()
    st = _lib.gemm_plan_create(ctypes.byref(h), M, N, K, _enum(OP, op_a), _enum(OP, op_b), lda, ldb,
                               ldc, _enum(DTYPE, ab_type), _enum(DTYPE, cd_type),
                               _enum(EPILOGUE, epilogue))
    return st, h.value


def gemm_plan_create_batched(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue, batch,
                             stride_a, stride_b, stride_c, stride_bias):
    """Returns (status, handle) of a strided-batched plan (strides in elements)."""
    h = _vp()
    st = _lib.gemm_plan_create_batched(ctypes.byref(h), M, N, K, _enum(OP, op_a), _enum(OP, op_b),
                                       lda, ldb, ldc, _enum(DTYPE, ab_type), _enum(DTYPE, cd_type),
                                       _enum(EPILOGUE, epilogue), batch, stride_a, stride_b,
                                       stride_c, stride_bias)
    return st, h.value


def gemm_plan_create_desc(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue,
                          batch=1, stride_a=0, stride_b=0, stride_c=0, stride_bias=0,
                          transform_a="none", transform_b="none", transform_c="none",
                          kind_a="dense", kind_b="dense"):
    """Returns (status, handle) of a plan built from a full gemm_desc_t."""
    d = GemmDesc(M, N, K, _enum(OP, op_a), _enum(OP, op_b), lda, ldb, ldc, _enum(DTYPE, ab_type),
                 _enum(DTYPE, cd_type), _enum(EPILOGUE, epilogue), batch, stride_a, stride_b,
                 stride_c, stride_bias, _enum(TRANSFORM, transform_a),
                 _enum(TRANSFORM, transform_b), _enum(TRANSFORM, transform_c),
                 _enum(KIND, kind_a), _enum(KIND, kind_b))
    h = _vp()
    st = _lib.gemm_plan_create_desc(ctypes.byref(h), ctypes.byref(d))
    return st, h.value


def gemm_run(plan, A, B, C, D, bias, alpha, beta, stream):
    """Raw pointers (ints or None) and a hipStream_t handle (int or None)."""
    return _lib.gemm_run(plan, A, B, C, D, bias, alpha, beta, stream)


def gemm_plan_destroy(plan):
    return _lib.gemm_plan_destroy(plan)


def gemm_plan_describe(plan):
    buf = ctypes.create_string_buffer(256)
    st = _lib.gemm_plan_describe(plan, buf, 256)
    return st, buf.value.decode()


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


# ---- torch-facing wrapper ---------------------------------------------------------------------

def _torch_dtype(name):
    """torch dtype of a real element type; None for the complex and dual types, whose storage
    (interleaved parts) is passed as is."""
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
            "i32": torch.int32}.get(name)


def _ptr(t, want, what):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if want is not None and _torch_dtype(want) is not None and t.dtype != _torch_dtype(want):
        raise TypeError(f"{what} must be {want}, got {t.dtype}")
    return t.data_ptr()


class Plan:
    """A plan for one problem description (see include/gemm.h for the storage rules).  With
    batch != 1 it is a strided-batched plan (gemm_plan_create_batched; strides in elements);
    with a transform or a diagonal operand it is built from a full description
    (gemm_plan_create_desc)."""

    def __init__(self, M, N, K, op_a="N", op_b="N", lda=None, ldb=None, ldc=None, ab="f16",
                 cd="f16", epilogue="none", batch=1, stride_a=0, stride_b=0, stride_c=0,
                 stride_bias=0, transform_a="none", transform_b="none", transform_c="none",
                 kind_a="dense", kind_b="dense"):
        self.M, self.N, self.K = M, N, K
        self.op_a, self.op_b, self.ab, self.cd, self.epilogue = op_a, op_b, ab, cd, epilogue
        self.lda = lda if lda is not None else max(1, K if op_a == "N" else M)
        self.ldb = ldb if ldb is not None else max(1, N if op_b == "N" else K)
        self.ldc = ldc if ldc is not None else max(1, N)
        self.batch = batch
        xf = (transform_a, transform_b, transform_c)
        if any(_enum(TRANSFORM, t) for t in xf) or _enum(KIND, kind_a) or _enum(KIND, kind_b):
            st, h = gemm_plan_create_desc(M, N, K, op_a, op_b, self.lda, self.ldb, self.ldc, ab, cd,
                                          epilogue, batch, stride_a, stride_b, stride_c,
                                          stride_bias, *xf, kind_a=kind_a, kind_b=kind_b)
        elif batch == 1 and not (stride_a or stride_b or stride_c or stride_bias):
            st, h = gemm_plan_create(M, N, K, op_a, op_b, self.lda, self.ldb, self.ldc, ab, cd,
                                     epilogue)
        else:
            st, h = gemm_plan_create_batched(M, N, K, op_a, op_b, self.lda, self.ldb, self.ldc, ab,
                                             cd, epilogue, batch, stride_a, stride_b, stride_c,
                                             stride_bias)
        if st != STATUS_SUCCESS:
            raise GemmError(st, "gemm_plan_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def describe(self):
        return gemm_plan_describe(self._h)[1]

    def run(self, A, B, C, D, bias=None, alpha=1.0, beta=0.0, stream=None):
        """Enqueue on `stream` (a torch.cuda.Stream, a raw handle, or None for torch's current
        stream).  Tensors must be device tensors of the plan's types; their storage must follow
        the plan's layouts and leading dimensions."""
        import torch
        if stream is None:
            s = torch.cuda.current_stream().cuda_stream
        elif isinstance(stream, int):
            s = stream
        else:
            s = stream.cuda_stream
        bias_dt = "i32" if self.ab == "i8" else "f32"
        st = gemm_run(self._h, _ptr(A, self.ab, "A"), _ptr(B, self.ab, "B"), _ptr(C, self.cd, "C"),
                      _ptr(D, self.cd, "D"), _ptr(bias, bias_dt, "bias"), float(alpha), float(beta),
                      s)
        if st != STATUS_SUCCESS:
            raise GemmError(st, "gemm_run")

    def close(self):
        if getattr(self, "_h", None):
            gemm_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
