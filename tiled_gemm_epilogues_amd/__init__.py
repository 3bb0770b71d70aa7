"""Python binding of libtge.so, the MI355X tiled GEMM with a fused register epilogue:

    D = act(alpha * op(A) * op(B) + beta * C + bias[j])

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C
ABI (include/gemm.h).  The low-level functions carry the C names (gemm_plan_create, gemm_run,
gemm_run_noalloc, gemm_plan_create_batched, gemm_plan_create_desc, gemm_plan_destroy,
gemm_status_string, gemm_plan_describe); `Plan` wraps them for torch tensors, whose device
memory and streams are the only things taken from PyTorch.

The library is loaded on first use, not at import, so that the build module of this package
can run on a checkout that has no library yet.  There is no fallback: the first call fails with
an ImportError when the HIP library has not been built (python -m
tiled_gemm_epilogues_amd.build, or __graft_entry__.build()).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtge.so")

OP = {"N": 0, "T": 1}
DTYPE = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "cf16": 5, "cf32": 6, "df16": 7,
         "df32": 8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4, "cf16": 4, "cf32": 8, "df16": 4,
              "df32": 8}
EPILOGUE = {"none": 0, "relu": 1, "bias": 2, "bias_relu": 3}
TRANSFORM = {"none": 0, "relu": 1, "from_f32": 2, "from_i8": 3}
# stored element type of an operand whose load transform converts it to the input type
STORED_BY_TRANSFORM = {"from_f32": "f32", "from_i8": "i8"}
KIND = {"dense": 0, "diagonal": 1}
ALGO = {"auto": 0, "fast": 1, "staged": 2, "general": 3, "skinny": 4, "split": 5, "nosplit": 6,
        "kmajor": 7}
(STATUS_SUCCESS, STATUS_INVALID_VALUE, STATUS_NOT_SUPPORTED, STATUS_HIP_ERROR,
 STATUS_ALLOC_FAILED, STATUS_SCRATCH_LIMIT) = range(6)
# device scratch of gemm_run_noalloc (GEMM_NOALLOC_SCRATCH_BYTES in include/gemm.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("gemm_plan_create", "gemm_plan_create_batched", "gemm_plan_create_desc", "gemm_run",
            "gemm_run_noalloc", "gemm_plan_destroy", "gemm_status_string", "gemm_plan_describe")

_i64, _vp, _ci, _f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float


class GemmDesc(ctypes.Structure):
    """gemm_desc_t of include/gemm.h (field order and types as declared there)."""
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("op_a", _ci), ("op_b", _ci),
                ("lda", _i64), ("ldb", _i64), ("ldc", _i64), ("ab_type", _ci), ("cd_type", _ci),
                ("epilogue", _ci), ("batch", _i64), ("stride_a", _i64), ("stride_b", _i64),
                ("stride_c", _i64), ("stride_bias", _i64), ("transform_a", _ci),
                ("transform_b", _ci), ("transform_c", _ci), ("kind_a", _ci), ("kind_b", _ci),
                ("algo", _ci), ("tile", _ci), ("batch2", _i64), ("stride2_a", _i64),
                ("stride2_b", _i64), ("stride2_c", _i64), ("stride2_bias", _i64)]


_lib = None


def lib():
    """The loaded libtge.so (loaded on the first call)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -m tiled_gemm_epilogues_amd.build)")
    # torch ships its own HIP runtime (same soname as ROCm's).  Load it first so that libtge.so
    # binds to that one runtime: device memory and streams come from torch, and a second runtime
    # in the process would own neither.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    L.gemm_plan_create.argtypes = [ctypes.POINTER(_vp), _i64, _i64, _i64, _ci, _ci, _i64, _i64,
                                   _i64, _ci, _ci, _ci]
    L.gemm_plan_create.restype = _ci
    L.gemm_plan_create_batched.argtypes = [ctypes.POINTER(_vp), _i64, _i64, _i64, _ci, _ci, _i64,
                                           _i64, _i64, _ci, _ci, _ci, _i64, _i64, _i64, _i64, _i64]
    L.gemm_plan_create_batched.restype = _ci
    L.gemm_plan_create_desc.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(GemmDesc)]
    L.gemm_plan_create_desc.restype = _ci
    L.gemm_run.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _vp]
    L.gemm_run.restype = _ci
    L.gemm_run_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _vp]
    L.gemm_run_noalloc.restype = _ci
    L.gemm_plan_destroy.argtypes = [_vp]
    L.gemm_plan_destroy.restype = _ci
    L.gemm_status_string.argtypes = [_ci]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_plan_describe.argtypes = [_vp, ctypes.c_char_p, ctypes.c_size_t]
    L.gemm_plan_describe.restype = _ci
    _lib = L
    return _lib


class GemmError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {gemm_status_string(status)}")


def gemm_status_string(status):
    return lib().gemm_status_string(int(status)).decode()


def gemm_plan_create(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue):
    """Returns (status, handle); enum arguments may be names ('N', 'f16', 'bias_relu') or ints."""
    h = _vp()
    st = lib().gemm_plan_create(ctypes.byref(h), M, N, K, _enum(OP, op_a), _enum(OP, op_b), lda,
                                ldb, ldc, _enum(DTYPE, ab_type), _enum(DTYPE, cd_type),
                                _enum(EPILOGUE, epilogue))
    return st, h.value


def gemm_plan_create_batched(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue, batch,
                             stride_a, stride_b, stride_c, stride_bias):
    """Returns (status, handle) of a strided-batched plan (strides in elements)."""
    h = _vp()
    st = lib().gemm_plan_create_batched(ctypes.byref(h), M, N, K, _enum(OP, op_a), _enum(OP, op_b),
                                        lda, ldb, ldc, _enum(DTYPE, ab_type),
                                        _enum(DTYPE, cd_type), _enum(EPILOGUE, epilogue), batch,
                                        stride_a, stride_b, stride_c, stride_bias)
    return st, h.value


def gemm_plan_create_desc(M, N, K, op_a, op_b, lda, ldb, ldc, ab_type, cd_type, epilogue,
                          batch=1, stride_a=0, stride_b=0, stride_c=0, stride_bias=0,
                          transform_a="none", transform_b="none", transform_c="none",
                          kind_a="dense", kind_b="dense", algo="auto", tile=0, batch2=1,
                          stride2_a=0, stride2_b=0, stride2_c=0, stride2_bias=0):
    """Returns (status, handle) of a plan built from a full gemm_desc_t."""
    d = GemmDesc(M, N, K, _enum(OP, op_a), _enum(OP, op_b), lda, ldb, ldc, _enum(DTYPE, ab_type),
                 _enum(DTYPE, cd_type), _enum(EPILOGUE, epilogue), batch, stride_a, stride_b,
                 stride_c, stride_bias, _enum(TRANSFORM, transform_a),
                 _enum(TRANSFORM, transform_b), _enum(TRANSFORM, transform_c),
                 _enum(KIND, kind_a), _enum(KIND, kind_b), _enum(ALGO, algo), int(tile),
                 batch2, stride2_a, stride2_b, stride2_c, stride2_bias)
    h = _vp()
    st = lib().gemm_plan_create_desc(ctypes.byref(h), ctypes.byref(d))
    return st, h.value


def gemm_run(plan, A, B, C, D, bias, alpha, beta, stream):
    """Raw pointers (ints or None) and a hipStream_t handle (int or None)."""
    return lib().gemm_run(plan, A, B, C, D, bias, alpha, beta, stream)


def gemm_run_noalloc(plan, A, B, C, D, bias, alpha, beta, stream):
    """gemm_run that allocates nothing (the library's per-device scratch); raw pointers."""
    return lib().gemm_run_noalloc(plan, A, B, C, D, bias, alpha, beta, stream)


def gemm_plan_destroy(plan):
    return lib().gemm_plan_destroy(plan)


def gemm_plan_describe(plan):
    buf = ctypes.create_string_buffer(256)
    st = lib().gemm_plan_describe(plan, buf, 256)
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


def _span(rows, cols, ld):
    """Elements from the first to one past the last element of a rows x cols row-major view."""
    return 0 if rows <= 0 or cols <= 0 else (rows - 1) * ld + cols


class Plan:
    """A plan for one problem description (see include/gemm.h for the storage rules).  With
    batch != 1 it is a strided-batched plan (strides in elements); a transform, a diagonal
    operand, or an explicit algorithm or tile builds it from a full description
    (gemm_plan_create_desc).  algo: "auto" (the plan's own choice), "fast", "staged",
    "general", "skinny", "split", "nosplit"; tile: 0 (auto), 256, 128 or 64."""

    def __init__(self, M, N, K, op_a="N", op_b="N", lda=None, ldb=None, ldc=None, ab="f16",
                 cd="f16", epilogue="none", batch=1, stride_a=0, stride_b=0, stride_c=0,
                 stride_bias=0, transform_a="none", transform_b="none", transform_c="none",
                 kind_a="dense", kind_b="dense", algo="auto", tile=0, batch2=1, stride2_a=0,
                 stride2_b=0, stride2_c=0, stride2_bias=0):
        self._h = None
        self.M, self.N, self.K = M, N, K
        self.op_a, self.op_b, self.ab, self.cd, self.epilogue = op_a, op_b, ab, cd, epilogue
        self.lda = lda if lda is not None else max(1, K if op_a == "N" else M)
        self.ldb = ldb if ldb is not None else max(1, N if op_b == "N" else K)
        self.ldc = ldc if ldc is not None else max(1, N)
        self.batch = batch
        self.stride_a, self.stride_b, self.stride_c = stride_a, stride_b, stride_c
        self.stride_bias = stride_bias
        self.kind_a, self.kind_b = kind_a, kind_b
        self.transform_a, self.transform_b = transform_a, transform_b
        self.batch2 = batch2
        self.stride2 = {"A": stride2_a, "B": stride2_b, "C": stride2_c, "D": stride2_c,
                        "bias": stride2_bias}
        xf = (transform_a, transform_b, transform_c)
        if (any(_enum(TRANSFORM, t) for t in xf) or _enum(KIND, kind_a) or _enum(KIND, kind_b)
                or _enum(ALGO, algo) or tile or batch2 != 1):
            st, h = gemm_plan_create_desc(M, N, K, op_a, op_b, self.lda, self.ldb, self.ldc, ab, cd,
                                          epilogue, batch, stride_a, stride_b, stride_c,
                                          stride_bias, *xf, kind_a=kind_a, kind_b=kind_b,
                                          algo=algo, tile=tile, batch2=batch2, stride2_a=stride2_a,
                                          stride2_b=stride2_b, stride2_c=stride2_c,
                                          stride2_bias=stride2_bias)
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

    # elements (of each operand's own type) that the plan's runs may touch, from the pointer on
    def spans(self):
        """{operand: (elements spanned, stored row length)}; row length None where a tensor's
        last dimension is not checked (diagonal vectors, bias)."""
        M, N, K, nb = self.M, self.N, self.K, max(self.batch, 1)
        more = lambda stride: (nb - 1) * stride if self.batch > 1 else 0
        if self.kind_a == "diagonal":
            a = (K + more(self.stride_a) if K else 0, None)
        elif self.op_a == "N":
            a = (_span(M, K, self.lda) + more(self.stride_a) if M and K else 0, self.lda)
        else:
            a = (_span(K, M, self.lda) + more(self.stride_a) if M and K else 0, self.lda)
        if self.kind_b == "diagonal":
            b = (K + more(self.stride_b) if K else 0, None)
        elif self.op_b == "N":
            b = (_span(K, N, self.ldb) + more(self.stride_b) if N and K else 0, self.ldb)
        else:
            b = (_span(N, K, self.ldb) + more(self.stride_b) if N and K else 0, self.ldb)
        cd = (_span(M, N, self.ldc) + more(self.stride_c) if M and N else 0, self.ldc)
        bias = (N + more(self.stride_bias) if N else 0, None)
        out = {"A": a, "B": b, "C": cd, "D": cd, "bias": bias}
        if self.batch2 > 1:   # the second batch mode moves every operand by its stride2 too
            out = {k: (n + (self.batch2 - 1) * self.stride2[k] if n else 0, ld)
                   for k, (n, ld) in out.items()}
        return out

    def dtype_of(self, what):
        """Stored element type of operand `what` ("A", "B", "C", "D" or "bias")."""
        if what == "A":
            return STORED_BY_TRANSFORM.get(self.transform_a, self.ab)
        if what == "B":
            return STORED_BY_TRANSFORM.get(self.transform_b, self.ab)
        if what in ("C", "D"):
            return self.cd
        return "i32" if self.ab == "i8" else "f32"

    def check(self, what, t):
        """Checks tensor t against the plan's storage for operand `what`: its dtype, that it is
        contiguous, that a 2-D or higher tensor's rows are the matrix's leading dimension long,
        and that it holds every element the plan's runs may touch.  Raises TypeError or
        ValueError; the device is checked by run()."""
        dtype = self.dtype_of(what)
        need, row_len = self.spans()[what]
        want = _torch_dtype(dtype)
        if want is not None and t.dtype != want:
            raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous (the plan's leading dimension and "
                             "strides describe its layout)")
        if row_len is not None and want is not None and t.dim() >= 2 and t.shape[-1] != row_len:
            raise ValueError(f"{what}: rows of {t.shape[-1]} elements, the plan's leading "
                             f"dimension is {row_len}")
        have = t.numel() * t.element_size()
        need_bytes = need * ELEM_BYTES[dtype]
        if have < need_bytes:
            raise ValueError(f"{what} holds {have} bytes, the plan spans {need_bytes}")

    def _ptr(self, t, what):
        """Device pointer of tensor t after checking it against the plan; raw ints pass as is."""
        if t is None or isinstance(t, int):
            return t
        import torch
        if not t.is_cuda:
            raise ValueError(f"{what} must be a device tensor")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{what} is on {t.device}, the current device is "
                             f"cuda:{torch.cuda.current_device()}")
        self.check(what, t)
        return t.data_ptr()

    def _args(self, A, B, C, D, bias, beta):
        raw = lambda t: t if t is None or isinstance(t, int) else t.data_ptr()
        has_bias = self.epilogue in ("bias", "bias_relu")
        # C is read only when beta != 0; a bias only when the epilogue has one
        return (self._ptr(A, "A"), self._ptr(B, "B"),
                self._ptr(C, "C") if beta != 0 else raw(C), self._ptr(D, "D"),
                self._ptr(bias, "bias") if has_bias else raw(bias))

    @staticmethod
    def _stream(stream):
        import torch
        if stream is None:
            return torch.cuda.current_stream().cuda_stream
        if isinstance(stream, int):
            return stream
        return stream.cuda_stream

    def run(self, A, B, C, D, bias=None, alpha=1.0, beta=0.0, stream=None):
        """Enqueue on `stream` (a torch.cuda.Stream, a raw handle, or None for torch's current
        stream).  Tensors must be contiguous device tensors of the plan's types on the current
        device, each holding at least the elements the plan's layout spans (a 2-D or higher
        tensor's last dimension must equal that matrix's leading dimension); raw integer
        pointers are passed unchecked.  Raises ValueError / TypeError before anything is
        enqueued when a tensor does not fit the plan."""
        args = self._args(A, B, C, D, bias, beta)
        st = gemm_run(self._h, *args, float(alpha), float(beta), self._stream(stream))
        if st != STATUS_SUCCESS:
            raise GemmError(st, "gemm_run")

    def run_noalloc(self, A, B, C, D, bias=None, alpha=1.0, beta=0.0, stream=None):
        """run() through gemm_run_noalloc: nothing is allocated; a run that needs more scratch
        than the library holds raises GemmError (GEMM_STATUS_SCRATCH_LIMIT) before enqueueing."""
        args = self._args(A, B, C, D, bias, beta)
        st = gemm_run_noalloc(self._h, *args, float(alpha), float(beta), self._stream(stream))
        if st != STATUS_SUCCESS:
            raise GemmError(st, "gemm_run_noalloc")

    def close(self):
        if getattr(self, "_h", None):
            gemm_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
