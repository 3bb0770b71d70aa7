"""Seeded synthetic inputs for the fused-epilogue GEMM: shared by the tests, the smoke check and
the benchmark.  This module only draws and stores numbers; it holds none of the GEMM's
arithmetic, and neither the HIP path nor the oracle imports it.

Every draw comes from numpy's PCG64 seeded by SeedSequence([*key, operand id]), where key is
(workload id, shape index[, case]) and the operand ids are A=0, B=1, C=2, bias=3.  A logical op(A) (M x K) and op(B) (K x N) are drawn
once per shape and then stored in the requested physical layout, so all four N/T layouts of one
shape hold the same logical problem.  Float values are drawn in float64 and quantised once to
the storage type with round-to-nearest-even; the raw arrays (uint16 bit patterns for f16 and
bf16) are exactly what both the GPU and the oracle receive.  Leading dimensions are tight
unless a padded ld is asked for.
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np

RAW_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "i32": np.int32,
          "cf16": np.uint16, "df16": np.uint16, "cf32": np.float32, "df32": np.float32}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4, "cf16": 4, "df16": 4, "cf32": 8,
              "df32": 8}
# complex / dual types: numbers of two parts of this real type, stored interleaved
PART = {"cf16": "f16", "df16": "f16", "cf32": "f32", "df32": "f32"}
# stored element type of an operand whose load transform converts it to the input type
STORED_BY_TRANSFORM = {"from_f32": "f32", "from_i8": "i8"}


def rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def quantize(dtype, x):
    """float64 values -> raw storage array of `dtype` (RNE)."""
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        import torch  # vectorised float32 -> float16 RNE, far faster than numpy's on big arrays
        return torch.from_numpy(x.astype(np.float32)).to(torch.float16).view(torch.int16) \
            .numpy().view(np.uint16)
    if dtype == "bf16":
        # float64 -> float32 (RNE), then float32 -> bfloat16 by rounding the 32-bit pattern to
        # its upper 16 bits, ties to even (inputs here are finite).
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    if dtype in ("i8", "i32"):
        return x.astype(RAW_NP[dtype])
    raise ValueError(dtype)


def draw(g, dist, n):
    kind = dist[0]
    if kind == "uniform":
        return g.uniform(dist[1], dist[2], n)
    if kind == "normal":
        return g.standard_normal(n) * dist[1]
    if kind == "int":          # integers in [lo, hi] inclusive
        return g.integers(dist[1], dist[2], n, endpoint=True).astype(np.float64)
    raise ValueError(kind)


@dataclass
class Problem:
    M: int
    N: int
    K: int
    op_a: str = "N"
    op_b: str = "N"
    ab: str = "f16"
    cd: str = "f16"
    epi: str = "none"            # none | relu | bias | bias_relu
    alpha: float = 1.0
    beta: float = 0.0
    lda: int = 0                 # 0 -> tight
    ldb: int = 0
    ldc: int = 0
    a_dist: tuple = ("uniform", -1.0, 1.0)
    b_dist: tuple = ("uniform", -1.0, 1.0)
    c_dist: tuple = ("uniform", -1.0, 1.0)
    bias_dist: tuple = ("uniform", -0.5, 0.5)
    key: tuple = (0, 0)
    name: str = ""
    # strided batch: `batch` products, operand x of product b starting stride_x elements after
    # that of product b-1; -1 -> one stored matrix further (tight), 0 -> shared by all products
    # load transforms on op(A), op(B), C: "none" or "relu"
    transform_a: str = "none"
    transform_b: str = "none"
    transform_c: str = "none"
    # "dense" or "diagonal" (the operand is the vector of a square diagonal matrix's elements)
    kind_a: str = "dense"
    kind_b: str = "dense"
    batch: int = 1
    stride_a: int = -1
    stride_b: int = -1
    stride_c: int = -1
    stride_bias: int = -1
    # a second batch mode: product (b1, b2), b2 < batch2, at b1 * stride + b2 * stride2 (the
    # strides of this mode are given explicitly; 0 broadcasts an operand along it)
    batch2: int = 1
    stride2_a: int = 0
    stride2_b: int = 0
    stride2_c: int = 0
    stride2_bias: int = 0

    def __post_init__(self):
        if not self.lda:
            self.lda = max(1, self.K if self.op_a == "N" else self.M)
        if not self.ldb:
            self.ldb = max(1, self.N if self.op_b == "N" else self.K)
        if not self.ldc:
            self.ldc = max(1, self.N)
        if self.kind_a == "diagonal":
            self.lda = 1
        if self.kind_b == "diagonal":
            self.ldb = 1
        if self.batch <= 1:
            self.stride_a = self.stride_b = self.stride_c = self.stride_bias = 0
        else:
            if self.stride_a < 0:
                self.stride_a = self.M if self.kind_a == "diagonal" else self.a_shape()[0] * self.lda
            if self.stride_b < 0:
                self.stride_b = self.N if self.kind_b == "diagonal" else self.b_shape()[0] * self.ldb
            if self.stride_c < 0:
                self.stride_c = self.M * self.ldc
            if self.stride_bias < 0:
                self.stride_bias = self.N if self.has_bias else 0

    @property
    def a_store(self):
        """Element type A is stored in: the input type, or the source type of a converting
        load transform ("from_f32" / "from_i8")."""
        return STORED_BY_TRANSFORM.get(self.transform_a, self.ab)

    @property
    def b_store(self):
        return STORED_BY_TRANSFORM.get(self.transform_b, self.ab)

    @property
    def bias_dt(self):
        return "i32" if self.ab == "i8" else "f32"

    @property
    def has_bias(self):
        return self.epi in ("bias", "bias_relu")

    @property
    def relu(self):
        return self.epi in ("relu", "bias_relu")

    @property
    def flops(self):
        """2 x the real multiply-adds the product needs: M*N*K, or for a diagonal operand only
        the non-zero terms (one per output element; with both diagonal, one per diagonal
        element); x4 for complex numbers (four real products), x3 for dual numbers."""
        nb = max(self.batch, 0) * max(self.batch2, 0)
        if self.ab in ("cf16", "df16"):
            return (4.0 if self.ab == "cf16" else 3.0) * 2.0 * self.M * self.N * self.K * nb
        if self.kind_a == "diagonal" and self.kind_b == "diagonal":
            return 2.0 * min(self.M, self.N) * nb
        if self.kind_a == "diagonal" or self.kind_b == "diagonal":
            return 2.0 * self.M * self.N * nb
        return 2.0 * self.M * self.N * self.K * nb

    def a_shape(self):   # stored 2-D shape (rows, ld)
        return (self.M, self.lda) if self.op_a == "N" else (self.K, self.lda)

    def b_shape(self):
        return (self.K, self.ldb) if self.op_b == "N" else (self.N, self.ldb)

    def algorithmic_bytes(self):
        """Compulsory HBM traffic: op(A), op(B) read once, C if beta != 0, bias, D written once
        (per product; an operand shared by a batch is counted once)."""
        ea, eb, ec = ELEM_BYTES[self.a_store], ELEM_BYTES[self.b_store], ELEM_BYTES[self.cd]
        b1, b2 = max(self.batch, 0), max(self.batch2, 0)
        nb = b1 * b2
        # distinct copies of an operand: a zero stride shares it along that batch mode
        per = lambda s1, s2: (b1 if (b1 <= 1 or s1 != 0) else 1) * (b2 if (b2 <= 1 or s2 != 0) else 1)
        na = self.M if self.kind_a == "diagonal" else self.M * self.K
        nbb = self.N if self.kind_b == "diagonal" else self.K * self.N
        b = na * per(self.stride_a, self.stride2_a) * ea + nbb * per(self.stride_b, self.stride2_b) * eb
        b += self.M * self.N * ec * nb
        if self.beta != 0:
            b += self.M * self.N * ec * nb
        if self.has_bias:
            b += self.N * 4 * per(self.stride_bias, self.stride2_bias)
        return b

    def label(self):
        bt = f":batch{self.batch}" if self.batch != 1 else ""
        bt += f"x{self.batch2}" if self.batch2 != 1 else ""
        return (f"{self.name or 'gemm'}:{self.M}x{self.N}x{self.K}{bt}:{self.op_a}{self.op_b}:"
                f"{self.ab}->{self.cd}:{self.epi}:a{self.alpha:g}b{self.beta:g}")


def _store(logical, op, ld, fill):
    """Store a logical rows x cols matrix as a row-major array with leading dim ld (op N) or its
    transpose (op T).  Padding columns hold `fill`."""
    rows, cols = logical.shape
    if op == "N":
        out = np.full((rows, ld), fill, dtype=logical.dtype)
        out[:, :cols] = logical
    else:
        out = np.full((cols, ld), fill, dtype=logical.dtype)
        out[:, :rows] = logical.T
    return out


def make_inputs(p: Problem, pad_fill=0):
    """Raw stored arrays {A, B, C, bias} (C and bias None when unused) for problem p.  For a
    batch, flat arrays holding product b at b * stride (product b drawn with key (*key, 1000+b);
    a shared operand is product 0's; gaps hold pad_fill).  Complex and dual numbers: both parts
    drawn from the operand's distribution (first parts, then second parts), stored interleaved
    as (rows, ld, 2) raw arrays of the part type."""
    if p.batch != 1 or p.batch2 != 1:
        return _make_batched_inputs(p, pad_fill)
    if p.ab in PART:
        return _make_pair_inputs(p, pad_fill)
    ga, gb, gc, gbias = (rng(*p.key, i) for i in range(4))
    if p.kind_a == "diagonal":
        A = quantize(p.a_store, draw(ga, p.a_dist, p.M))
    else:
        a = quantize(p.a_store, draw(ga, p.a_dist, p.M * p.K)).reshape(p.M, p.K)
        A = _store(a, p.op_a, p.lda, pad_fill)
    if p.kind_b == "diagonal":
        B = quantize(p.b_store, draw(gb, p.b_dist, p.N))
    else:
        b = quantize(p.b_store, draw(gb, p.b_dist, p.K * p.N)).reshape(p.K, p.N)
        B = _store(b, p.op_b, p.ldb, pad_fill)
    C = None
    if p.beta != 0:
        c = quantize(p.cd, draw(gc, p.c_dist, p.M * p.N)).reshape(p.M, p.N)
        C = _store(c, "N", p.ldc, pad_fill)
    bias = quantize(p.bias_dt, draw(gbias, p.bias_dist, p.N)) if p.has_bias else None
    return {"A": A, "B": B, "C": C, "bias": bias}


def _make_pair_inputs(p: Problem, pad_fill=0):
    ga, gb, gc = (rng(*p.key, i) for i in range(3))
    pa, pc = PART[p.ab], PART[p.cd]

    def pair(g, dist, rows, cols, part):
        re = quantize(part, draw(g, dist, rows * cols)).reshape(rows, cols)
        im = quantize(part, draw(g, dist, rows * cols)).reshape(rows, cols)
        return np.stack([re, im], axis=-1)

    def store(logical, op, ld):
        rows, cols = logical.shape[:2]
        if op == "N":
            out = np.full((rows, ld, 2), pad_fill, dtype=logical.dtype)
            out[:, :cols] = logical
        else:
            out = np.full((cols, ld, 2), pad_fill, dtype=logical.dtype)
            out[:, :rows] = logical.transpose(1, 0, 2)
        return out

    A = store(pair(ga, p.a_dist, p.M, p.K, pa), p.op_a, p.lda)
    B = store(pair(gb, p.b_dist, p.K, p.N, pa), p.op_b, p.ldb)
    C = store(pair(gc, p.c_dist, p.M, p.N, pc), "N", p.ldc) if p.beta != 0 else None
    return {"A": A, "B": B, "C": C, "bias": None}


def _make_batched_inputs(p: Problem, pad_fill=0):
    """Flat arrays holding product (b1, b2) at b1 * stride + b2 * stride2 (one batch mode: b2 = 0);
    product (b1, b2) is drawn with key (*key, 1000 + b1 * batch2 + b2), an operand shared along a
    mode (stride 0) is written by the products at index 0 of that mode."""
    out = {"A": None, "B": None, "C": None, "bias": None}
    # strides count numbers: raw (part) elements per number for complex / dual types
    fa, fc = (2 if p.ab in PART else 1), (2 if p.cd in PART else 1)
    strides = {"A": (p.stride_a * fa, p.stride2_a * fa), "B": (p.stride_b * fa, p.stride2_b * fa),
               "C": (p.stride_c * fc, p.stride2_c * fc), "bias": (p.stride_bias, p.stride2_bias)}
    dtypes = {"A": p.a_store, "B": p.b_store, "C": p.cd, "bias": p.bias_dt}
    nb1, nb2 = max(p.batch, 0), max(p.batch2, 0)
    for b1 in range(nb1):
        for b2 in range(nb2):
            one = make_inputs(replace(p, batch=1, batch2=1, key=(*p.key, 1000 + b1 * nb2 + b2)),
                              pad_fill)
            for name, arr in one.items():
                if arr is None:
                    continue
                flat = arr.reshape(-1)
                s1, s2 = strides[name]
                if out[name] is None:
                    n = flat.size + (s1 * (nb1 - 1) if s1 > 0 else 0) + (s2 * (nb2 - 1) if s2 > 0 else 0)
                    out[name] = np.full(n, pad_fill, dtype=RAW_NP[dtypes[name]])
                if (s1 > 0 or b1 == 0) and (s2 > 0 or b2 == 0):
                    o = b1 * s1 + b2 * s2
                    out[name][o: o + flat.size] = flat
    return out


# ---- the workloads ---------------------------------------------------------------------------

def sgemm_256():
    """fp32 256^3, NN, alpha=1, beta=0, A,B ~ U[-1,1], no epilogue."""
    return [Problem(256, 256, 256, "N", "N", "f32", "f32", "none", 1.0, 0.0, key=(1, 0),
                    name="sgemm_256")]


def fp16_8192_bias_relu():
    """fp16 8192^3 NN, A,B ~ N(0,1)/sqrt(K), C absent (beta=0), D = ReLU(acc + bias[N]) -> fp16,
    bias fp32 ~ U[-0.5,0.5]."""
    K = 8192
    s = 1.0 / math.sqrt(K)
    return [Problem(8192, 8192, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(2, 0),
                    name="fp16_8192_bias_relu")]


def fp16_long_k():
    """Few output tiles and a long K (the fast kernel's K split): fp16 2048 x 2048 x 8192 NN,
    A,B ~ N(0,1)/sqrt(K), D = ReLU(acc + bias[N]) -> fp16, bias fp32 ~ U[-0.5,0.5]."""
    K = 8192
    s = 1.0 / math.sqrt(K)
    return [Problem(2048, 2048, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(11, 0),
                    name="fp16_long_k")]


def mid_size():
    """Mid-size products on the 128x128 tiles: fp16 2048^3 NN, A,B ~ N(0,1)/sqrt(K),
    D = ReLU(acc + bias[N]) -> fp16 (bias fp32 ~ U[-0.5,0.5]); and bf16 -> fp32 2048^3 NN with
    alpha = 1.5, beta = -0.5, A,B,C ~ U[-1,1]."""
    K = 2048
    s = 1.0 / math.sqrt(K)
    return [Problem(2048, 2048, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(13, 0), name="mid_size"),
            Problem(2048, 2048, K, "N", "N", "bf16", "f32", "none", 1.5, -0.5, key=(13, 1),
                    name="mid_size")]


def bf16_layout_sweep():
    """bf16 in, fp32 C/D, alpha=1.5, beta=-0.5, A,B,C ~ U[-1,1], NN/NT/TN/TT on the ragged
    shapes 4095x3073x2047 and 5000^3."""
    out = []
    for si, (M, N, K) in enumerate([(4095, 3073, 2047), (5000, 5000, 5000)]):
        for la in "NT":
            for lb in "NT":
                out.append(Problem(M, N, K, la, lb, "bf16", "f32", "none", 1.5, -0.5,
                                   key=(3, si), name="bf16_layout_sweep"))
    return out


def int8_4096_bias():
    """int8 4096^3 NN, A,B integers in [-128,127], int32 accumulate, D = acc + bias_i32[N],
    bias ~ integers in [-2^20, 2^20]."""
    return [Problem(4096, 4096, 4096, "N", "N", "i8", "i32", "bias", 1.0, 0.0,
                    a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                    bias_dist=("int", -(1 << 20), 1 << 20), key=(4, 0), name="int8_4096_bias")]


def fc_layers(layouts=("NN",)):
    """Fully-connected shapes, fp16 in / fp32 acc / fp16 out with bias+ReLU: activations A ~
    N(0,1), weights B ~ N(0,1/K), bias fp32 ~ U[-0.5,0.5].  The three shapes NN, then the
    memory-bound one again with the weights stored N x K (B transposed, the layout of a linear
    layer's weight matrix)."""
    out = []
    shapes = [(16, 4096, 4096), (8192, 16384, 4096), (8192, 4096, 16384)]
    for si, (M, N, K) in enumerate(shapes):
        for lay in layouts:
            out.append(Problem(M, N, K, lay[0], lay[1], "f16", "f16", "bias_relu", 1.0, 0.0,
                               a_dist=("normal", 1.0), b_dist=("normal", 1.0 / math.sqrt(K)),
                               key=(5, si), name="fc_layers"))
    M, N, K = shapes[0]
    out.append(Problem(M, N, K, "N", "T", "f16", "f16", "bias_relu", 1.0, 0.0,
                       a_dist=("normal", 1.0), b_dist=("normal", 1.0 / math.sqrt(K)),
                       key=(5, 0), name="fc_layers"))
    return out


def batched_fp16():
    """A strided batch of 16 independent fp16 2048^3 products (NN, bias per product, ReLU ->
    fp16), A,B ~ N(0,1)/sqrt(K), bias ~ U[-0.5,0.5]: the batched operand layout of "Flexible
    Performant GEMM Kernels on GPUs", section 4, at a size where one launch fills the chip
    (16 x 64 tiles of 256x256)."""
    K = 2048
    s = 1.0 / math.sqrt(K)
    return [Problem(2048, 2048, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(6, 0), name="batched_fp16",
                    batch=16)]


def batched2_fp16():
    """A two-mode batch (the index map of a tensor contraction whose batch index has two modes):
    D[b1, b2] = ReLU(A[b1] B[b2] + bias[b1, b2]) for b1, b2 < 4, fp16 2048^3 products, A moving
    with b1 only, B with b2 only (each broadcast along the other mode), D blocks b2-major;
    A,B ~ N(0,1)/sqrt(K), bias ~ U[-0.5,0.5]."""
    K = 2048
    s = 1.0 / math.sqrt(K)
    n = 2048 * 2048
    return [Problem(2048, 2048, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(12, 0), name="batched2_fp16",
                    batch=4, stride_a=n, stride_b=0, stride_c=n, stride_bias=2048,
                    batch2=4, stride2_a=0, stride2_b=n, stride2_c=4 * n, stride2_bias=4 * 2048)]


def fp16_8192_transforms():
    """The headline shape with the load transforms of "Flexible Performant GEMM Kernels on
    GPUs" section 5.3 (Table 2, bias + ReLU on C and D) plus a ReLU on A as it is loaded (an
    activation fused into the next layer's GEMM): fp16 8192^3 NN, D = ReLU(relu(A) B +
    relu(C) + bias), A,B ~ N(0,1)/sqrt(K), C ~ U[-1,1] fp16, bias ~ U[-0.5,0.5]."""
    K = 8192
    s = 1.0 / math.sqrt(K)
    return [Problem(8192, 8192, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 1.0,
                    a_dist=("normal", s), b_dist=("normal", s), key=(7, 0),
                    name="fp16_8192_transforms", transform_a="relu", transform_c="relu")]


def diag_fp16():
    """A diagonal-operand product at the headline size: D = diag(a) B + bias, ReLU, fp16
    8192 x 8192 (K = M = 8192), a ~ U[-1,1], B ~ N(0,1), bias ~ U[-0.5,0.5].  Memory-bound:
    read B, write D ("Flexible Performant GEMM Kernels on GPUs", section 5.2, Table 1)."""
    return [Problem(8192, 8192, 8192, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                    b_dist=("normal", 1.0), key=(8, 0), name="diag_fp16", kind_a="diagonal")]


def complex_fp16():
    """Complex and dual numbers with fp16 parts, fp32 accumulation and output, 4096^3 NN, parts
    ~ U[-1,1] ("Flexible Performant GEMM Kernels on GPUs", section 5.4, Figure 12)."""
    return [Problem(4096, 4096, 4096, "N", "N", "cf16", "cf32", "none", 1.0, 0.0, key=(9, 0),
                    name="complex_fp16"),
            Problem(4096, 4096, 4096, "N", "N", "df16", "df32", "none", 1.0, 0.0, key=(9, 1),
                    name="complex_fp16")]


def convert_fp16():
    """Type-converting load transforms ("Flexible Performant GEMM Kernels on GPUs", section 4: a
    transform after every load, including a type conversion) at fully-connected and headline
    sizes: [0] fp16 activations 8192 x 4096 ~ N(0,1)/sqrt(K) times int8 weights 4096 x 16384
    (integers in [-8, 8]) converted to fp16 as they are loaded, bias+ReLU -> fp16; [1] fp32
    operands 8192^3 ~ N(0,1)/sqrt(K) rounded to bf16 as they are loaded, bias+ReLU -> bf16."""
    K = 4096
    out = [Problem(8192, 16384, K, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                   a_dist=("normal", 1.0 / math.sqrt(K)), b_dist=("int", -8, 8), key=(10, 0),
                   name="convert_fp16", transform_b="from_i8")]
    K = 8192
    s = 1.0 / math.sqrt(K)
    out.append(Problem(8192, 8192, K, "N", "N", "bf16", "bf16", "bias_relu", 1.0, 0.0,
                       a_dist=("normal", s), b_dist=("normal", s), key=(10, 1),
                       name="convert_fp16", transform_a="from_f32", transform_b="from_f32"))
    return out


WORKLOADS = {
    "sgemm_256": sgemm_256,
    "fp16_8192_bias_relu": fp16_8192_bias_relu,
    "fp16_long_k": fp16_long_k,
    "mid_size": mid_size,
    "bf16_layout_sweep": bf16_layout_sweep,
    "int8_4096_bias": int8_4096_bias,
    "fc_layers": fc_layers,
    "batched_fp16": batched_fp16,
    "batched2_fp16": batched2_fp16,
    "fp16_8192_transforms": fp16_8192_transforms,
    "diag_fp16": diag_fp16,
    "complex_fp16": complex_fp16,
    "convert_fp16": convert_fp16,
}


def exact_integer_problem(M, N, K, op_a, op_b, ab, cd, epi, alpha, beta, key, ld_pad=0, **batch):
    """Inputs whose every partial sum is an integer of magnitude <= 16*K + small, so fp32
    accumulation (any order) and the fp32 epilogue are exact whenever 16*K < 2^24 and alpha,
    beta are small powers of two: A,B integers in [-4,4], C integers in [-8,8], bias integers in
    [-8,8]."""
    p = Problem(M, N, K, op_a, op_b, ab, cd, epi, alpha, beta,
                a_dist=("int", -4, 4), b_dist=("int", -4, 4), c_dist=("int", -8, 8),
                bias_dist=("int", -8, 8), key=key, name="exact_int", **batch)
    if ld_pad:
        p = replace(p, lda=p.lda + ld_pad, ldb=p.ldb + ld_pad, ldc=p.ldc + ld_pad)
    return p
