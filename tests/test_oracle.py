"""Pins of the CPU oracle against facts that do not come from the oracle itself: IEEE format
definitions (exhaustive decoder checks against numpy / torch), library products on tiny inputs,
loop-order invariance, identities, the transpose law (AB)^T = B^T A^T, alpha/beta linearity and
a hand-worked epilogue instance."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- decoders and rounding --------------------------------------------------------------------

def test_f16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode("f16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode("bf16", bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _finite_patterns(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.decode(dtype, bits)
    keep = np.isfinite(v)
    return bits[keep], v[keep]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_round_is_inverse_of_decode(dtype):
    bits, v = _finite_patterns(dtype)
    assert np.array_equal(oracle.round_to(dtype, v), bits)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_round_ties_to_even_and_neighbours(dtype):
    # positive finite values in increasing order: every midpoint goes to the even pattern and
    # points just off the midpoint go to the nearer neighbour
    bits, v = _finite_patterns(dtype)
    pos = (v > 0)
    b, x = bits[pos], v[pos]
    order = np.argsort(x)
    b, x = b[order], x[order]
    lo, hi, blo, bhi = x[:-1], x[1:], b[:-1], b[1:]
    mid = (lo + hi) / 2                       # exact in float64
    got = oracle.round_to(dtype, mid)
    even = np.where((blo & 1) == 0, blo, bhi)
    assert np.array_equal(got, even)
    eps = (hi - lo) * 1e-6
    assert np.array_equal(oracle.round_to(dtype, mid - eps), blo)
    assert np.array_equal(oracle.round_to(dtype, mid + eps), bhi)


def test_f16_round_matches_numpy_random():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(200000) * 10.0 ** g.integers(-9, 6, 200000),
                        g.uniform(-70000, 70000, 10000)])
    assert np.array_equal(oracle.round_to("f16", x), x.astype(np.float16).view(np.uint16))


def test_bf16_round_matches_torch_on_float32_values():
    g = np.random.default_rng(8)
    x = (g.standard_normal(200000) * 10.0 ** g.integers(-30, 30, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to("bf16", x.astype(np.float64)), ref)


def test_round_overflow_and_signed_zero():
    r = oracle.round_to("f16", np.array([65504.0, 65519.99, 65520.0, -1e9, -0.0, 2.0 ** -26]))
    assert list(r) == [0x7BFF, 0x7BFF, 0x7C00, 0xFC00, 0x8000, 0x0000]


# ---- the product ------------------------------------------------------------------------------

def _random_problem(g, M, N, K, la, lb, integer, pad=0):
    lda = (K if la == "N" else M) + pad
    ldb = (N if lb == "N" else K) + pad
    if integer:
        X = g.integers(-128, 128, (M, K)).astype(np.int8)
        Y = g.integers(-128, 128, (K, N)).astype(np.int8)
    else:
        X = g.uniform(-1, 1, (M, K)).astype(np.float32)
        Y = g.uniform(-1, 1, (K, N)).astype(np.float32)
    A = np.zeros((M, lda) if la == "N" else (K, lda), X.dtype)
    B = np.zeros((K, ldb) if lb == "N" else (N, ldb), Y.dtype)
    if la == "N":
        A[:, :K] = X
    else:
        A[:, :M] = X.T
    if lb == "N":
        B[:, :N] = Y
    else:
        B[:, :K] = Y.T
    return X, Y, A, lda, B, ldb


@pytest.mark.parametrize("shape", [(64, 48, 80), (37, 53, 129)])
@pytest.mark.parametrize("ab", ["f32", "i8"])
def test_loop_orders_bit_identical(shape, ab):
    M, N, K = shape
    g = np.random.default_rng(11)
    X, Y, A, lda, B, ldb = _random_problem(g, M, N, K, "N", "N", ab == "i8")
    outs = [oracle.gemm(M, N, K, "N", "N", A, lda, B, ldb, ab, order=o, threads=t)
            for o in ("ijk", "kij", "tiled") for t in (1, 3)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_brute_force_tiny_against_numpy(lay):
    g = np.random.default_rng(12)
    for M in (1, 2, 3):
        for N in (1, 2, 3):
            for K in (1, 2, 3):
                # int8 in {-2..2}: exact in int64
                X = g.integers(-2, 3, (M, K)).astype(np.int8)
                Y = g.integers(-2, 3, (K, N)).astype(np.int8)
                A = X if lay[0] == "N" else np.ascontiguousarray(X.T)
                B = Y if lay[1] == "N" else np.ascontiguousarray(Y.T)
                lda = A.shape[1]
                ldb = B.shape[1]
                got = oracle.gemm(M, N, K, lay[0], lay[1], A, lda, B, ldb, "i8")
                assert np.array_equal(got, X.astype(np.int64) @ Y.astype(np.int64))
                # float32 inputs: K <= 3 products of float32 values are exact in float64 and
                # the sum of <= 3 such products differs from numpy's only by summation order,
                # so compare to an expansion that adds in ascending k
                Xf = g.uniform(-1, 1, (M, K)).astype(np.float32)
                Yf = g.uniform(-1, 1, (K, N)).astype(np.float32)
                A = Xf if lay[0] == "N" else np.ascontiguousarray(Xf.T)
                B = Yf if lay[1] == "N" else np.ascontiguousarray(Yf.T)
                got = oracle.gemm(M, N, K, lay[0], lay[1], A, A.shape[1], B, B.shape[1], "f32")
                ref = np.zeros((M, N))
                for k in range(K):
                    ref = ref + np.outer(Xf[:, k].astype(np.float64), Yf[k, :].astype(np.float64))
                assert np.array_equal(got, ref)
                np.testing.assert_allclose(got, Xf.astype(np.float64) @ Yf.astype(np.float64),
                                           rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_layouts_against_numpy_with_padded_ld(lay):
    g = np.random.default_rng(13)
    for (M, N, K) in [(5, 7, 3), (1, 9, 4), (8, 1, 6), (6, 6, 1), (13, 11, 17)]:
        X, Y, A, lda, B, ldb = _random_problem(g, M, N, K, lay[0], lay[1], True, pad=3)
        got = oracle.gemm(M, N, K, lay[0], lay[1], A, lda, B, ldb, "i8")
        assert np.array_equal(got, X.astype(np.int64) @ Y.astype(np.int64))


def test_identity_and_zero():
    g = np.random.default_rng(14)
    M = K = N = 24
    X = g.uniform(-1, 1, (M, K)).astype(np.float32)
    I = np.eye(K, dtype=np.float32)
    assert np.array_equal(oracle.gemm(M, N, K, "N", "N", X, K, I, N, "f32"), X.astype(np.float64))
    assert np.array_equal(oracle.gemm(M, N, K, "N", "N", I, K, X, N, "f32"), X.astype(np.float64))
    Z = np.zeros((M, K), np.float32)
    C = g.uniform(-1, 1, (M, N)).astype(np.float32)
    bias = g.uniform(-1, 1, N).astype(np.float32)
    got = oracle.gemm(M, N, K, "N", "N", Z, K, X, N, "f32", C=C, ldc=N, cd="f32", bias=bias,
                      alpha=3.0, beta=0.5, relu=False)
    assert np.array_equal(got, 0.5 * C.astype(np.float64) + bias.astype(np.float64)[None, :])


@pytest.mark.parametrize("ab", ["f32", "i8"])
def test_transpose_law(ab):
    # (XY)^T = Y^T X^T: the TT problem on the same stored arrays gives the transpose bit for bit
    g = np.random.default_rng(15)
    M, N, K = 29, 41, 67
    X, Y, A, lda, B, ldb = _random_problem(g, M, N, K, "N", "N", ab == "i8")
    R = oracle.gemm(M, N, K, "N", "N", A, lda, B, ldb, ab)
    RT = oracle.gemm(N, M, K, "T", "T", B, ldb, A, lda, ab)
    assert np.array_equal(RT, R.T)


def test_alpha_beta_linearity():
    g = np.random.default_rng(16)
    M, N, K = 33, 21, 45
    X, Y, A, lda, B, ldb = _random_problem(g, M, N, K, "T", "N", False)
    C = g.uniform(-1, 1, (M, N)).astype(np.float32)
    base = oracle.gemm(M, N, K, "T", "N", A, lda, B, ldb, "f32")
    got = oracle.gemm(M, N, K, "T", "N", A, lda, B, ldb, "f32", C=C, ldc=N, cd="f32",
                      alpha=1.5, beta=-0.5)
    np.testing.assert_allclose(got, 1.5 * base - 0.5 * C.astype(np.float64), rtol=1e-15, atol=1e-15)


def test_epilogue_hand_worked_instance():
    d = json.load(open(os.path.join(GOLDEN, "epilogue_2x2.json")))
    A = np.array(d["A"], np.float32)
    B = np.array(d["B"], np.float32)
    C = np.array(d["C"], np.float32)
    bias = np.array(d["bias"], np.float32)
    M, N, K = d["M"], d["N"], d["K"]
    common = dict(C=C, ldc=N, cd="f32", alpha=d["alpha"], beta=d["beta"])
    got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "f32", bias=bias, relu=False, **common)
    assert np.array_equal(got, np.array(d["expected_none"]))
    got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "f32", bias=bias, relu=True, **common)
    assert np.array_equal(got, np.array(d["expected_relu"]))
    got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "f32", relu=True, **common)
    assert np.array_equal(got, np.array(d["expected_no_bias_relu"]))


def test_bias_is_per_column_and_beta_zero_ignores_c():
    M, N, K = 5, 7, 3
    A = np.zeros((M, K), np.float32)
    B = np.ones((K, N), np.float32)
    bias = np.arange(N, dtype=np.float32) - 3
    C = np.full((M, N), np.nan, np.float32)
    got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "f32", C=C, ldc=N, cd="f32", bias=bias,
                      alpha=1.0, beta=0.0, relu=True)
    assert np.array_equal(got, np.tile(np.maximum(bias.astype(np.float64), 0), (M, 1)))


def test_int8_full_range_exact():
    g = np.random.default_rng(17)
    M, N, K = 16, 16, 512
    A = np.full((M, K), -128, np.int8)
    B = np.full((K, N), -128, np.int8)
    bias = g.integers(-(1 << 20), (1 << 20) + 1, N).astype(np.int32)
    got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "i8", bias=bias)
    assert np.array_equal(got, np.full((M, N), 128 * 128 * K, np.int64) + bias.astype(np.int64))


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("bf16", "f32"), ("i8", "i32")])
def test_points_equal_full_result(lay, ab, cd):
    p = synth.Problem(37, 45, 70, lay[0], lay[1], ab, cd, "bias_relu" if ab != "i8" else "bias",
                      1.5 if ab != "i8" else 1.0, -0.5 if ab != "i8" else 1.0, key=(99, 1),
                      a_dist=("int", -100, 100) if ab == "i8" else ("uniform", -1, 1),
                      b_dist=("int", -100, 100) if ab == "i8" else ("uniform", -1, 1),
                      c_dist=("int", -1000, 1000) if ab == "i8" else ("uniform", -1, 1),
                      bias_dist=("int", -1000, 1000) if ab == "i8" else ("uniform", -0.5, 0.5))
    x = synth.make_inputs(p)
    kw = dict(C=x["C"], ldc=p.ldc, cd=cd, bias=x["bias"], alpha=p.alpha, beta=p.beta, relu=p.relu)
    full = oracle.gemm(p.M, p.N, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, ab,
                       order="ijk", **kw)
    g = np.random.default_rng(3)
    ii = g.integers(0, p.M, 200)
    jj = g.integers(0, p.N, 200)
    pts = oracle.points(ii, jj, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, ab, **kw)
    assert np.array_equal(pts, full[ii, jj])


def test_row_subset_equals_full():
    p = synth.Problem(70, 33, 51, "T", "N", "f16", "f16", "bias_relu", key=(98, 0))
    x = synth.make_inputs(p)
    full = oracle.gemm(p.M, p.N, p.K, "T", "N", x["A"], p.lda, x["B"], p.ldb, "f16",
                       bias=x["bias"], relu=True)
    part = oracle.gemm(p.M, p.N, p.K, "T", "N", x["A"], p.lda, x["B"], p.ldb, "f16",
                       bias=x["bias"], relu=True, rows=(13, 47))
    assert np.array_equal(part, full[13:47])


def test_exact_integer_inputs_are_integers():
    p = synth.exact_integer_problem(20, 30, 40, "N", "T", "bf16", "bf16", "bias_relu", 2.0, -1.0,
                                    key=(97, 0))
    x = synth.make_inputs(p)
    for k in ("A", "B"):
        v = oracle.decode("bf16", x[k])
        assert np.array_equal(v, np.round(v)) and np.abs(v).max() <= 4
    ref = oracle.gemm(p.M, p.N, p.K, "N", "T", x["A"], p.lda, x["B"], p.ldb, "bf16", C=x["C"],
                      ldc=p.ldc, cd="bf16", bias=x["bias"], alpha=2.0, beta=-1.0, relu=True)
    assert np.array_equal(ref, np.round(ref))


# ---- strided batch ------------------------------------------------------------------------------

@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_batched_against_numpy_strided_views(lay):
    """Each product of a strided batch is the plain product of the operands at b * stride:
    checked against numpy's batched matmul on as_strided views of the same flat buffers
    (int8 values, exact in int64), with padded strides, a shared (stride 0) operand and
    per-product bias."""
    g = np.random.default_rng(31)
    for (M, N, K, batch) in [(3, 5, 4, 3), (1, 7, 2, 4), (6, 1, 5, 2), (4, 4, 4, 1)]:
        lda = (K if lay[0] == "N" else M) + 2
        ldb = (N if lay[1] == "N" else K) + 1
        ldc = N + 3
        sa = ((M if lay[0] == "N" else K) * lda) + 5
        sb_shared = 0                                  # B shared by every product
        sc = M * ldc + 2
        sbias = N + 1
        A = g.integers(-3, 4, sa * batch + 8).astype(np.int8)
        B = g.integers(-3, 4, (K if lay[1] == "N" else N) * ldb + 8).astype(np.int8)
        C = g.integers(-5, 6, sc * batch + 8).astype(np.int32)
        bias = g.integers(-9, 10, sbias * batch + 4).astype(np.int32)
        got = oracle.gemm_batched(M, N, K, lay[0], lay[1], A, lda, B, ldb, "i8", C=C, ldc=ldc,
                                  cd="i32", bias=bias, alpha=1, beta=1, relu=True, batch=batch,
                                  stride_a=sa, stride_b=sb_shared, stride_c=sc,
                                  stride_bias=sbias)
        st = np.lib.stride_tricks.as_strided
        A64, B64, C64, b64 = (x.astype(np.int64) for x in (A, B, C, bias))
        e = 8
        if lay[0] == "N":
            Av = st(A64, (batch, M, K), (sa * e, lda * e, e))
        else:
            Av = st(A64, (batch, K, M), (sa * e, lda * e, e)).transpose(0, 2, 1)
        if lay[1] == "N":
            Bv = st(B64, (batch, K, N), (0, ldb * e, e))
        else:
            Bv = st(B64, (batch, N, K), (0, ldb * e, e)).transpose(0, 2, 1)
        Cv = st(C64, (batch, M, N), (sc * e, ldc * e, e))
        bv = st(b64, (batch, 1, N), (sbias * e, 0, e))
        ref = np.maximum(np.matmul(Av, Bv) + Cv + bv, 0)
        assert np.array_equal(got, ref)


def test_batched_of_one_and_zero_strides_repeat_the_product():
    g = np.random.default_rng(32)
    M, N, K = 5, 6, 7
    A = g.integers(-4, 5, M * K).astype(np.int8)
    B = g.integers(-4, 5, K * N).astype(np.int8)
    one = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "i8")
    rep = oracle.gemm_batched(M, N, K, "N", "N", A, K, B, N, "i8", batch=3, stride_c=M * N)
    for b in range(3):
        assert np.array_equal(rep[b], one)


# ---- load transforms ---------------------------------------------------------------------------

def test_zero_negative_rule():
    """max(x, 0) for non-NaN x, read as: sign bit set -> +0 (so -0 -> +0, -NaN -> 0, +NaN kept)."""
    x = np.array([-2.5, -0.0, 0.0, 1.5, -np.inf, np.inf, np.nan, -np.nan])
    y = oracle.zero_negative(x)
    assert list(y[:6]) == [0.0, 0.0, 0.0, 1.5, 0.0, np.inf]
    assert not np.signbit(y[:2]).any()
    assert np.isnan(y[6]) and y[7] == 0.0 and not np.signbit(y[7])
    assert list(oracle.zero_negative(np.array([-128, -1, 0, 1, 127], np.int64))) == [0, 0, 0, 1, 127]


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_transforms_against_numpy(lay):
    """tA, tB on the operands and tC on C against numpy with np.maximum(., 0) applied to the
    logical matrices (int8 values, exact in int64)."""
    g = np.random.default_rng(33)
    for (M, N, K) in [(4, 5, 6), (1, 3, 7), (9, 2, 4)]:
        X, Y, A, lda, B, ldb = _random_problem(g, M, N, K, lay[0], lay[1], True, pad=2)
        C = g.integers(-50, 50, M * N).astype(np.int32)
        for ta, tb, tc in [("relu", "none", "none"), ("none", "relu", "relu"), ("relu", "relu", "relu")]:
            got = oracle.gemm(M, N, K, lay[0], lay[1], A, lda, B, ldb, "i8", C=C, ldc=N, cd="i32",
                              alpha=1, beta=1, transform_a=ta, transform_b=tb, transform_c=tc)
            Xt = np.maximum(X.astype(np.int64), 0) if ta == "relu" else X.astype(np.int64)
            Yt = np.maximum(Y.astype(np.int64), 0) if tb == "relu" else Y.astype(np.int64)
            Ct = C.astype(np.int64).reshape(M, N)
            Ct = np.maximum(Ct, 0) if tc == "relu" else Ct
            assert np.array_equal(got, Xt @ Yt + Ct)


# ---- diagonal operands ---------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["A", "B", "AB"])
def test_diagonal_operands_against_numpy(which):
    """A diagonal operand given by its vector equals the dense product with numpy's np.diag of
    that vector (int8 values, exact), for row subsets too."""
    g = np.random.default_rng(34)
    for (M, N) in [(5, 7), (6, 6), (9, 3)]:
        if which == "AB":
            N = M
        K = M if "A" in which else N
        avec = g.integers(-5, 6, M).astype(np.int8)
        bvec = g.integers(-5, 6, N).astype(np.int8)
        X = g.integers(-5, 6, (M, K)).astype(np.int8)
        Y = g.integers(-5, 6, (K, N)).astype(np.int8)
        Aref = np.diag(avec.astype(np.int64)) if "A" in which else X.astype(np.int64)
        Bref = np.diag(bvec.astype(np.int64)) if "B" in which else Y.astype(np.int64)
        A = avec if "A" in which else X
        B = bvec if "B" in which else Y
        kw = dict(kind_a="diagonal" if "A" in which else "dense",
                  kind_b="diagonal" if "B" in which else "dense")
        got = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "i8", **kw)
        assert np.array_equal(got, Aref @ Bref)
        part = oracle.gemm(M, N, K, "N", "N", A, K, B, N, "i8", rows=(1, M - 1), **kw)
        assert np.array_equal(part, (Aref @ Bref)[1:M - 1])


# ---- complex and dual numbers -------------------------------------------------------------------

def _pairs(g, rows, cols, lo=-4, hi=4):
    re = g.integers(lo, hi + 1, (rows, cols)).astype(np.float64)
    im = g.integers(lo, hi + 1, (rows, cols)).astype(np.float64)
    return re, im


def _store_pairs(re, im, op, pad):
    if op == "T":
        re, im = re.T, im.T
    rows, cols = re.shape
    out = np.zeros((rows, cols + pad, 2), np.uint16)
    out[:, :cols, 0] = oracle.round_to("f16", re)
    out[:, :cols, 1] = oracle.round_to("f16", im)
    return out, cols + pad


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_complex_against_numpy(lay):
    """Complex numbers against numpy's complex128 matmul (integer parts: exact)."""
    g = np.random.default_rng(35)
    for (M, N, K) in [(3, 4, 5), (1, 6, 2), (7, 1, 3)]:
        ar, ai = _pairs(g, M, K)
        br, bi = _pairs(g, K, N)
        cr, ci = _pairs(g, M, N)
        A, lda = _store_pairs(ar, ai, lay[0], 2)
        B, ldb = _store_pairs(br, bi, lay[1], 1)
        C = np.stack([cr, ci], axis=-1).astype(np.float32)
        got = oracle.gemm_pair(M, N, K, lay[0], lay[1], A, lda, B, ldb, "cf16", C=C, ldc=N,
                               cd="cf32", alpha=2.0, beta=-1.0)
        ref = 2.0 * ((ar + 1j * ai) @ (br + 1j * bi)) - (cr + 1j * ci)
        assert np.array_equal(got[..., 0], ref.real) and np.array_equal(got[..., 1], ref.imag)


def test_dual_numbers_carry_the_derivative():
    """Dual numbers X + eps X': the second part of the product is d/dt (X + tX')(Y + tY') at 0 =
    X'Y + XY' (numpy real matmuls), the first part XY."""
    g = np.random.default_rng(36)
    M, N, K = 5, 6, 7
    xr, xd = _pairs(g, M, K)
    yr, yd = _pairs(g, K, N)
    A, lda = _store_pairs(xr, xd, "N", 0)
    B, ldb = _store_pairs(yr, yd, "N", 0)
    got = oracle.gemm_pair(M, N, K, "N", "N", A, lda, B, ldb, "df16")
    assert np.array_equal(got[..., 0], xr @ yr)
    assert np.array_equal(got[..., 1], xd @ yr + xr @ yd)
    # and differs from the complex product exactly by the dropped -Xd*Yd term
    c = oracle.gemm_pair(M, N, K, "N", "N", A, lda, B, ldb, "cf16")
    assert np.array_equal(c[..., 0], got[..., 0] - xd @ yd)


# ---- the tolerance normaliser ------------------------------------------------------------------

def check_max_abs_op_pins(mod):
    """max |op(X)| over the elements op(X) uses, on hand-built stored arrays whose padding and
    trailing storage hold larger values that must be left out (the tolerance's denominator,
    K * max|op(A)| * max|op(B)|, is defined over op(A) and op(B) only)."""
    h = lambda v: np.asarray(v, np.float16).view(np.uint16)
    # op N, 2 x 3 stored with ld 5: padding columns hold 99; max |.| = 7
    xn = h([[1, -7, 2, 99, 99], [3, 0.5, -4, 99, 99]])
    assert mod.max_abs_op("f16", xn, "N", 2, 3, 5) == 7.0
    # op T: op(X) is 3 x 2, stored 2 x 3 with ld 4 (column 3 is padding, -70 there); max = 9
    xt = h([[1, 2, -9, 50], [0.25, 6, 3, -70]])
    assert mod.max_abs_op("f16", xt, "T", 3, 2, 4) == 9.0
    # the same storage read as op N 2 x 3 (ld 4) has the same elements
    assert mod.max_abs_op("f16", xt, "N", 2, 3, 4) == 9.0
    # storage past the last used element (a larger array, another product) is not part of it
    tail = np.concatenate([h([[0.5, -1.5, 1]]).reshape(-1), h([-64.0])])
    assert mod.max_abs_op("f16", tail, "N", 1, 3, 3) == 1.5
    # the largest element sits in the last used position of the last stored row
    xl = h([[1, 2, 0, 100], [3, -11, 0, 100]])
    assert mod.max_abs_op("f16", xl, "T", 2, 2, 4) == 11.0
    # int8, bf16, fp32 decode by value; empty operands give 0
    assert mod.max_abs_op("i8", np.array([[-128, 5], [3, 127]], np.int8), "N", 2, 2, 2) == 128.0
    bf = (np.array([[-2.5, 1.0], [0.75, 300.0]], np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert mod.max_abs_op("bf16", bf, "N", 2, 1, 2) == 2.5
    assert mod.max_abs_op("f32", np.array([1.0, -3.0, 8.0], np.float32), "T", 2, 1, 3) == 3.0
    assert mod.max_abs_op("f16", xn, "N", 0, 3, 5) == 0.0


def test_max_abs_op_pins():
    check_max_abs_op_pins(oracle)


def test_max_abs_op_matches_a_dense_view():
    # random stored arrays with padded ld: the maximum over the numpy view op(X)
    g = np.random.default_rng(5)
    for op in ("N", "T"):
        rows, cols, pad = 37, 23, 6
        srows, slen = (rows, cols) if op == "N" else (cols, rows)
        ld = slen + pad
        vals = g.uniform(-1, 1, (srows, ld))
        vals[:, slen:] = 1e4                      # padding larger than every used value
        x = vals.astype(np.float16)
        view = x[:, :slen] if op == "N" else x[:, :slen].T
        want = float(np.abs(view.astype(np.float64)).max())
        assert oracle.max_abs_op("f16", x.view(np.uint16), op, rows, cols, ld) == want


# ---- type-converting load transforms -------------------------------------------------------------

def check_conversion_pins(mod):
    """The conversion applied by the type-converting load transforms, and its use in gemm():
    round to nearest even, checked against numpy's and torch's casts and hand-placed ties, and
    op(A) I = the converted operand."""
    _rne_pins(mod)
    g = np.random.default_rng(45)
    X32 = g.normal(0, 100, (7, 5)).astype(np.float32)
    I16 = np.eye(5, dtype=np.float16).view(np.uint16)
    got = mod.gemm(7, 5, 5, "N", "N", X32, 5, I16, 5, "f16", cd="f32", transform_a="from_f32")
    assert np.array_equal(got, X32.astype(np.float16).astype(np.float64))
    # B stored 7 x 5 and transposed: I op(B) = X32^T, converted
    got = mod.gemm(5, 7, 5, "N", "T", I16, 5, X32, 5, "f16", cd="f32", transform_b="from_f32")
    assert np.array_equal(got, X32.T.astype(np.float16).astype(np.float64))


def test_conversion_pins():
    check_conversion_pins(oracle)


def _rne_pins(mod):
    # fp32 -> fp16: numpy's float32 -> float16 cast rounds to nearest even; fp32 -> bf16: torch's
    # float32 -> bfloat16 cast does; both on random values and on hand-placed ties
    oracle = mod
    g = np.random.default_rng(41)
    x = np.concatenate([g.normal(0, 3, 4000), g.uniform(-70000, 70000, 1000)]).astype(np.float32)
    ties = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(1 + 2.0 ** -11), 2048 + 1, 2048 + 3,
                     65504, 65519.99, 65520, 2.0 ** -25, 3 * 2.0 ** -25, 0.0, -0.0], np.float32)
    x = np.concatenate([x, ties])
    want16 = x.astype(np.float16).astype(np.float64)
    got16 = oracle.convert_to("f16", x.astype(np.float64))
    assert np.array_equal(got16, want16)
    assert np.array_equal(np.signbit(got16), np.signbit(want16))
    # the ties themselves, by hand: to the even neighbour
    assert list(oracle.convert_to("f16", ties[:5].astype(np.float64))) == \
        [1.0, 1 + 2.0 ** -9, -1.0, 2048.0, 2052.0]
    assert oracle.convert_to("f16", np.array([65520.0]))[0] == np.inf
    assert oracle.convert_to("f16", np.array([2.0 ** -25]))[0] == 0.0          # tie to +0
    assert oracle.convert_to("f16", np.array([3 * 2.0 ** -25]))[0] == 2.0 ** -23
    xb = x[np.abs(x) < 1e30]
    wantb = torch.from_numpy(xb).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.convert_to("bf16", xb.astype(np.float64)), wantb)
    assert list(oracle.convert_to("bf16", np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))) == \
        [1.0, 1 + 2.0 ** -6]


def test_int8_converts_exactly():
    v = np.arange(-128, 128, dtype=np.float64)
    for ab in ("f16", "bf16"):
        assert np.array_equal(oracle.convert_to(ab, v), v)


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("ab", ["f16", "bf16"])
def test_converting_transforms_against_numpy(lay, ab):
    """A stored as fp32 and B as int8 (and the reverse), converted to the input type as they
    are loaded, against numpy on the converted logical matrices (integer-valued conversions of
    small magnitude keep every product and sum exact in fp64)."""
    g = np.random.default_rng(43)
    cast = (lambda v: v.astype(np.float16).astype(np.float64)) if ab == "f16" else \
        (lambda v: torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy())
    for (M, N, K) in [(4, 5, 6), (1, 3, 7), (9, 2, 4)]:
        X32 = (g.integers(-64, 64, (M, K)) / 8.0 + g.uniform(-1e-3, 1e-3, (M, K))).astype(np.float32)
        Y8 = g.integers(-128, 128, (K, N)).astype(np.int8)
        A = _store_logical(X32, lay[0], 2)
        B = _store_logical(Y8, lay[1], 3)
        lda, ldb = A.shape[1], B.shape[1]
        got = oracle.gemm(M, N, K, lay[0], lay[1], A, lda, B, ldb, ab, cd="f32",
                          transform_a="from_f32", transform_b="from_i8")
        want = cast(X32) @ Y8.astype(np.float64)
        assert np.array_equal(got, want)
        # the other way round
        A8 = _store_logical(Y8.T.copy(), lay[0], 1)
        B32 = _store_logical(X32.T.copy(), lay[1], 0)
        got = oracle.gemm(N, M, K, lay[0], lay[1], A8, A8.shape[1], B32, B32.shape[1], ab, cd="f32",
                          transform_a="from_i8", transform_b="from_f32")
        assert np.array_equal(got, Y8.T.astype(np.float64) @ cast(X32.T.copy()))


def test_converting_transform_times_identity_is_the_conversion():
    # op(A) I = op(A): the result is the converted operand itself, element for element
    g = np.random.default_rng(44)
    M, K = 37, 29
    X32 = g.normal(0, 100, (M, K)).astype(np.float32)
    I16 = np.eye(K, dtype=np.float16).view(np.uint16)
    for ab in ("f16", "bf16"):
        Ib = I16 if ab == "f16" else (np.eye(K, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        got = oracle.gemm(M, K, K, "N", "N", X32, K, Ib, K, ab, cd="f32", transform_a="from_f32")
        assert np.array_equal(got, oracle.convert_to(ab, X32.astype(np.float64)))


def test_max_abs_op_of_a_converted_operand():
    x = np.array([[1.0, -65519.99, 7.0, 1e6]], np.float32)      # last column is padding
    assert oracle.max_abs_op("f16", x, "N", 1, 3, 4, transform="from_f32") == 65504.0
    x8 = np.array([[-128, 5, 127]], np.int8)
    assert oracle.max_abs_op("bf16", x8, "T", 2, 1, 3, transform="from_i8") == 128.0


def _store_logical(X, op, pad):
    """Row-major storage of logical X (op N) or of its transpose (op T), `pad` extra columns of
    junk that must never be read."""
    S = X if op == "N" else X.T
    out = np.full((S.shape[0], S.shape[1] + pad), 99, dtype=X.dtype)
    out[:, : S.shape[1]] = S
    return out


# ---- two batch modes -----------------------------------------------------------------------------

def check_two_mode_pins(mod):
    for lay in ("NN", "NT", "TN", "TT"):
        _two_mode_case(mod, lay)


@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_two_mode_batch_against_numpy_strided_views(lay):
    """Product (b1, b2) of a two-mode batch uses the operands at b1 * stride + b2 * stride2:
    checked against numpy's broadcasting matmul on 4-D as_strided views of the same flat buffers
    (int8, exact in int64).  A varies with b1 only (broadcast along b2), B with b2 only, C, D
    and the bias with both; padded leading dimensions and strides."""
    _two_mode_case(oracle, lay)


def _two_mode_case(oracle, lay):
    g = np.random.default_rng(47)
    st = np.lib.stride_tricks.as_strided
    e = 8
    for (M, N, K, b1, b2) in [(3, 5, 4, 2, 3), (1, 6, 3, 3, 2), (4, 2, 5, 1, 4), (2, 3, 2, 3, 1)]:
        lda = (K if lay[0] == "N" else M) + 1
        ldb = (N if lay[1] == "N" else K) + 2
        ldc = N + 1
        rows_a, rows_b = (M if lay[0] == "N" else K), (K if lay[1] == "N" else N)
        sa, sa2 = rows_a * lda + 3, 0                  # A: moves with b1, shared along b2
        sb, sb2 = 0, rows_b * ldb + 1                  # B: shared along b1, moves with b2
        sc2 = M * ldc + 2
        sc = b2 * sc2 + 5                              # D blocks laid out b1-major
        sbias, sbias2 = 1, N + 2
        A = g.integers(-3, 4, sa * b1 + 8).astype(np.int8)
        B = g.integers(-3, 4, sb2 * b2 + 8).astype(np.int8)
        C = g.integers(-5, 6, sc * b1 + 8).astype(np.int32)
        bias = g.integers(-9, 10, sbias * b1 + sbias2 * b2 + N + 4).astype(np.int32)
        got = oracle.gemm_batched(M, N, K, lay[0], lay[1], A, lda, B, ldb, "i8", C=C, ldc=ldc,
                                  cd="i32", bias=bias, alpha=1, beta=1, relu=True, batch=b1,
                                  stride_a=sa, stride_b=sb, stride_c=sc, stride_bias=sbias,
                                  batch2=b2, stride2_a=sa2, stride2_b=sb2, stride2_c=sc2,
                                  stride2_bias=sbias2)
        A64, B64, C64, bb = (x.astype(np.int64) for x in (A, B, C, bias))
        if lay[0] == "N":
            Av = st(A64, (b1, b2, M, K), (sa * e, sa2 * e, lda * e, e))
        else:
            Av = st(A64, (b1, b2, K, M), (sa * e, sa2 * e, lda * e, e)).transpose(0, 1, 3, 2)
        if lay[1] == "N":
            Bv = st(B64, (b1, b2, K, N), (sb * e, sb2 * e, ldb * e, e))
        else:
            Bv = st(B64, (b1, b2, N, K), (sb * e, sb2 * e, ldb * e, e)).transpose(0, 1, 3, 2)
        Cv = st(C64, (b1, b2, M, N), (sc * e, sc2 * e, ldc * e, e))
        bv = st(bb, (b1, b2, 1, N), (sbias * e, sbias2 * e, 0, e))
        ref = np.maximum(np.matmul(Av, Bv) + Cv + bv, 0)
        assert got.size == b1 * b2 * M * N
        assert np.array_equal(got.reshape(b1, b2, M, N), ref)


def test_two_mode_batch_of_one_mode_is_the_strided_batch():
    g = np.random.default_rng(48)
    M, N, K = 5, 4, 3
    A = g.integers(-3, 4, 4 * M * K).astype(np.int8)
    B = g.integers(-3, 4, K * N).astype(np.int8)
    one = oracle.gemm_batched(M, N, K, "N", "N", A, K, B, N, "i8", ldc=N, cd="i32", batch=4,
                              stride_a=M * K, stride_c=M * N)
    two = oracle.gemm_batched(M, N, K, "N", "N", A, K, B, N, "i8", ldc=N, cd="i32", batch=2,
                              stride_a=2 * M * K, stride_c=2 * M * N, batch2=2, stride2_a=M * K,
                              stride2_c=M * N)
    assert np.array_equal(two.reshape(4, M, N), one)
