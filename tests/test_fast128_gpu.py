"""GPU parity of the fast kernel's 128x128-tile variant (mid-size 16-bit products, operands read
in place): every layout and 16-bit type pair on ragged shapes (M and N off the tile, a K tail),
the epilogue variants, batches of one and two modes, and the plan's own choice of the variant,
against the oracle through the C ABI.  Exact-integer inputs make every comparison bit-exact."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
import tiled_gemm_epilogues_amd as tge
from gpu_helpers import (FORCE, batch_offset, check, reference, reference_batched, run, run_batched,
                         sentinel, to_dev, to_host)

pytestmark = pytest.mark.gpu

LAYOUTS = ["NN", "NT", "TN", "TT"]
PAIRS = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture
def tile128(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    monkeypatch.setitem(FORCE, "tile", 128)


# (M, N, K, epilogue, alpha, beta, ld_pad): M and N multiples of 8 so that every layout can be
# read in place; K tails of 8, 0 and 40 elements
SHAPES = [((296, 264, 200), "bias_relu", 1.0, 0.0, 0),
          ((1000, 776, 1024), "bias", 2.0, -1.0, 8),
          ((128, 128, 64), "none", 1.0, 1.0, 0),
          ((520, 392, 360), "relu", 0.5, 0.5, 16)]


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("pair", range(len(PAIRS)))
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_fast128_exact(shape, pair, lay, tile128):
    (M, N, K), epi, alpha, beta, pad = SHAPES[shape]
    ab, cd = PAIRS[pair]
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta,
                                    key=(170, shape * 16 + pair * 4 + LAYOUTS.index(lay)), ld_pad=pad)
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 "), d
    check(p, x, D, reference(p, x), exact=True)


def test_fast128_random_within_tolerance(tile128):
    p = synth.Problem(1536, 1536, 1536, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                      a_dist=("normal", 1.0 / np.sqrt(1536)), b_dist=("normal", 1.0 / np.sqrt(1536)),
                      key=(171, 0))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert pl.describe().startswith("gemm_fast_128x128 "), pl.describe()
    err = check(p, x, D, reference(p, x, threads=16))
    print(f"normalised error {err:.3e}", flush=True)


@pytest.mark.parametrize("modes", [1, 2])
def test_fast128_batches(modes, tile128):
    M, N, K = 264, 392, 256
    if modes == 1:
        p = synth.exact_integer_problem(M, N, K, "N", "T", "bf16", "f32", "bias", 1.0, 1.0,
                                        key=(172, 0), batch=3, stride_a=M * K + 8, stride_b=0,
                                        stride_c=M * N + 16, stride_bias=N)
    else:
        p = synth.exact_integer_problem(M, N, K, "T", "N", "f16", "f16", "bias_relu", 1.0, 0.0,
                                        key=(172, 1), batch=2, batch2=3, stride_a=K * M, stride_b=0,
                                        stride2_a=0, stride2_b=K * N, stride_c=3 * M * N,
                                        stride2_c=M * N, stride_bias=0, stride2_bias=N)
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    print(pl.describe(), flush=True)
    assert pl.describe().startswith("gemm_fast_128x128 "), pl.describe()
    ref = reference_batched(p, x)
    for b in range(p.batch * p.batch2):
        off = batch_offset(p, b)
        Db = Df[off: off + p.M * p.ldc].reshape(p.M, p.ldc)
        check(p, x, Db, ref[b], exact=True)


def test_fast128_chosen_for_mid_size_products():
    # the plan's own choice: 128-wide tiles where 256-wide ones would leave most CUs idle
    for (M, N, K) in [(2048, 2048, 2048), (4096, 2048, 2048), (1536, 1536, 1536)]:
        p = synth.exact_integer_problem(M, N, K, "N", "N", "f16", "f32", "bias_relu", 1.0, 0.0,
                                        key=(173, M))
        x = synth.make_inputs(p)
        D, pl = run(p, x)
        print(pl.describe(), flush=True)
        assert pl.describe().startswith("gemm_fast_128x128 "), pl.describe()
        check(p, x, D, reference(p, x, threads=16), exact=True)


def test_fast128_noalloc_and_unaligned_pointer(tile128):
    # no workspace: the no-allocation run is the same run; a pointer off 16 bytes at run time
    # takes the same tiles on an aligned copy instead, with the same result
    p = synth.exact_integer_problem(520, 264, 512, "N", "N", "f16", "f32", "bias", 1.0, 0.5,
                                    key=(174, 0))
    x = synth.make_inputs(p)
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                  algo="fast", tile=128)
    assert pl.describe().startswith("gemm_fast_128x128 "), pl.describe()
    A, B = to_dev(p.a_store, x["A"]), to_dev(p.b_store, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    outs = []
    for runner in (pl.run, pl.run_noalloc, pl.run_noalloc):
        D = to_dev(p.cd, np.full(p.M * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]))
        runner(A, B, C, D, bias, p.alpha, p.beta)
        torch.cuda.synchronize()
        outs.append(to_host(p.cd, D).reshape(p.M, p.ldc))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    check(p, x, outs[0], reference(p, x), exact=True)
    D2, _ = run(p, x, offset=1, plan=pl)
    assert np.array_equal(D2, outs[0])


# (M, N, K, layout, ab, cd, epilogue, alpha, beta): short products on the 128-wide tiles with K
# split over workgroups (pinned: tile 128 with the split algorithm)
SPLITS = [((128, 1024, 1024), "NN", "f16", "f16", "bias_relu", 1.0, 0.0),
          ((200, 520, 2048), "NT", "bf16", "f32", "bias", 2.0, -1.0),
          ((256, 392, 1536), "TN", "f16", "f32", "relu", 1.0, 1.0),
          ((96, 264, 4096), "TT", "bf16", "bf16", "bias_relu", 0.5, 0.0),
          ((520, 520, 3072), "NN", "f16", "f16", "bias", 2.0, 0.5),
          ((1000, 776, 4096), "TN", "bf16", "f32", "bias_relu", 1.0, -1.0),
          ((2048, 2048, 1024), "NT", "f16", "f32", "relu", 1.0, 0.0)]


@pytest.mark.parametrize("case", range(len(SPLITS)))
def test_fast128_split_exact(case, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "split")
    monkeypatch.setitem(FORCE, "tile", 128)
    (M, N, K), lay, ab, cd, epi, alpha, beta = SPLITS[case]
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key=(175, case))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d
    check(p, x, D, reference(p, x), exact=True)


# int8 -> int32 (alpha 1, beta 0 or 1): M and N multiples of 16 so that every layout is read in
# place (and K a multiple of 16: rows of whole chunks); K tails of 0, 112 and 0 elements
I8_SHAPES = [((304, 272, 384), "bias_relu", 0.0), ((1008, 784, 1008), "bias", 1.0), ((128, 128, 128), "none", 1.0)]


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("shape", range(len(I8_SHAPES)))
def test_fast128_int8_exact(shape, lay, tile128):
    (M, N, K), epi, beta = I8_SHAPES[shape]
    p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, beta,
                      a_dist=("int", -128, 127), b_dist=("int", -128, 127), c_dist=("int", -1000, 1000),
                      bias_dist=("int", -(1 << 20), 1 << 20), key=(176, shape * 4 + LAYOUTS.index(lay)))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 "), d
    check(p, x, D, reference(p, x), exact=True)


def test_fast128_int8_split_exact(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "split")
    monkeypatch.setitem(FORCE, "tile", 128)
    p = synth.Problem(200, 528, 8192, "N", "T", "i8", "i32", "bias", 1.0, 1.0,
                      a_dist=("int", -128, 127), b_dist=("int", -128, 127), c_dist=("int", -1000, 1000),
                      bias_dist=("int", -(1 << 20), 1 << 20), key=(177, 0))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(d, flush=True)
    assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d
    check(p, x, D, reference(p, x), exact=True)


# (M, N, K, layout, ab, cd, epilogue, alpha, beta, ld_pad, transform_a, what the description must
# show): operands the direct loads cannot read in place (odd leading dimensions, an M/N-contiguous
# extent off the 16-byte grid) or carrying a load transform, copied, the 128-wide tiles on the copies
COPIES = [((520, 392, 360), "NN", "f16", "f16", "bias_relu", 1.0, 0.0, 3, "none", "repack AB"),
          ((300, 264, 1000), "NT", "bf16", "f32", "bias", 2.0, -1.0, 1, "none", "repack AB"),
          ((521, 264, 512), "TN", "f16", "f32", "relu", 1.0, 1.0, 0, "none", "repack A (A to K-major)"),
          ((264, 250, 640), "TT", "bf16", "bf16", "none", 0.5, 0.0, 2, "none", "repack AB"),
          ((392, 520, 256), "NN", "f16", "f16", "bias", 1.0, 0.5, 0, "relu", "repack A"),
          ((400, 304, 768), "TN", "bf16", "f32", "bias_relu", 1.0, 0.0, 0, "relu", "repack A (A to K-major)"),
          ((300, 256, 1280), "NT", "i8", "i32", "bias", 1.0, 1.0, 5, "none", "repack AB"),
          ((600, 520, 640), "TN", "i8", "i32", "bias_relu", 1.0, 0.0, 0, "relu", "repack AB (A to K-major)")]


@pytest.mark.parametrize("case", range(len(COPIES)))
def test_fast128_on_copies_exact(case, tile128):
    (M, N, K), lay, ab, cd, epi, alpha, beta, pad, xa, shows = COPIES[case]
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key=(178, case),
                                    ld_pad=pad, transform_a=xa)
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 ") and shows in d, d
    check(p, x, D, reference(p, x), exact=True)


def test_fast128_on_copies_chosen_and_noalloc():
    # the plan's own choice for a mid-size product with an odd leading dimension; the
    # no-allocation run takes its copy from the scratch, with the same result
    p = synth.exact_integer_problem(2048, 2048, 2048, "N", "N", "f16", "f32", "bias_relu", 1.0, 0.5,
                                    key=(179, 0), ld_pad=1)
    x = synth.make_inputs(p)
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi)
    d = pl.describe()
    print(d, flush=True)
    assert d.startswith("gemm_fast_128x128 ") and "repack AB" in d, d
    A, B = to_dev(p.a_store, x["A"]), to_dev(p.b_store, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    outs = []
    for runner in (pl.run, pl.run_noalloc, pl.run_noalloc):
        D = to_dev(p.cd, np.full(p.M * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]))
        runner(A, B, C, D, bias, p.alpha, p.beta)
        torch.cuda.synchronize()
        outs.append(to_host(p.cd, D).reshape(p.M, p.ldc))
    # (the sentinel past column N is a NaN)
    assert np.array_equal(outs[0], outs[1], equal_nan=True) and np.array_equal(outs[1], outs[2], equal_nan=True)
    check(p, x, outs[0], reference(p, x, threads=16), exact=True)


@pytest.mark.parametrize("shared", [False, True])
def test_fast128_on_copies_batched(shared, tile128):
    # a batch whose operands are copied (odd leading dimensions): one copy per product, or one
    # for all when the stride is 0
    M, N, K = 264, 392, 256
    lda, ldb, ldc = K + 1, K + 1, N + 3
    p = synth.exact_integer_problem(M, N, K, "N", "T", "bf16", "f32", "bias", 1.0, 1.0,
                                    key=(180, int(shared)), batch=3, stride_a=M * lda + 8,
                                    stride_b=0 if shared else N * ldb + 5, stride_c=M * ldc + 16,
                                    stride_bias=N)
    p = replace(p, lda=lda, ldb=ldb, ldc=ldc)
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    d = pl.describe()
    print(d, flush=True)
    assert d.startswith("gemm_fast_128x128 ") and "repack AB" in d and "batch 3" in d, d
    ref = reference_batched(p, x)
    for b in range(p.batch):
        off = batch_offset(p, b)
        Db = Df[off: off + p.M * p.ldc].reshape(p.M, p.ldc)
        check(p, x, Db, ref[b], exact=True)


# Seeded draws of shape, layout, type pair, leading-dimension padding per operand, pointer offset
# and load transforms on the 128x128 tiles (read in place, or from the aligned copies): exact
# inputs (small integers; int8 over its whole range with alpha 1), so every case must match the
# oracle bit for bit.
RANDOM_PAIRS = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("i8", "i32")]
RANDOM_SCALARS = [(1.0, 0.0), (2.0, -1.0), (-0.5, 0.5), (1.0, 1.0)]


@pytest.mark.parametrize("case", range(40))
def test_fast128_random_shapes_exact(case, tile128):
    rng = np.random.default_rng(np.random.SeedSequence([181, case]))
    ab, cd = RANDOM_PAIRS[case % len(RANDOM_PAIRS)]
    lay = LAYOUTS[int(rng.integers(4))]
    M, N = (int(v) for v in rng.integers(16, 700, size=2))
    K = int(rng.integers(128 if ab == "i8" else 64, 700))
    epi = ["none", "relu", "bias", "bias_relu"][int(rng.integers(4))]
    xa, xb = ("relu" if rng.random() < 0.25 else "none" for _ in range(2))
    if ab == "i8":
        beta = float(rng.integers(2))
        p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, beta,
                          a_dist=("int", -128, 127), b_dist=("int", -128, 127), c_dist=("int", -1000, 1000),
                          bias_dist=("int", -(1 << 20), 1 << 20), key=(182, case),
                          transform_a=xa, transform_b=xb)
    else:
        alpha, beta = RANDOM_SCALARS[int(rng.integers(4))]
        p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key=(182, case),
                                        transform_a=xa, transform_b=xb)
    pa, pb, pc = (int(v) for v in rng.integers(0, 10, size=3))
    p = replace(p, lda=p.lda + pa, ldb=p.ldb + pb, ldc=p.ldc + pc)
    offset = int(rng.integers(2))
    x = synth.make_inputs(p)
    D, pl = run(p, x, offset=offset)
    d = pl.describe()
    print(p.label(), "lda", p.lda, "ldb", p.ldb, "ldc", p.ldc, "offset", offset, "->", d, flush=True)
    assert d.startswith("gemm_fast_128x128 "), d
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("case", range(3))
def test_fast128_split_chosen_exact(case):
    # the plan's own choice: fewer 128x128 tiles than CUs and at least 48 slabs of K
    (M, N, K), lay, ab, cd, epi, alpha, beta = [((600, 600, 4096), "NT", "f16", "f16", "bias_relu", 1.0, 0.0),
                                                ((768, 768, 3072), "TN", "bf16", "f32", "bias", 1.0, 1.0),
                                                ((384, 1040, 8192), "TT", "f16", "f32", "relu", 0.5, -0.5)][case]
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key=(185, case))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d
    check(p, x, D, reference(p, x, threads=16), exact=True)


# (M, N, K, layout, ab, cd, epilogue, alpha, beta, ld_pad, pointer offset, what the description
# must show): the K split of the 128x128 tiles on aligned copies (odd leading dimensions, M/N
# off the 16-byte grid, a pointer off it at run time), A stored transposed copied K-major
SPLIT_COPIES = [((512, 520, 3072), "NN", "f16", "f16", "bias_relu", 1.0, 0.0, 1, 0, "repack AB"),
                ((300, 264, 6144), "NT", "bf16", "f32", "bias", 2.0, -1.0, 3, 0, "repack AB"),
                ((768, 770, 3072), "TN", "f16", "f16", "relu", 1.0, 1.0, 0, 0, "repack B"),
                ((770, 768, 3072), "TN", "f16", "f32", "bias", 0.5, 0.5, 0, 0, "repack A (A to K-major)"),
                ((600, 528, 6144), "NN", "i8", "i32", "bias", 1.0, 1.0, 1, 0, "repack AB"),
                ((768, 768, 3072), "TN", "bf16", "bf16", "bias_relu", 1.0, 0.0, 0, 1, ""),
                ((520, 600, 4096), "NT", "f16", "f32", "none", 1.0, 0.0, 0, 1, "")]


@pytest.mark.parametrize("case", range(len(SPLIT_COPIES)))
def test_fast128_split_on_copies_exact(case):
    (M, N, K), lay, ab, cd, epi, alpha, beta, pad, offset, shows = SPLIT_COPIES[case]
    if ab == "i8":
        p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, beta,
                          a_dist=("int", -128, 127), b_dist=("int", -128, 127), c_dist=("int", -1000, 1000),
                          bias_dist=("int", -(1 << 20), 1 << 20), key=(186, case))
        if pad:
            p = replace(p, lda=p.lda + pad, ldb=p.ldb + pad, ldc=p.ldc + pad)
    else:
        p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key=(186, case),
                                        ld_pad=pad)
    x = synth.make_inputs(p)
    D, pl = run(p, x, offset=offset)
    d = pl.describe()
    print(f"{p.label()} offset {offset} -> {d}", flush=True)
    assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d and shows in d, d
    check(p, x, D, reference(p, x, threads=16), exact=True)
