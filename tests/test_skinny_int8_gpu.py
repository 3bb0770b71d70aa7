"""GPU parity of the memory-bound kernel for short int8 products (M <= 64 pinned, up to 32 rows
by the plan's own choice; B stored transposed: the N x K weights layout): 64-column blocks with
and without the K split (int32 partial sums, the integer finishing kernel), 16-column blocks,
every epilogue with beta 0 and 1, load transforms on A, B and C, batches, and the plan's own
choice.  int8 -> int32 is exact, so every comparison with the oracle is bit for bit."""
import pytest
import torch

import synth
from gpu_helpers import (FORCE, batch_offset, check, reference, reference_batched, run,
                         run_batched)

pytestmark = pytest.mark.gpu

EPIS = ["none", "relu", "bias", "bias_relu"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _int8(M, N, K, epi, beta, key, **kw):
    return synth.Problem(M, N, K, "N", "T", "i8", "i32", epi, 1.0, beta,
                         a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                         c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                         key=key, **kw)


# (M, N, K): M across the four row tiles (1..64), N off the 64- and 16-column blocks, K from one
# 64-deep chunk to long ones (the plan splits K where the blocks are too few)
SHAPES = [(1, 64, 64), (5, 1000, 2048), (16, 4096, 4096), (17, 520, 1024), (33, 4096, 8192),
          (48, 776, 640), (64, 8192, 4096), (64, 200, 128)]


@pytest.mark.parametrize("case", range(len(SHAPES)))
@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_skinny_int8_exact(case, beta, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    M, N, K = SHAPES[case]
    p = _int8(M, N, K, EPIS[(case + int(beta)) % 4], beta, key=(190, 2 * case + int(beta)))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert d.startswith("gemm_skinny"), d
    check(p, x, D, reference(p, x), exact=True)


def test_skinny_int8_chosen_split_and_narrow():
    # the plan's own choice: 64-column blocks with K split (int32 partial sums and the integer
    # finishing kernel), and 16-column blocks
    for j, ((M, N, K), shows) in enumerate([((32, 8192, 4096), " ksplit "), ((32, 4096, 8192), " ksplit "),
                                            ((16, 4096, 4096), "gemm_skinny_m16_n16")]):
        p = _int8(M, N, K, "bias_relu", 1.0, key=(191, j))
        x = synth.make_inputs(p)
        D, pl = run(p, x)
        d = pl.describe()
        print(d, flush=True)
        assert d.startswith("gemm_skinny") and shows in d, d
        check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("xf", [("relu", "none", "none"), ("none", "relu", "relu"), ("relu", "relu", "relu")])
def test_skinny_int8_transforms(xf, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    for j, (M, N, K) in enumerate([(16, 4096, 4096), (40, 1000, 2048)]):
        p = _int8(M, N, K, "bias", 1.0, key=(192, j), transform_a=xf[0], transform_b=xf[1],
                  transform_c=xf[2])
        x = synth.make_inputs(p)
        D, pl = run(p, x)
        print(pl.describe(), flush=True)
        assert pl.describe().startswith("gemm_skinny"), pl.describe()
        check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("narrow", [False, True])
def test_skinny_int8_batched(narrow, monkeypatch):
    # a batch runs one kernel, unsplit (the integer finishing kernel takes one product)
    monkeypatch.setitem(FORCE, "algo", "skinny")
    M, N, K = (16, 4096, 1024) if narrow else (40, 520, 2048)
    p = _int8(M, N, K, "bias_relu", 1.0, key=(193, int(narrow)), batch=3, stride_a=M * K + 64,
              stride_b=0 if narrow else N * K, stride_c=M * N + 16, stride_bias=N)
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    d = pl.describe()
    print(d, flush=True)
    assert d.startswith("gemm_skinny") and "batch 3" in d and "ksplit" not in d, d
    ref = reference_batched(p, x)
    for b in range(p.batch):
        off = batch_offset(p, b)
        Db = Df[off: off + p.M * p.ldc].reshape(p.M, p.ldc)
        check(p, x, Db, ref[b], exact=True)


def test_skinny_int8_b_not_transposed_takes_another_kernel(monkeypatch):
    # B stored K x N: not this kernel; the result is the same
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = synth.Problem(16, 1024, 2048, "N", "N", "i8", "i32", "bias", 1.0, 1.0,
                      a_dist=("int", -128, 127), b_dist=("int", -128, 127), c_dist=("int", -1000, 1000),
                      bias_dist=("int", -(1 << 20), 1 << 20), key=(194, 0))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert not pl.describe().startswith("gemm_skinny"), pl.describe()
    check(p, x, D, reference(p, x), exact=True)
