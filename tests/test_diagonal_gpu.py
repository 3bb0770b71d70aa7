"""GPU parity of diagonal operands (gemm_operand_t GEMM_OPERAND_DIAGONAL: the operand is the
vector of a square diagonal matrix; each output element takes its one product) against the
oracle, bit-exact on exact-integer inputs: diagonal A, B or both, every type pair, ragged edges,
the dense operand in both layouts (row and transposed streaming kernels), with C, bias,
transforms and a batch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import check, reference, reference_batched, run, run_batched

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


PAIRS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
         ("i8", "i32")]
# (which, M, N, op of the dense operand)
SHAPES = [("A", 1000, 776, "N"), ("A", 257, 129, "T"), ("B", 776, 1000, "N"), ("B", 130, 257, "T"),
          ("AB", 300, 300, "N"), ("A", 128, 64, "N")]


def _problem(which, M, N, op, ab, cd, key, **kw):
    K = M if "A" in which else N
    if "A" in which and "B" in which:
        K = M
    kinds = dict(kind_a="diagonal" if "A" in which else "dense",
                 kind_b="diagonal" if "B" in which else "dense")
    lay = ("N" + op) if "A" in which else (op + "N")
    if ab == "i8":
        return synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", "bias_relu", 1.0, 1.0,
                             a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                             c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                             key=key, name="exact_int", **kinds, **kw)
    return synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, "bias_relu", 2.0, -1.0,
                                       key, **kinds, **kw)


@pytest.mark.parametrize("shape", range(len(SHAPES)))
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_diagonal_exact(pair, shape):
    which, M, N, op = SHAPES[shape]
    ab, cd = PAIRS[pair]
    p = _problem(which, M, N, op, ab, cd, (140, pair * 8 + shape))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "_diag" in pl.describe() and f"diag {which}" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def test_diagonal_with_transforms():
    p = _problem("A", 600, 520, "T", "f16", "f16", (141, 0), transform_a="relu",
                 transform_b="relu", transform_c="relu")
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    check(p, x, D, reference(p, x), exact=True)


def test_diagonal_batched():
    p = _problem("B", 264, 300, "N", "bf16", "f32", (142, 0), batch=3)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "batch 3" in pl.describe()
    ref = reference_batched(p, x)
    for b in range(p.batch):
        Db = D[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)[:, : p.N]
        assert np.array_equal(oracle.decode("f32", Db), ref[b])


def test_diagonal_full_size_random():
    p = synth.diag_fp16()[0]
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    for r0, r1 in [(0, 96), (4000, 4064), (8128, 8192)]:
        check(p, x, D, reference(p, x, rows=(r0, r1)), rows=slice(r0, r1))


# odd leading dimensions and operand pointers one element off alignment, tiny and one-tile
# shapes, through both streaming kernels
EDGE = [("A", 333, 517, "N", 3), ("A", 333, 517, "T", 1), ("B", 517, 333, "N", 5),
        ("B", 517, 333, "T", 7), ("AB", 65, 65, "N", 1), ("A", 1, 1, "N", 0), ("B", 1, 9, "T", 0),
        ("A", 64, 64, "T", 0)]


@pytest.mark.parametrize("ab,cd", [("f16", "f32"), ("bf16", "bf16"), ("i8", "i32"), ("f32", "f32")])
@pytest.mark.parametrize("case", range(len(EDGE)))
def test_diagonal_odd_layouts_and_unaligned(case, ab, cd):
    which, M, N, op, pad = EDGE[case]
    p = _problem(which, M, N, op, ab, cd, (143, case))
    p.lda += pad; p.ldb += pad; p.ldc += pad
    x = synth.make_inputs(p)
    ref = reference(p, x)
    for off in (0, 1):
        D, pl = run(p, x, offset=off)
        assert ("gemm_diag_cols" in pl.describe()) == (op == "T" and which != "AB"), pl.describe()
        check(p, x, D, ref, exact=True)


def test_diagonal_batched_transposed_dense():
    p = _problem("A", 200, 136, "T", "f16", "f16", (144, 0), batch=2)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "gemm_diag_cols" in pl.describe() and "batch 2" in pl.describe()
    ref = reference_batched(p, x)
    for b in range(p.batch):
        Db = D[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)[:, : p.N]
        assert np.array_equal(oracle.decode("f16", Db), oracle.decode("f16", oracle.round_to("f16", ref[b])))
