"""GPU parity of the load transforms (gemm_plan_create_desc: ReLU on op(A), op(B) and C as they
are loaded) against the oracle: bit-exact on exact-integer inputs (which hold negatives, so
every transform changes the result) through the fast, general and skinny kernels, in every
layout, alone and together with a strided batch.  The fast path is covered both ways: the
operand transforms applied by the aligned copy before the kernel ("fast"), and fused into the
kernel's loads ("staged": no copies)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import FORCE, check, reference, reference_batched, run, run_batched

pytestmark = pytest.mark.gpu

LAYOUTS = ["NN", "NT", "TN", "TT"]
XFORMS = [("relu", "none", "none"), ("none", "relu", "relu"), ("relu", "relu", "relu"),
          ("none", "none", "relu")]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _problem(M, N, K, lay, ab, cd, epi, alpha, beta, key, xf, **kw):
    if ab == "i8":
        p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, beta,
                          a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                          c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                          key=key, name="exact_int", transform_a=xf[0], transform_b=xf[1],
                          transform_c=xf[2], **kw)
    else:
        p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key,
                                        transform_a=xf[0], transform_b=xf[1], transform_c=xf[2],
                                        **kw)
    return p


CASES = [
    # kernel, M, N, K, ab, cd, epi, alpha, beta
    ("fast", 304, 520, 200, "f16", "f16", "bias_relu", 1.0, 1.0),
    ("fast", 512, 264, 128, "bf16", "f32", "bias", 2.0, -1.0),
    ("fast", 304, 528, 208, "i8", "i32", "bias", 1.0, 1.0),
    ("staged", 304, 520, 200, "f16", "f16", "bias_relu", 1.0, 1.0),
    ("staged", 512, 264, 128, "bf16", "f32", "bias", 2.0, -1.0),
    ("staged", 304, 528, 208, "i8", "i32", "bias", 1.0, 1.0),
    ("general", 200, 136, 150, "f32", "f32", "relu", 0.5, 0.5),
    ("general", 130, 70, 90, "bf16", "bf16", "bias", -1.0, 1.0),
    ("general", 96, 80, 300, "i8", "i32", "bias_relu", 1.0, 1.0),
]


@pytest.mark.parametrize("xf", range(len(XFORMS)))
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_transforms_exact(case, lay, xf, monkeypatch):
    kern, M, N, K, ab, cd, epi, alpha, beta = CASES[case]
    monkeypatch.setitem(FORCE, "algo", kern)
    i = case * 16 + LAYOUTS.index(lay) * 4 + xf
    p = _problem(M, N, K, lay, ab, cd, epi, alpha, beta, (130, i), XFORMS[xf])
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert ("gemm_fast" in pl.describe()) == (kern != "general"), pl.describe()
    assert "relu-in" in pl.describe()
    # the copy applies the operand transforms (aligned operands are copied only for them)
    copies = kern == "fast" and "relu" in XFORMS[xf][:2]
    assert (" repack " in pl.describe()) == copies, pl.describe()
    check(p, x, D, reference(p, x), exact=True)
    # a pointer one element off: copied (and transformed) at run time, or register-staged
    D2, _ = run(p, x, offset=1)
    check(p, x, D2, reference(p, x), exact=True)


@pytest.mark.parametrize("xf", range(len(XFORMS)))
@pytest.mark.parametrize("lb", ["N", "T"])
def test_transforms_skinny_exact(lb, xf, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = _problem(33, 200, 1024, "N" + lb, "f16", "f32", "bias_relu", 1.0, -0.5,
                 (131, xf * 2 + (lb == "T")), XFORMS[xf])
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_skinny" in pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("lb", ["N", "T"])
def test_transforms_skinny_split_k_exact(lb, monkeypatch):
    # K long enough that the skinny plan splits it over workgroups: the operand transforms run
    # in the splitting kernel, the C transform in the finishing one
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = _problem(33, 200, 4096, "N" + lb, "f16", "f32", "bias_relu", 1.0, -0.5,
                 (133, lb == "T"), ("relu", "relu", "relu"))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_skinny" in pl.describe() and "ksplit" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def test_transforms_random_within_tolerance(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    p = synth.Problem(1000, 776, 1000, "N", "N", "f16", "f16", "bias_relu", 1.0, 0.5,
                      key=(132, 0), transform_a="relu", transform_b="none", transform_c="relu")
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_fast" in pl.describe()
    check(p, x, D, reference(p, x))


def test_transforms_with_a_batch(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    p = _problem(264, 264, 192, "NN", "f16", "f16", "bias", 1.0, 1.0, (133, 0),
                 ("relu", "relu", "relu"), batch=3, stride_b=0)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "gemm_fast" in pl.describe() and "batch 3" in pl.describe()
    ref = reference_batched(p, x)
    import oracle
    for b in range(p.batch):
        Db = D[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)[:, : p.N]
        assert np.array_equal(oracle.decode("f16", Db), oracle.decode("f16", oracle.round_to("f16", ref[b])))
