"""GPU parity of strided-batched plans (gemm_plan_create_batched) against the oracle's batched
product: every product bit-exact on exact-integer inputs, through the fast, general and skinny
kernels, with padded, shared (zero) and per-product strides; the gaps between products of D are
never written."""
import numpy as np
import pytest
import torch

import oracle
import synth
from dataclasses import replace
from gpu_helpers import FORCE, check, reference_batched, run_batched, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_exact(p, Dflat, ref):
    for b in range(p.batch):
        Db = Dflat[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)
        if p.cd == "i32":
            assert np.array_equal(Db[:, : p.N].astype(np.int64), ref[b]), f"product {b}"
        else:
            want = oracle.round_to(p.cd, ref[b])
            assert np.array_equal(oracle.decode(p.cd, Db[:, : p.N]), oracle.decode(p.cd, want)), \
                f"product {b}"
        # padding columns of D and the gap after the product keep the sentinel
        if p.ldc > p.N:
            assert (Db[:, p.N:].view(np.uint32 if p.cd in ("f32", "i32") else np.uint16) ==
                    np.array(sentinel(p.cd)).view(np.uint32 if p.cd in ("f32", "i32") else np.uint16)).all()
        gap_end = (b + 1) * p.stride_c if b + 1 < p.batch else Dflat.size
        gap = Dflat[b * p.stride_c + p.M * p.ldc: gap_end]
        if gap.size:
            raw = gap.view(np.uint32 if p.cd in ("f32", "i32") else np.uint16)
            assert (raw == np.array(sentinel(p.cd)).view(raw.dtype)).all(), f"gap after product {b}"


CASES = [
    # (kernel, M, N, K, layout, ab, cd, epi, alpha, beta, batch, stride overrides)
    ("fast", 264, 520, 200, "NN", "f16", "f16", "bias_relu", 1.0, 0.0, 3,
     dict(stride_a=264 * 200 + 64, stride_b=0)),
    ("fast", 304, 264, 192, "TT", "bf16", "f32", "bias", 2.0, -1.0, 2, dict(stride_bias=0)),
    ("fast", 512, 272, 256, "NT", "i8", "i32", "bias_relu", 1.0, 1.0, 3, dict()),
    ("fast", 256, 256, 128, "TN", "f16", "f32", "relu", 0.5, 0.0, 4, dict(stride_a=0)),
    ("general", 200, 136, 150, "NT", "f32", "f32", "bias", 1.0, 0.5, 3, dict(stride_c=200 * 136 + 7)),
    ("general", 130, 70, 90, "TN", "bf16", "bf16", "relu", -1.0, 0.0, 2, dict()),
    ("skinny", 16, 520, 320, "NN", "f16", "f16", "bias_relu", 1.0, 0.0, 4, dict(stride_b=0)),
    ("skinny", 33, 200, 1024, "NT", "bf16", "f32", "bias", 1.0, -0.5, 2, dict()),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_batched_exact(case, monkeypatch):
    kern, M, N, K, lay, ab, cd, epi, alpha, beta, batch, strides = CASES[case]
    monkeypatch.setitem(FORCE, "algo", kern)
    if ab == "i8":
        p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, beta,
                          a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                          c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                          key=(120, case), name="exact_int", batch=batch, **strides)
    else:
        p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta,
                                        key=(120, case), batch=batch, **strides)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert f"gemm_{kern}" in pl.describe() or (kern == "general" and "gemm_mfma" in pl.describe()), \
        pl.describe()
    assert f"batch {batch}" in pl.describe()
    _check_exact(p, D, reference_batched(p, x))


@pytest.mark.parametrize("mode", ["fast", "staged"])
def test_batched_unaligned_stride(mode, monkeypatch):
    # a stride that moves product 1 off 16-byte alignment: the direct loads cannot read A in
    # place; A is copied per product into aligned rows (fast) or the register-staged kernel runs
    monkeypatch.setitem(FORCE, "algo", mode)
    p = synth.exact_integer_problem(256, 264, 128, "N", "N", "f16", "f16", "bias", 1.0, 0.0,
                                    key=(121, 0), batch=2, stride_a=256 * 128 + 3)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    if mode == "staged":
        assert "gemm_fast_256x256_rs" in pl.describe(), pl.describe()
    else:
        assert "gemm_fast_256x256 " in pl.describe() and "repack A " in pl.describe() + " ", pl.describe()
    _check_exact(p, D, reference_batched(p, x))


@pytest.mark.parametrize("lay", ["NN", "TN", "NT", "TT"])
def test_batched_repack_shared_and_strided(lay, monkeypatch):
    # odd leading dimensions and strides, B shared by every product (stride 0, one copy) and
    # a per-product bias; bf16 -> f32 with beta over three products
    monkeypatch.setitem(FORCE, "algo", "fast")
    M, N, K = 300, 261, 200
    ra = (M if lay[0] == "N" else K)
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], "bf16", "f32", "bias_relu", 1.0, 1.0,
                                    key=(123, ["NN", "TN", "NT", "TT"].index(lay)), ld_pad=1,
                                    batch=3, stride_b=0, stride_bias=N)
    p = replace(p, stride_a=ra * p.lda + 5, stride_c=M * p.ldc + 3)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "gemm_fast_256x256 " in pl.describe() and "repack AB" in pl.describe(), pl.describe()
    _check_exact(p, D, reference_batched(p, x))


def test_batch_of_zero_launches_nothing():
    import tiled_gemm_epilogues_amd as tge
    pl = tge.Plan(64, 64, 64, "N", "N", ab="f16", cd="f16", batch=0, stride_c=64 * 64)
    D = torch.full((64 * 64,), 3.0, dtype=torch.float16, device="cuda")
    A = torch.ones(64 * 64, dtype=torch.float16, device="cuda")
    pl.run(A, A, None, D)
    torch.cuda.synchronize()
    assert bool((D == 3.0).all())


# ---- two batch modes ---------------------------------------------------------------------------

# (M, N, K, layout, ab, cd, algo, kernel expected, batch, batch2, odd stride2 of A)
TWO_MODE = [(520, 304, 320, "NN", "f16", "f16", "fast", "gemm_fast_256x256 ", 2, 3, False),
            (304, 264, 200, "TN", "bf16", "f32", "fast", "gemm_fast_256x256 ", 3, 2, False),
            (264, 520, 384, "NT", "i8", "i32", "fast", "gemm_fast_256x256 ", 2, 2, False),
            (520, 300, 320, "NN", "f16", "f32", "fast", "gemm_fast_256x256_rs", 2, 2, True),
            (150, 97, 70, "TT", "f16", "f16", "general", "gemm_mfma", 3, 2, True),
            (16, 1024, 2048, "NN", "f16", "f16", "auto", "gemm_skinny", 2, 2, False),
            (100, 60, 33, "NT", "f32", "f32", "auto", "gemm_mfma", 2, 3, False)]


@pytest.mark.parametrize("case", range(len(TWO_MODE)))
def test_two_mode_batch_exact(case, monkeypatch):
    """Product (b1, b2) at b1 * stride + b2 * stride2: A moves with b1 only (broadcast along b2),
    B with b2 only, C/D and the bias with both (D blocks b2-major), exact against the oracle on
    every product."""
    M, N, K, lay, ab, cd, algo, kern, b1, b2, odd = TWO_MODE[case]
    monkeypatch.setitem(FORCE, "algo", algo)
    rows_a = M if lay[0] == "N" else K
    rows_b = K if lay[1] == "N" else N
    base = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, "bias_relu",
                                       1.0 if ab == "i8" else 2.0, 1.0 if ab == "i8" else -1.0,
                                       key=(160, case))
    if ab == "i8":
        base = replace(base, alpha=1.0, beta=1.0)
    sc = M * base.ldc + 24
    p = replace(base, batch=b1, stride_a=rows_a * base.lda + (1 if odd else 0), stride_b=0,
                stride_c=sc, stride_bias=N, batch2=b2, stride2_a=0,
                stride2_b=rows_b * base.ldb + 16, stride2_c=b1 * sc + 40, stride2_bias=b1 * N)
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    d = pl.describe()
    print(f"{p.label()} batch {b1}x{b2} -> {d}", flush=True)
    assert kern in d and f"batch {b1}x{b2}" in d, d
    ref = reference_batched(p, x).reshape(b1, b2, M, N)   # product b1 * batch2 + b2
    for i in range(b1):
        for j in range(b2):
            o = i * p.stride_c + j * p.stride2_c
            Db = Df[o: o + M * p.ldc].reshape(M, p.ldc)
            check(p, x, Db, ref[i, j], exact=True)
