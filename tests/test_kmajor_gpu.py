"""GPU parity of the transposed copy of A (A stored transposed, B not): A is copied into
K-contiguous rows and the fast kernel of the non-transposed layout runs on the copy.  Every case
uses exact-integer inputs, so the result must equal the oracle's bit for bit whatever the
summation order: ragged M, N and K, an A that must be copied anyway (odd leading dimension), a B
copied too, int8, the K split, batches with a shared and a strided A, the load transform carried
by the copy, and the no-allocation entry point (including a copy too large for its scratch,
where the plan reads A in place instead)."""
import numpy as np
import pytest
import torch

import synth
import tiled_gemm_epilogues_amd as tge
from gpu_helpers import (FORCE, check, reference, reference_batched, run, run_batched, sentinel,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (M, N, K, ab, cd, epi, alpha, beta, ld_pad, what the description must show)
CASES = [((520, 304, 640), "f16", "f16", "bias_relu", 1.0, 0.0, 0, "repack A (A to K-major)"),
         ((520, 300, 640), "f16", "f32", "bias", 2.0, -1.0, 0, "repack AB (A to K-major)"),
         ((1000, 776, 384), "bf16", "f32", "bias", 1.0, -1.0, 0, "repack A (A to K-major)"),
         ((777, 520, 1000), "f16", "f32", "relu", 0.5, 1.0, 3, "repack AB (A to K-major)"),
         ((512, 512, 200), "f16", "f16", "none", 1.0, 0.0, 0, "repack A (A to K-major)"),
         ((600, 528, 640), "i8", "i32", "bias", 1.0, 1.0, 0, "repack A (A to K-major)"),
         ((300, 256, 1280), "i8", "i32", "bias_relu", 1.0, 0.0, 5, "repack AB (A to K-major)"),
         ((257, 264, 129), "bf16", "bf16", "bias_relu", 1.0, 0.0, 1, "repack AB (A to K-major)")]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_kmajor_copy_exact(case, monkeypatch):
    (M, N, K), ab, cd, epi, alpha, beta, pad, shows = CASES[case]
    monkeypatch.setitem(FORCE, "algo", "kmajor")
    p = synth.exact_integer_problem(M, N, K, "T", "N", ab, cd, epi, alpha, beta, key=(160, case),
                                    ld_pad=pad)
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} -> {d}", flush=True)
    assert "gemm_fast_256x256 " in d and shows in d, d
    check(p, x, D, reference(p, x), exact=True)


def test_kmajor_matches_in_place():
    # the same exact-integer product read in place (32x32 schedule) and from the copy
    p = synth.exact_integer_problem(768, 1024, 512, "T", "N", "bf16", "f32", "bias", 1.0, 0.5,
                                    key=(161, 0))
    x = synth.make_inputs(p)
    outs = []
    for algo in ("fast", "kmajor"):
        pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi, algo=algo)
        D, _ = run(p, x, plan=pl)
        print(pl.describe(), flush=True)
        assert ("K-major" in pl.describe()) == (algo == "kmajor"), pl.describe()
        outs.append(D)
    assert np.array_equal(outs[0], outs[1])
    check(p, x, outs[1], reference(p, x), exact=True)


def test_kmajor_with_k_split(monkeypatch):
    # few tiles and a long K: the split chunks read the transposed copy along K
    monkeypatch.setitem(FORCE, "algo", "kmajor")
    p = synth.exact_integer_problem(512, 2048, 8192, "T", "N", "f16", "f32", "bias_relu", 1.0, 0.0,
                                    key=(162, 0))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    d = pl.describe()
    print(d, flush=True)
    assert " ksplit " in d and "K-major" in d, d
    check(p, x, D, reference(p, x, threads=16), exact=True)


@pytest.mark.parametrize("shared", [False, True])
def test_kmajor_batch(shared, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "kmajor")
    M, N, K = 300, 264, 320
    p = synth.exact_integer_problem(M, N, K, "T", "N", "f16", "f16", "bias", 1.0, 1.0,
                                    key=(163, int(shared)), batch=3,
                                    stride_a=0 if shared else K * M + 5, stride_b=K * N + 8,
                                    stride_c=M * N + 16, stride_bias=N)
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    print(pl.describe(), flush=True)
    assert "K-major" in pl.describe() and "batch 3" in pl.describe(), pl.describe()
    ref = reference_batched(p, x)
    for b in range(p.batch):
        Db = Df[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)
        check(p, x, Db, ref[b], exact=True)


@pytest.mark.parametrize("ab", ["f16", "i8"])
def test_kmajor_copy_carries_the_load_transform(ab, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "kmajor")
    cd = "i32" if ab == "i8" else "f16"
    p = synth.exact_integer_problem(400, 512, 384, "T", "N", ab, cd, "bias", 1.0, 0.0, key=(164, 0 if ab == "f16" else 1),
                                    transform_a="relu")
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    print(pl.describe(), flush=True)
    assert "K-major" in pl.describe() and "relu-in A" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def _noalloc_pair(p, x, algo):
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi, algo=algo)
    A, B = to_dev(p.a_store, x["A"]), to_dev(p.b_store, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    outs = []
    for runner in (pl.run, pl.run_noalloc, pl.run_noalloc):
        D = to_dev(p.cd, np.full(p.M * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]))
        runner(A, B, C, D, bias, p.alpha, p.beta)
        torch.cuda.synchronize()
        outs.append(to_host(p.cd, D).reshape(p.M, p.ldc))
    return pl, outs


@pytest.mark.parametrize("big", [False, True])
def test_kmajor_noalloc(big):
    # small: the copy comes from the scratch; big: A's copy (8192 x 4352 fp16 = 71 MB) exceeds
    # the 64 MiB scratch, so the no-allocation run reads A in place
    M, N, K = (8192, 256, 4352) if big else (1024, 768, 1024)
    p = synth.exact_integer_problem(M, N, K, "T", "N", "f16", "f32", "bias_relu", 1.0, 0.5,
                                    key=(165, int(big)))
    x = synth.make_inputs(p)
    pl, outs = _noalloc_pair(p, x, "kmajor")
    print(pl.describe(), flush=True)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    check(p, x, outs[1], reference(p, x, threads=16), exact=True)
