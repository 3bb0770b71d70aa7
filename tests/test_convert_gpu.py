"""GPU parity of the type-converting load transforms (an operand stored as fp32 or int8 and
converted to the 16-bit input type as it is loaded) against the oracle, through the C ABI:

* exact-integer values on every layout and on each route the converted product can take (the
  fast kernel, its K split, the skinny kernel, the general kernel, a batch), bit for bit;
* the rounding itself: op(A) times the identity returns the converted operand, which must equal
  the oracle's round-to-nearest-even conversion bit for bit (random values and ties);
* random values within the normalised tolerance; the no-allocation entry point."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_gemm_epilogues_amd as tge
from gpu_helpers import (FORCE, check, reference, reference_batched, run, run_batched, sentinel,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu

LAYOUTS = ["NN", "NT", "TN", "TT"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (shape, ab, cd, transform_a, transform_b, algo, expected kernel)
ROUTES = [((520, 300, 640), "f16", "f16", "from_f32", "none", "fast", "gemm_fast_256x256"),
          ((1000, 776, 384), "bf16", "f32", "none", "from_i8", "fast", "gemm_fast_256x256"),
          ((2048, 2048, 8192), "f16", "f32", "from_i8", "from_f32", "auto", "ksplit"),
          ((16, 4096, 4096), "f16", "f16", "none", "from_f32", "auto", "gemm_skinny"),
          ((200, 136, 150), "bf16", "bf16", "from_f32", "from_i8", "auto", "gemm_fast_128x128"),
          ((200, 136, 150), "bf16", "bf16", "from_f32", "from_i8", "general", "gemm_mfma"),
          ((77, 45, 33), "f16", "f32", "from_i8", "from_i8", "auto", "gemm_mfma")]


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("case", range(len(ROUTES)))
def test_converted_operands_exact(case, lay, monkeypatch):
    (M, N, K), ab, cd, ta, tb, algo, kern = ROUTES[case]
    if kern == "gemm_skinny" and lay[0] == "T":
        pytest.skip("the skinny kernel reads A not transposed")
    monkeypatch.setitem(FORCE, "algo", algo)
    i = case * 4 + LAYOUTS.index(lay)
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, "bias_relu", 2.0, -1.0,
                                    key=(150, i), ld_pad=i % 3, transform_a=ta, transform_b=tb)
    x = synth.make_inputs(p)
    assert x["A"].dtype == synth.RAW_NP[p.a_store] and x["B"].dtype == synth.RAW_NP[p.b_store]
    D, pl = run(p, x)
    d = pl.describe()
    print(f"{p.label()} {ta}/{tb} -> {d}", flush=True)
    if lay == "NN":
        assert kern in d, d
    assert ("convert A" in d) == (ta != "none") and ("convert B" in d) == (tb != "none"), d
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("route", ["fast", "auto"])
def test_conversion_rounds_to_nearest_even(ab, route, monkeypatch):
    # op(A) I = the converted A: D (fp32) must equal the oracle's conversion of every element,
    # ties to even included (a tie at every 7th element)
    monkeypatch.setitem(FORCE, "algo", route)
    M, K = 300, 256
    g = np.random.default_rng(151)
    A = g.normal(0, 100, (M, K)).astype(np.float32)
    step = 2.0 ** -11 if ab == "f16" else 2.0 ** -8     # half an ulp of values in [1, 2)
    ties = (1 + np.arange(M * K) % 64 / 64.0 + step).astype(np.float32).reshape(M, K)
    A[::7] = ties[::7] * np.sign(g.normal(size=(len(A[::7]), K))).astype(np.float32)
    eye = np.eye(K, dtype=np.float32)
    I = eye.astype(np.float16).view(np.uint16) if ab == "f16" else \
        (eye.view(np.uint32) >> 16).astype(np.uint16)
    p = synth.Problem(M, K, K, "N", "N", ab, "f32", "none", 1.0, 0.0, transform_a="from_f32")
    x = {"A": A, "B": I, "C": None, "bias": None}
    D, pl = run(p, x)
    want = oracle.convert_to(ab, A.astype(np.float64))
    got = D[:, :K].astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} differ ({pl.describe()}), first {bad[0]}: " \
                          f"{got[tuple(bad[0])]} vs {want[tuple(bad[0])]} from {A[tuple(bad[0])]}"


@pytest.mark.parametrize("lay", LAYOUTS)
def test_converted_random_within_tolerance(lay):
    M, N, K = 1024, 1040, 2048
    i = LAYOUTS.index(lay)
    p = synth.Problem(M, N, K, lay[0], lay[1], "bf16", "bf16", "bias_relu", 1.0, 0.0,
                      a_dist=("normal", 1.0), b_dist=("int", -128, 127), key=(152, i),
                      transform_a="from_f32", transform_b="from_i8")
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    print(f"{p.label()} -> {pl.describe()}", flush=True)
    err = check(p, x, D, reference(p, x))
    print(f"normalised error {err:.3e}", flush=True)


def test_converted_batch_shared_and_strided():
    # A stored fp32 and shared by the products (stride 0); B stored int8 per product
    p = synth.exact_integer_problem(300, 264, 320, "N", "T", "f16", "f16", "bias", 1.0, 1.0,
                                    key=(153, 0), batch=3, stride_a=0, stride_b=264 * 320 + 7,
                                    stride_c=300 * 264 + 16, stride_bias=264,
                                    transform_a="from_f32", transform_b="from_i8")
    x = synth.make_inputs(p)
    Df, pl = run_batched(p, x)
    print(pl.describe(), flush=True)
    ref = reference_batched(p, x)
    for b in range(p.batch):
        Db = Df[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)
        check(p, x, Db, ref[b], exact=True)


def test_converted_noalloc_two_calls():
    for i, (M, N, K) in enumerate([(1024, 768, 1024), (300, 200, 136)]):
        p = synth.exact_integer_problem(M, N, K, "T", "N", "bf16", "f32", "bias_relu", 1.0, 0.5,
                                        key=(154, i), transform_a="from_i8", transform_b="from_f32")
        x = synth.make_inputs(p)
        pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                      transform_a=p.transform_a, transform_b=p.transform_b, algo="fast")
        A, B = to_dev(p.a_store, x["A"]), to_dev(p.b_store, x["B"])
        C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
        outs = []
        for runner in (pl.run, pl.run_noalloc):
            D = to_dev(p.cd, np.full(p.M * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]))
            runner(A, B, C, D, bias, p.alpha, p.beta)
            torch.cuda.synchronize()
            outs.append(to_host(p.cd, D).reshape(p.M, p.ldc))
        assert np.array_equal(outs[0], outs[1])
        check(p, x, outs[1], reference(p, x), exact=True)
