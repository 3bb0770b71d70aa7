"""gemm_run_noalloc (the entry point that allocates nothing) against gemm_run, through the C ABI:
on every route that needs scratch (skinny split-K, the fast kernel's K split, aligned operand
copies, complex numbers as real blocks) and one that needs none, two calls in a row, the second
with a smaller problem, each equal bit for bit to gemm_run's result on the same inputs and
exact against the oracle (exact-integer inputs); a captured graph of no-allocation runs replays
to the same result; a run beyond the scratch is rejected."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_gemm_epilogues_amd as tge
from gpu_helpers import check, reference, sentinel, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(p, x, offset=0):
    A, B = to_dev(p.ab, x["A"], offset), to_dev(p.ab, x["B"], offset)
    C = to_dev(p.cd, x["C"], offset) if x["C"] is not None else None
    bias = to_dev(p.bias_dt, x["bias"], offset) if x["bias"] is not None else None
    return A, B, C, bias


def _ptr(t):
    return None if t is None else t.data_ptr()


def _both(p, plan, x, offset=0):
    """(D from gemm_run, D from gemm_run_noalloc) on the same device inputs, raw pointers
    through the C ABI on torch's current stream."""
    A, B, C, bias = _inputs(p, x, offset)
    outs = []
    for fn in (tge.gemm_run, tge.gemm_run_noalloc):
        D = to_dev(p.cd, np.full(p.M * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]), offset)
        st = fn(plan.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(bias), p.alpha, p.beta,
                torch.cuda.current_stream().cuda_stream)
        assert st == tge.STATUS_SUCCESS, tge.gemm_status_string(st)
        torch.cuda.synchronize()
        outs.append(to_host(p.cd, D).reshape(p.M, p.ldc))
    return outs


def _plan(p, algo="auto"):
    return tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                    algo=algo)


# (first, second) problem of each route: the second smaller, so that it runs on scratch that
# still holds the first call's data
ROUTES = {
    "skinny_split": (((64, 4096, 8192), "NN", "f16", "f16"), ((16, 2048, 4096), "NN", "f16", "f16"),
                     "gemm_skinny", " ksplit "),
    "fast_split": (((2560, 2560, 8192), "NT", "f16", "f16"), ((2048, 3072, 4096), "NN", "bf16", "f32"),
                   "gemm_fast_256x256", " ksplit "),
    "fast128_split": (((2048, 2048, 4096), "NN", "f16", "f16"), ((1024, 1024, 8192), "NT", "bf16", "f32"),
                      "gemm_fast_128x128", " ksplit "),
    "short_int8_split": (((64, 8192, 4096), "NT", "i8", "i32"), ((16, 4096, 2048), "NN", "i8", "i32"),
                         "gemm_fast_128x128", " ksplit "),
    "repack": (((4095, 3073, 2047), "NN", "bf16", "f32"), ((1001, 777, 513), "TN", "bf16", "f32"),
               "gemm_fast_256x256", "repack"),
    "no_scratch": (((1024, 1024, 1024), "NN", "f16", "f16"), ((512, 384, 256), "TT", "f16", "f16"),
                   "", ""),
}


def _exact(shape, lay, ab, cd, key):
    M, N, K = shape
    if ab == "i8":
        return synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", "bias_relu", 1.0, 1.0,
                             a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                             c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                             key=key, name="exact_int")
    return synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, "bias_relu", 2.0, -1.0,
                                       key=key)


@pytest.mark.parametrize("route", sorted(ROUTES))
def test_noalloc_matches_gemm_run_two_calls(route):
    first, second, kern, marker = ROUTES[route]
    for i, (shape, lay, ab, cd) in enumerate((first, second)):
        p = _exact(shape, lay, ab, cd, key=(140, sorted(ROUTES).index(route), i))
        algo = "auto"
        if route == "repack":
            p.lda += 2       # odd leading dimensions: the operands are copied first
            p.ldb += 3
            algo = "fast"
        x = synth.make_inputs(p)
        pl = _plan(p, algo)
        d = pl.describe()
        print(f"{route} call {i}: {p.label()} -> {d}", flush=True)
        assert kern in d and marker in d + " ", d
        Dr, Dn = _both(p, pl, x)
        assert np.array_equal(Dr, Dn), f"{route} call {i}: gemm_run_noalloc differs from gemm_run"
        check(p, x, Dn, reference(p, x), exact=True)


def test_noalloc_complex_as_real_blocks_two_calls():
    for i, (M, N, K) in enumerate([(512, 384, 640), (200, 136, 96)]):
        p = synth.Problem(M, N, K, "T", "N", "cf16", "cf32", "none", 1.0, 0.0,
                          a_dist=("int", -4, 4), b_dist=("int", -4, 4), key=(141, i))
        x = synth.make_inputs(p)
        pl = _plan(p, algo="fast")
        assert "as real 2x2 blocks" in pl.describe(), pl.describe()
        A = torch.from_numpy(np.ascontiguousarray(x["A"]).reshape(-1).view(np.int16).copy()).cuda()
        B = torch.from_numpy(np.ascontiguousarray(x["B"]).reshape(-1).view(np.int16).copy()).cuda()
        outs = []
        for fn in (tge.gemm_run, tge.gemm_run_noalloc):
            D = torch.full((M * N * 2,), float("nan"), dtype=torch.float32, device="cuda")
            st = fn(pl.handle, A.data_ptr(), B.data_ptr(), None, D.data_ptr(), None, 1.0, 0.0,
                    torch.cuda.current_stream().cuda_stream)
            assert st == tge.STATUS_SUCCESS, tge.gemm_status_string(st)
            torch.cuda.synchronize()
            outs.append(D.cpu().numpy())
        assert np.array_equal(outs[0], outs[1])
        ref = oracle.gemm_pair(M, N, K, "T", "N", x["A"], p.lda, x["B"], p.ldb, "cf16")
        assert np.array_equal(outs[1].reshape(M, N, 2).astype(np.float64), ref)


def test_noalloc_graph_capture_replays():
    # after one eager call on the device (which finds the scratch address), a run inside a
    # capture needs no allocation: the split route is captured as is, and every replay, with
    # eager work between, gives the exact result
    p = _exact((1024, 1024, 8192), "NN", "f16", "f32", key=(142, 0))
    x = synth.make_inputs(p)
    pl = _plan(p)
    assert " ksplit " in pl.describe(), pl.describe()
    A, B, C, bias = _inputs(p, x)
    D = torch.zeros(p.M * p.ldc, dtype=torch.float32, device="cuda")
    pl.run_noalloc(A, B, C, D, bias, p.alpha, p.beta)      # first call on the device: eager
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pl.run_noalloc(A, B, C, D, bias, p.alpha, p.beta, stream=s)
    torch.cuda.synchronize()
    want = reference(p, x)
    for _ in range(3):
        D.zero_()
        g.replay()
        torch.cuda.synchronize()
        check(p, x, to_host(p.cd, D).reshape(p.M, p.ldc), want, exact=True)
        pl.run(A, B, C, D, bias, p.alpha, p.beta)          # eager work between the replays
        torch.cuda.synchronize()


def test_noalloc_rejects_beyond_the_scratch():
    p = synth.Problem(8192, 8192, 8192, "N", "N", "f16", "f16", "none", 1.0, 0.0, lda=8193)
    pl = _plan(p)
    A = torch.empty(8192 * 8193, dtype=torch.float16, device="cuda")
    B = torch.empty(8192 * 8192, dtype=torch.float16, device="cuda")
    D = torch.empty(8192 * 8192, dtype=torch.float16, device="cuda")
    with pytest.raises(tge.GemmError, match="SCRATCH_LIMIT"):
        pl.run_noalloc(A, B, None, D)
