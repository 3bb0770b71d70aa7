"""GPU parity of complex and dual GEMM (fp16 parts, fp32 accumulation) against the oracle's
four-real-product definition: bit-exact on integer parts in every layout, with ragged edges, K
tails, beta, both output types and a batch.  Both routes are covered: the complex kernel
(interleaved in global memory, split in LDS) and, where the real fast kernels apply, the real
product on 2 x 2 blocks (the algorithm "fast" makes small shapes take it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_gemm_epilogues_amd as tge
from gpu_helpers import FORCE

pytestmark = pytest.mark.gpu
LAYOUTS = ["NN", "NT", "TN", "TT"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(raw):
    flat = np.ascontiguousarray(raw).reshape(-1)
    if flat.dtype == np.uint16:
        return torch.from_numpy(flat.view(np.int16).copy()).to("cuda")
    return torch.from_numpy(flat.copy()).to("cuda")


def _run(p, x):
    part = synth.PART[p.cd]
    nD = (max(p.batch - 1, 0) * p.stride_c + p.M * p.ldc) * 2
    D = torch.full((nD,), float("nan"), dtype=torch.float16 if part == "f16" else torch.float32,
                   device="cuda")
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, "none",
                  batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c,
                  algo=FORCE["algo"])
    C = _dev(x["C"]) if x["C"] is not None else None
    pl.run(_dev(x["A"]), _dev(x["B"]), C, D, None, p.alpha, p.beta)
    torch.cuda.synchronize()
    Dh = D.cpu()
    Dh = Dh.view(torch.int16).numpy().view(np.uint16) if part == "f16" else Dh.numpy()
    return Dh, pl


def _check(p, Dh, ref, b=0):
    part = synth.PART[p.cd]
    Db = Dh[2 * b * p.stride_c: 2 * (b * p.stride_c + p.M * p.ldc)].reshape(p.M, p.ldc, 2)[:, : p.N]
    want = ref if part == "f32" else oracle.decode("f16", oracle.round_to("f16", ref))
    assert np.array_equal(oracle.decode(part, Db), want)


SHAPES = [(300, 200, 100), (129, 257, 65), (64, 64, 64), (1, 1, 1), (257, 3, 190), (5, 300, 64)]
TYPES = [("cf16", "cf32"), ("cf16", "cf16"), ("df16", "df32"), ("df16", "df16")]


def _route_ok(pl, ab, mode, K):
    d = pl.describe()
    if mode == "fast" and 2 * K >= 64:
        return "as real 2x2 blocks: gemm_fast" in d
    return ("gemm_dual" if ab.startswith("d") else "gemm_complex") in d


@pytest.mark.parametrize("mode", ["auto", "fast"])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("types", range(len(TYPES)))
def test_complex_dual_exact(types, lay, shape, mode, monkeypatch):
    if mode == "fast":
        monkeypatch.setitem(FORCE, "algo", "fast")
    ab, cd = TYPES[types]
    M, N, K = SHAPES[shape]
    i = types * 100 + LAYOUTS.index(lay) * 10 + shape
    alpha, beta = [(1.0, 0.0), (2.0, -1.0), (-0.5, 0.5), (1.0, 1.0)][i % 4]
    p = synth.Problem(M, N, K, lay[0], lay[1], ab, cd, "none", alpha, beta,
                      a_dist=("int", -4, 4), b_dist=("int", -4, 4), c_dist=("int", -8, 8),
                      key=(150, i), lda=(K if lay[0] == "N" else M) + (i % 3),
                      ldb=(N if lay[1] == "N" else K) + (i % 2))
    x = synth.make_inputs(p)
    Dh, pl = _run(p, x)
    assert _route_ok(pl, ab, mode, K), pl.describe()
    ref = oracle.gemm_pair(M, N, K, lay[0], lay[1], x["A"], p.lda, x["B"], p.ldb, ab, C=x["C"],
                           ldc=p.ldc, cd=cd, alpha=alpha, beta=beta)
    _check(p, Dh, ref)


@pytest.mark.parametrize("mode", ["auto", "fast"])
def test_complex_batched(mode, monkeypatch):
    if mode == "fast":
        monkeypatch.setitem(FORCE, "algo", "fast")
    p = synth.Problem(200, 136, 96, "N", "T", "cf16", "cf32", "none", 1.0, 0.0,
                      a_dist=("int", -4, 4), b_dist=("int", -4, 4), key=(151, 0), batch=3,
                      stride_b=0)
    x = synth.make_inputs(p)
    Dh, pl = _run(p, x)
    assert "batch 3" in pl.describe()
    assert _route_ok(pl, "cf16", mode, p.K), pl.describe()
    A = x["A"].reshape(-1, 2)
    for b in range(p.batch):
        ref = oracle.gemm_pair(p.M, p.N, p.K, "N", "T", A[b * p.stride_a:], p.lda, x["B"], p.ldb,
                               "cf16")
        _check(p, Dh, ref, b)


def test_complex_random_full_size_rows():
    for p in synth.complex_fp16():
        x = synth.make_inputs(p)
        Dh, pl = _run(p, x)
        D = Dh.reshape(p.M, p.ldc, 2)
        for r0 in (0, 2000, p.M - 3):
            ref = oracle.gemm_pair(p.M, p.N, p.K, "N", "N", x["A"], p.lda, x["B"], p.ldb, p.ab,
                                   rows=(r0, r0 + 3))
            got = D[r0:r0 + 3, : p.N]
            # parts U[-1,1]: |products| <= 1, normalised error as for the real GEMM
            err = np.max(np.abs(got - ref)) / p.K
            assert err <= 2e-3, err


@pytest.mark.parametrize("lay", LAYOUTS)
def test_complex_as_real_blocks_batched_strided(lay, monkeypatch):
    # dual numbers through the real product: per-product A (odd stride), shared B, beta, fp16
    # output, odd leading dimensions
    monkeypatch.setitem(FORCE, "algo", "fast")
    M, N, K = 130, 72, 90
    ra = M if lay[0] == "N" else K
    p = synth.Problem(M, N, K, lay[0], lay[1], "df16", "df16", "none", 2.0, -1.0,
                      a_dist=("int", -4, 4), b_dist=("int", -4, 4), c_dist=("int", -8, 8),
                      key=(152, LAYOUTS.index(lay)), batch=2, stride_b=0,
                      lda=(K if lay[0] == "N" else M) + 1, ldb=(N if lay[1] == "N" else K) + 3)
    from dataclasses import replace
    p = replace(p, stride_a=ra * p.lda + 3)
    x = synth.make_inputs(p)
    Dh, pl = _run(p, x)
    assert "as real 2x2 blocks: gemm_fast" in pl.describe() and "batch 2" in pl.describe(), pl.describe()
    A = x["A"].reshape(-1, 2)
    for b in range(p.batch):
        ref = oracle.gemm_pair(M, N, K, lay[0], lay[1], A[b * p.stride_a:], p.lda, x["B"], p.ldb,
                               "df16", C=x["C"].reshape(-1, 2)[b * p.stride_c:], ldc=p.ldc,
                               cd="df16", alpha=p.alpha, beta=p.beta)
        _check(p, Dh, ref, b)


def test_complex_as_real_blocks_graph_capture(monkeypatch):
    # a first run inside a capture has no workspace for the rewritten operands: the complex
    # kernel runs; after an eager run, captured runs take the real product; every replay, with
    # eager work between, gives the exact result
    monkeypatch.setitem(FORCE, "algo", "fast")
    p = synth.Problem(200, 136, 96, "T", "N", "cf16", "cf32", "none", 1.0, 0.0,
                      a_dist=("int", -4, 4), b_dist=("int", -4, 4), key=(153, 0))
    x = synth.make_inputs(p)
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, "none",
                  algo=FORCE["algo"])
    assert "as real 2x2 blocks" in pl.describe(), pl.describe()
    ref = oracle.gemm_pair(p.M, p.N, p.K, "T", "N", x["A"], p.lda, x["B"], p.ldb, "cf16")
    A, B = _dev(x["A"]), _dev(x["B"])
    D = torch.zeros(p.M * p.ldc * 2, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(s):
        g0 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g0, stream=s):
            pl.run(A, B, None, D, None, 1.0, 0.0)
        graphs.append(g0)
        pl.run(A, B, None, D, None, 1.0, 0.0)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=s):
            pl.run(A, B, None, D, None, 1.0, 0.0)
        graphs.append(g1)
    torch.cuda.synchronize()
    for _ in range(3):
        for g in graphs:
            D.zero_()
            g.replay()
            torch.cuda.synchronize()
            _check(p, D.cpu().numpy(), ref)
            pl.run(A, B, None, D, None, 1.0, 0.0)
            torch.cuda.synchronize()
