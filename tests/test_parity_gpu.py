"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

* exact-integer inputs (every fp32 partial sum exact, so D must equal RNE(ref) bit for bit) on
  every type pair, layout and tile size, at shapes spanning several tiles with ragged M/N/K;
* random inputs within the normalised tolerance on every pair and layout;
* edge cases: K = 0, single rows/columns, beta = 0 with NaN in C, in-place C == D, padded and
  odd leading dimensions, unaligned pointers, guard bands, determinism;
* the workloads at full size on sampled outputs (every product of a batch in full), plus
  properties that hold everywhere.
"""
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (FORCE, batch_offset, check, check_points, normaliser, reference, reference_batched, run,
                         run_batched)

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
         ("i8", "i32")]
LAYOUTS = ["NN", "NT", "TN", "TT"]
BK = {"f32": 32, "f16": 64, "bf16": 64, "i8": 128}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _exact(M, N, K, lay, ab, cd, epi, alpha, beta, key, ld_pad=0):
    if ab == "i8":
        p = synth.Problem(M, N, K, lay[0], lay[1], "i8", "i32", epi, 1.0, 1.0 if beta else 0.0,
                          a_dist=("int", -128, 127), b_dist=("int", -128, 127),
                          c_dist=("int", -1000, 1000), bias_dist=("int", -(1 << 20), 1 << 20),
                          key=key, name="exact_int")
        if ld_pad:
            p.lda += ld_pad; p.ldb += ld_pad; p.ldc += ld_pad
        return p
    return synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta, key,
                                       ld_pad=ld_pad)


EPIS = ["none", "relu", "bias", "bias_relu"]
SCALARS = [(1.0, 0.0), (2.0, -1.0), (-0.5, 0.5), (1.0, 1.0)]


@pytest.mark.parametrize("tile", [256, 128, 64])
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab,cd", PAIRS)
def test_exact_integer_all_tiles(ab, cd, lay, tile, monkeypatch):
    monkeypatch.setitem(FORCE, "tile", tile)
    i = PAIRS.index((ab, cd)) * 4 + LAYOUTS.index(lay)
    M, N, K = 2 * tile + 7, tile + 33, 2 * BK[ab] + 5
    epi = EPIS[i % 4]
    alpha, beta = SCALARS[(i // 4 + tile) % 4]
    p = _exact(M, N, K, lay, ab, cd, epi, alpha, beta, key=(100, i))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert f"tile {tile}x{tile}" in pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab,cd", PAIRS)
def test_random_within_tolerance(ab, cd, lay):
    i = PAIRS.index((ab, cd)) * 4 + LAYOUTS.index(lay)
    M, N, K = 333, 517, 301
    if ab == "i8":
        p = _exact(M, N, K, lay, ab, cd, "bias_relu", 1.0, 1.0, key=(101, i))
    else:
        p = synth.Problem(M, N, K, lay[0], lay[1], ab, cd, "bias_relu", 1.5, -0.5, key=(101, i))
    x = synth.make_inputs(p)
    D, _ = run(p, x)
    ref = reference(p, x)
    err = check(p, x, D, ref)
    if cd != "i32":
        # beyond the tolerance: the error should be what the output rounding (half an ulp,
        # relative 2^-8 bf16, 2^-11 f16, 2^-24 f32) and fp32 accumulation (about K * 2^-24 of
        # the normaliser) explain, far below it
        half_ulp = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}[cd]
        bound = np.abs(ref).max() * half_ulp / normaliser(p, x) + 4 * p.K * 2.0 ** -24
        assert err <= bound, f"error {err:.2e} above rounding + accumulation bound {bound:.2e}"


SHAPES = [(1, 1, 1), (1, 64, 64), (64, 1, 64), (5, 7, 3), (31, 33, 17), (64, 64, 64),
          (65, 63, 129), (127, 129, 1), (200, 3, 300), (3, 200, 300), (257, 255, 200)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("bf16", "f32"), ("i8", "i32"), ("f32", "f32")])
def test_shape_sweep_exact(ab, cd, shape):
    M, N, K = shape
    for j, lay in enumerate(LAYOUTS):
        p = _exact(M, N, K, lay, ab, cd, "bias_relu", 2.0, -1.0, key=(102, SHAPES.index(shape), j))
        x = synth.make_inputs(p)
        D, _ = run(p, x)
        check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("ab,cd", PAIRS)
def test_k_zero(ab, cd):
    p = _exact(70, 90, 0, "NN", ab, cd, "bias_relu", 2.0, -1.0, key=(103, 0))
    x = synth.make_inputs(p)
    D, _ = run(p, x)
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("ab,cd", PAIRS)
def test_padded_and_odd_leading_dims_unaligned_pointers(ab, cd):
    for j, (pad, off) in enumerate([(8, 0), (3, 0), (1, 1), (5, 3)]):
        p = _exact(150, 130, 170, ["NN", "NT", "TN", "TT"][j], ab, cd, "bias", 0.5, 2.0,
                   key=(104, j), ld_pad=pad)
        x = synth.make_inputs(p)
        D, _ = run(p, x, offset=off, d_rows_extra=3)
        check(p, x, D, reference(p, x)[:, :], rows=slice(0, p.M), exact=True)
        # guard bands: padding columns and rows past M keep the sentinel
        tail = D[:, p.N:]
        below = D[p.M:, :]
        for blk in (tail, below):
            if blk.size:
                if cd == "i32":
                    assert (blk == -0x5A5A5A5A).all()
                elif cd == "f32":
                    assert np.isnan(blk).all()
                else:
                    assert (blk == {"f16": 0x7E00, "bf16": 0x7FC0}[cd]).all()


@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("bf16", "f32"), ("f32", "f32")])
def test_beta_zero_does_not_read_c(ab, cd):
    p = synth.Problem(100, 120, 80, "N", "T", ab, cd, "relu", 1.0, 0.0, key=(105, 0))
    x = synth.make_inputs(p)
    x["C"] = np.full((p.M, p.ldc), np.nan if cd == "f32" else 0x7E00,
                     dtype=synth.RAW_NP[cd])
    D, _ = run(p, x)
    x["C"] = None
    check(p, x, D, reference(p, x))


@pytest.mark.parametrize("ab,cd", [("f16", "f32"), ("bf16", "bf16"), ("i8", "i32")])
def test_in_place_c_equals_d(ab, cd):
    p = _exact(140, 260, 96, "TN", ab, cd, "bias_relu", 1.0, 1.0, key=(106, 0))
    x = synth.make_inputs(p)
    D, _ = run(p, x, c_is_d=True)
    check(p, x, D, reference(p, x), exact=True)


def test_deterministic_and_stream():
    p = synth.Problem(1000, 1100, 900, "T", "N", "f16", "f16", "bias_relu", key=(107, 0))
    x = synth.make_inputs(p)
    s = torch.cuda.Stream()
    D1, pl = run(p, x)
    D2, _ = run(p, x, plan=pl, stream=s)
    assert np.array_equal(D1, D2)


def test_nn_equals_tt_of_transposed_problem():
    # (XY)^T = Y^T X^T: the TT problem on the same stored arrays gives the transposed result
    p = synth.Problem(300, 200, 250, "N", "N", "bf16", "f32", "none", key=(108, 0))
    x = synth.make_inputs(p)
    D, _ = run(p, x)
    q = synth.Problem(200, 300, 250, "T", "T", "bf16", "f32", "none", lda=p.ldb, ldb=p.lda,
                      key=(108, 0))
    y = {"A": x["B"], "B": x["A"], "C": None, "bias": None}
    DT, _ = run(q, y)
    np.testing.assert_allclose(DT, D.T, rtol=0, atol=1e-5)


# ---- the workloads at full size -----------------------------------------------------------

# complex / dual workloads have their own full-size check (test_complex_gpu.py)
FULL = [(name, i) for name, fn in synth.WORKLOADS.items() for i, q in enumerate(fn())
        if q.ab not in synth.PART]


def _host_threads():
    """The host cores this process may use (the CPU share of the box), for the oracle."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap)) if cap and cap.isdigit() else n)


@pytest.mark.parametrize("name,idx", FULL)
def test_workload_full_output(name, idx):
    """Every output element of every workload at its full size against the oracle (int8 bit for
    bit, floats within the normalised tolerance), in the launch configuration the bench times."""
    p = synth.WORKLOADS[name]()[idx]
    x = synth.make_inputs(p)
    threads = _host_threads()
    if p.batch != 1 or p.batch2 != 1:
        Df, pl = run_batched(p, x)
        print(f"{p.label()} -> {pl.describe()}", flush=True)
        ref = reference_batched(p, x)
        errs = []
        for b in range(len(ref)):
            o = batch_offset(p, b)
            Db = Df[o: o + p.M * p.ldc].reshape(p.M, p.ldc)
            errs.append(check(p, x, Db, ref[b]))
        print(f"[full] {p.label()}: products {len(ref)} x rows {p.M} checked, max normalised "
              f"error {max(errs):.3e}", flush=True)
        return
    D, pl = run(p, x)
    print(f"{p.label()} -> {pl.describe()}", flush=True)
    ref = reference(p, x, threads=threads)
    err = check(p, x, D, ref)
    print(f"[full] {p.label()}: rows {p.M} of {p.M} checked, "
          f"{'bit-exact' if p.cd == 'i32' else f'max normalised error {err:.3e}'}", flush=True)
    Dv = D[:, : p.N]
    if p.relu:
        assert (synth_decode(p.cd, Dv) >= 0).all()


# Exact-integer inputs at full size: every fp32 partial sum is exact, so D must equal RNE(ref)
# on every element.  Unlike the normalised tolerance, this sees a dropped or repeated K slab, a
# misplaced tile or a stale round anywhere in the multi-round grids, the partial last round and
# the streaming-store epilogue that only the full-size launches exercise.
EXACT_FULL = [((8192, 8192, 8192), "NN", "f16", "f16", "bias_relu", 1.0, 0.0),
              ((5000, 5000, 5000), "TN", "bf16", "f32", "none", 2.0, -1.0),
              ((5000, 5000, 5000), "NT", "bf16", "f32", "bias", 0.5, 1.0),
              ((4095, 3073, 2047), "TT", "bf16", "bf16", "relu", 1.0, -0.5),
              ((8192, 4096, 16384), "NN", "f16", "f16", "bias_relu", 1.0, 0.0),
              ((8192, 16384, 4096), "NT", "f16", "f16", "bias_relu", 1.0, 0.0)]


@pytest.mark.parametrize("case", range(len(EXACT_FULL)))
def test_exact_integer_full_size(case):
    (M, N, K), lay, ab, cd, epi, alpha, beta = EXACT_FULL[case]
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], ab, cd, epi, alpha, beta,
                                    key=(120, case))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    print(f"{p.label()} -> {pl.describe()}", flush=True)
    assert "gemm_fast_256x256" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x, threads=_host_threads()), exact=True)
    print(f"[full] {p.label()}: rows {M} of {M} bit-exact", flush=True)


def synth_decode(cd, raw):
    import oracle
    return oracle.decode(cd, raw) if cd != "i32" else raw


# ---- the fast 256x256 path (16-bit inputs) ----------------------------------------------------

# shapes that meet the fast kernel's preconditions (16-byte aligned leading dimensions, M and N
# multiples of 8) with ragged tiles, K tails and one-tile edge cases
FAST_SHAPES = [(256, 256, 64), (304, 520, 200), (512, 264, 128), (264, 8, 72), (8, 304, 192),
               (640, 512, 320), (1000, 776, 1000)]


@pytest.mark.parametrize("shape", FAST_SHAPES)
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_fast_path_exact(ab, cd, lay, shape, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    M, N, K = shape
    i = LAYOUTS.index(lay) + 4 * FAST_SHAPES.index(shape)
    epi = EPIS[i % 4]
    alpha, beta = SCALARS[i % 4]
    p = _exact(M, N, K, lay, ab, cd, epi, alpha, beta, key=(109, i))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_fast" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("lay", LAYOUTS)
def test_fast_path_random_and_unaligned_fallback(lay, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    p = synth.Problem(776, 1024, 576, lay[0], lay[1], "f16", "f16", "bias_relu", 1.0, 0.0,
                      key=(110, LAYOUTS.index(lay)))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_fast" in pl.describe()
    ref = reference(p, x)
    check(p, x, D, ref)
    # a pointer offset by one element: the operands are copied to aligned rows at run time and
    # the same kernel runs on the copies; same result
    D2, _ = run(p, x, offset=1)
    check(p, x, D2, ref)


# ---- the memory-bound path for M <= 64 (16-bit inputs, A not transposed) ----------------------

# (K split over workgroups, with the split-K workspace, for (33, 200, 1024), (16, 4096, 4096),
# (16, 1000, 2048), (7, 4104, 8192) and (64, 8192, 1024))
# (with B transposed, (16, 4096, 4096), (5, 3072, 1024) and (16, 4000, 2048) take the
# 16-column variant: one round of 192-256 workgroups, no k split; the last has a partial block)
SKINNY_SHAPES = [(1, 16, 32), (5, 40, 64), (16, 520, 320), (17, 64, 96), (33, 200, 1024),
                 (48, 24, 160), (64, 4096, 128), (16, 4096, 4096), (16, 1000, 2048),
                 (7, 4104, 8192), (64, 8192, 1024), (5, 3072, 1024), (16, 4000, 2048)]


@pytest.mark.parametrize("shape", SKINNY_SHAPES)
@pytest.mark.parametrize("lb", ["N", "T"])
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_skinny_path_exact(ab, cd, lb, shape, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    M, N, K = shape
    i = SKINNY_SHAPES.index(shape) * 2 + (lb == "T")
    p = _exact(M, N, K, "N" + lb, ab, cd, EPIS[i % 4], *SCALARS[i % 4], key=(111, i))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_skinny" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def test_skinny_split_k_repeatable_and_graph_safe(monkeypatch):
    # the split-K counters reset themselves: repeated runs, a second plan of the same shape,
    # and graph replays after a first eager run give the same bits
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = _exact(16, 1000, 2048, "NN", "f16", "f32", "bias_relu", 2.0, -1.0, key=(118, 0))
    x = synth.make_inputs(p)
    D0, pl = run(p, x)
    assert "gemm_skinny" in pl.describe() and "ksplit" in pl.describe(), pl.describe()
    check(p, x, D0, reference(p, x), exact=True)
    for _ in range(3):
        D1, _ = run(p, x, plan=pl)
        assert np.array_equal(D0, D1)
    # graph capture of later runs (the first run allocated the workspace outside the capture)
    from gpu_helpers import to_dev, to_host
    A, B = to_dev(p.ab, x["A"]), to_dev(p.ab, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    D = torch.zeros(p.M * p.ldc, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pl.run(A, B, C, D, bias, p.alpha, p.beta)   # eager, on the capture stream
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(2):
                pl.run(A, B, C, D, bias, p.alpha, p.beta)
    torch.cuda.synchronize()
    for _ in range(3):
        D.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(p.cd, D).reshape(p.M, p.ldc), D0)


def test_skinny_split_k_batched(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = synth.exact_integer_problem(16, 520, 2048, "N", "T", "bf16", "bf16", "bias", 1.0, 1.0,
                                    key=(119, 0), batch=3, stride_bias=520)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "gemm_skinny" in pl.describe() and "ksplit" in pl.describe(), pl.describe()
    ref = reference_batched(p, x)
    import oracle
    for b in range(p.batch):
        Db = D[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)[:, : p.N]
        assert np.array_equal(oracle.decode(p.cd, Db), oracle.decode(p.cd, oracle.round_to(p.cd, ref[b])))


def test_skinny_narrow_blocks_batched(monkeypatch):
    # three products of 64 sixteen-column blocks each: one round of 192 narrow workgroups
    monkeypatch.setitem(FORCE, "algo", "skinny")
    p = synth.exact_integer_problem(13, 1024, 1024, "N", "T", "f16", "f32", "bias_relu", 2.0, -1.0,
                                    key=(126, 0), batch=3, stride_bias=1024)
    x = synth.make_inputs(p)
    D, pl = run_batched(p, x)
    assert "gemm_skinny_m16_n16" in pl.describe() and "batch 3" in pl.describe(), pl.describe()
    ref = reference_batched(p, x)
    import oracle
    for b in range(p.batch):
        Db = D[b * p.stride_c: b * p.stride_c + p.M * p.ldc].reshape(p.M, p.ldc)[:, : p.N]
        assert np.array_equal(oracle.decode(p.cd, Db), oracle.decode(p.cd, oracle.round_to(p.cd, ref[b])))


def test_skinny_ineligible_shapes_fall_back(monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "skinny")
    # K not a multiple of 32, and A transposed: the general kernel runs, same results
    for j, (lay, K) in enumerate([("NN", 100), ("TN", 64)]):
        p = _exact(16, 128, K, lay, "f16", "f16", "bias_relu", 1.0, 0.0, key=(112, j))
        x = synth.make_inputs(p)
        D, pl = run(p, x)
        assert "gemm_skinny" not in pl.describe()
        check(p, x, D, reference(p, x), exact=True)


# int8 through the fast path: K >= 128 and leading dimensions / M,N multiples of 16
FAST_SHAPES_I8 = [(256, 256, 128), (304, 528, 208), (512, 272, 256), (272, 16, 144),
                  (16, 304, 384), (640, 512, 640), (1008, 784, 1008)]


@pytest.mark.parametrize("shape", FAST_SHAPES_I8)
@pytest.mark.parametrize("lay", LAYOUTS)
def test_fast_path_int8_exact(lay, shape, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "fast")
    M, N, K = shape
    i = LAYOUTS.index(lay) + 4 * FAST_SHAPES_I8.index(shape)
    epi = ["none", "relu", "bias", "bias_relu"][i % 4]
    p = _exact(M, N, K, lay, "i8", "i32", epi, 1.0, 1.0 if i % 3 == 0 else 0.0, key=(113, i))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert "gemm_fast" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


# ---- layouts the direct loads cannot take: repacked copies, or the register-staged variant -----
# (M, N, K, leading-dimension padding): odd leading dimensions, M/N off the 16-byte grid with the
# tile crossing the edge, an M/N-contiguous extent of exactly one chunk, K tails.  Mode "fast"
# copies such operands into aligned, zero-padded rows and runs the direct-load kernel on the
# copies; mode "staged" runs the register-staged variant on the operands in place.
RS_SHAPES = [(300, 261, 200, 1), (257, 9, 136, 3), (9, 263, 72, 0), (520, 515, 333, 5),
             (264, 264, 64, 1), (16, 16, 128, 7)]
VE = {"f16": 8, "bf16": 8, "i8": 16}


def _direct_ok(p, pad):
    e = {"f16": 2, "bf16": 2, "i8": 1}[p.ab]
    return ((p.lda * e) % 16 == 0 and (p.ldb * e) % 16 == 0 and
            (p.op_a == "N" or p.M % VE[p.ab] == 0) and (p.op_b == "T" or p.N % VE[p.ab] == 0))


@pytest.mark.parametrize("mode", ["fast", "staged"])
@pytest.mark.parametrize("shape", RS_SHAPES)
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"),
                                   ("bf16", "f32"), ("i8", "i32")])
def test_fast_unaligned_layouts_exact(ab, cd, lay, shape, mode, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", mode)
    M, N, K, pad = shape
    if ab == "i8":
        K *= 2                              # one int8 slab is 128 deep
        if M < VE[ab] or N < VE[ab]:
            M, N = max(M, 16), max(N, 16)
    i = LAYOUTS.index(lay) + 4 * RS_SHAPES.index(shape)
    p = _exact(M, N, K, lay, ab, cd, EPIS[i % 4], *SCALARS[(i // 4) % 4], key=(114, i),
               ld_pad=pad)
    x = synth.make_inputs(p)
    print(p.label(), flush=True)
    D, pl = run(p, x)
    if _direct_ok(p, pad):
        want = "gemm_fast_256x256 "
    elif mode == "fast":
        want = "gemm_fast_256x256 "
        assert " repack " in pl.describe(), pl.describe()
    else:
        want = "gemm_fast_256x256_rs"
    assert want in pl.describe() + " ", pl.describe()
    check(p, x, D, reference(p, x), exact=True)
    # unaligned operand pointers: copied (fast) or register-staged at run time, same result
    D2, _ = run(p, x, offset=1)
    check(p, x, D2, reference(p, x), exact=True)


@pytest.mark.parametrize("mode", ["fast", "staged"])
@pytest.mark.parametrize("lay", LAYOUTS)
def test_fast_unaligned_layouts_random(lay, mode, monkeypatch):
    # random data, bf16 -> f32 with bias + ReLU, odd leading dimensions over several tiles
    monkeypatch.setitem(FORCE, "algo", mode)
    p = synth.Problem(777, 1031, 611, lay[0], lay[1], "bf16", "f32", "bias_relu", 1.0, 0.5,
                      key=(115, LAYOUTS.index(lay)))
    p.lda += 1; p.ldb += 3; p.ldc += 1
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    want = "gemm_fast_256x256_rs" if mode == "staged" else "gemm_fast_256x256 "
    assert want in pl.describe(), pl.describe()
    assert (" repack AB" in pl.describe()) == (mode == "fast"), pl.describe()
    check(p, x, D, reference(p, x))


@pytest.mark.parametrize("mode", ["fast", "staged"])
def test_fast_unaligned_layouts_with_transforms(mode, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", mode)
    p = synth.exact_integer_problem(300, 261, 200, "T", "N", "f16", "f32", "bias", 1.0, 1.0,
                                    key=(116, 0), ld_pad=1, transform_a="relu",
                                    transform_b="relu", transform_c="relu")
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    want = "gemm_fast_256x256_rs" if mode == "staged" else "gemm_fast_256x256 "
    assert want in pl.describe() and "relu-in ABC" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("mode", ["fast", "staged"])
def test_fast_extent_below_one_chunk(mode, monkeypatch):
    # N = 5 with B not transposed: no in-bounds 16-byte chunk exists in place.  Copied, B's rows
    # are padded to one whole chunk and the direct-load kernel runs; the register-staged variant
    # cannot take it and the general kernel runs
    monkeypatch.setitem(FORCE, "algo", mode)
    p = _exact(300, 5, 128, "NN", "f16", "f16", "bias", 1.0, 0.0, key=(117, 0))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    if mode == "fast":
        assert "gemm_fast_256x256 " in pl.describe() and "repack B" in pl.describe(), pl.describe()
    else:
        assert "gemm_fast" not in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def test_repack_graph_capture(monkeypatch):
    # a first run inside a capture cannot allocate the copy workspace: it runs the
    # register-staged kernel; after an eager run (which allocates it) captured runs copy the
    # operands; every replay, with eager work between, gives the eager result bit for bit
    monkeypatch.setitem(FORCE, "algo", "fast")
    p = _exact(520, 515, 333, "TN", "f16", "f32", "bias_relu", 2.0, -1.0, key=(122, 0), ld_pad=1)
    x = synth.make_inputs(p)
    ref = reference(p, x)
    from gpu_helpers import to_dev, to_host
    A, B = to_dev(p.ab, x["A"]), to_dev(p.ab, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    import tiled_gemm_epilogues_amd as tge
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                  algo=FORCE["algo"], tile=FORCE["tile"])
    assert "repack AB" in pl.describe(), pl.describe()
    D = torch.zeros(p.M * p.ldc, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(s):
        g0 = torch.cuda.CUDAGraph()                       # no workspace yet: register-staged
        with torch.cuda.graph(g0, stream=s):
            pl.run(A, B, C, D, bias, p.alpha, p.beta)
        graphs.append(g0)
        pl.run(A, B, C, D, bias, p.alpha, p.beta)          # eager: allocates the copies
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=s):
            for _ in range(2):
                pl.run(A, B, C, D, bias, p.alpha, p.beta)
        graphs.append(g1)
    torch.cuda.synchronize()
    D0 = to_host(p.cd, D).reshape(p.M, p.ldc).copy()
    check(p, x, D0, ref, exact=True)
    for _ in range(3):
        for g in graphs:
            D.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_host(p.cd, D).reshape(p.M, p.ldc), D0)
            pl.run(A, B, C, D, bias, p.alpha, p.beta)      # eager work between replays
            torch.cuda.synchronize()


def test_fast_streaming_stores_unaligned_d(monkeypatch):
    # more than one round of 256x256 tiles (17 x 17 = 289 workgroups): interior tiles write D with
    # non-temporal stores; an odd ldc makes those stores unaligned.  C read in place as well.
    monkeypatch.setitem(FORCE, "algo", "fast")
    for j, (cd, pad) in enumerate([("f16", 1), ("f32", 3), ("f16", 0)]):
        p = _exact(4200, 4200, 128, "NN", "f16", cd, "bias_relu", 2.0, -1.0, key=(122, j))
        p.ldc += pad
        x = synth.make_inputs(p)
        print(p.label(), "ldc", p.ldc, flush=True)
        D, pl = run(p, x)
        assert "gemm_fast_256x256 " in pl.describe() + " " and "grid 289" in pl.describe(), pl.describe()
        check(p, x, D, reference(p, x), exact=True)


# ---- randomized shapes through the fast path ----------------------------------------------------
# Seeded draws of shape, layout, type pair, leading-dimension padding per operand, pointer offset
# and route (aligned copies, or register-staged in place): exact-integer inputs, so every case
# must match the oracle bit for bit.
RANDOM_CASES = 48


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_fast_random_shapes_exact(case, monkeypatch):
    rng = np.random.default_rng(np.random.SeedSequence([124, case]))
    pairs = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("i8", "i32")]
    ab, cd = pairs[case % len(pairs)]
    lay = LAYOUTS[int(rng.integers(4))]
    mode = "fast" if case % 3 else "staged"
    monkeypatch.setitem(FORCE, "algo", mode)
    kmin = 128 if ab == "i8" else 64
    M, N = (int(v) for v in rng.integers(16, 700, size=2))
    K = int(rng.integers(kmin, 700))
    epi = EPIS[int(rng.integers(4))]
    alpha, beta = SCALARS[int(rng.integers(4))]
    p = _exact(M, N, K, lay, ab, cd, epi, alpha, beta, key=(125, case))
    pa, pb, pc = (int(v) for v in rng.integers(0, 10, size=3))
    p = replace(p, lda=p.lda + pa, ldb=p.ldb + pb, ldc=p.ldc + pc)
    offset = int(rng.integers(2))
    x = synth.make_inputs(p)
    print(p.label(), "lda", p.lda, "ldb", p.ldb, "ldc", p.ldc, "offset", offset, mode, flush=True)
    D, pl = run(p, x, offset=offset)
    assert "gemm_fast" in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


# ---- the fast kernel's K split (chunks of K as a batch into fp32 partial sums, then the
# finishing kernel) -------------------------------------------------------------------------------
# the algorithm "split" makes small shapes split (any S >= 2); the plan's own rule splits only
# large-K products with few tiles.  Exact-integer inputs: partial sums and their total are exact.
SPLIT_SHAPES = [(300, 264, 1024), (520, 300, 640), (256, 256, 128), (17, 600, 2048),
                (600, 9, 512), (777, 513, 1280)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_fast_k_split_exact(ab, cd, lay, shape, monkeypatch):
    monkeypatch.setitem(FORCE, "algo", "split")
    M, N, K = shape
    i = LAYOUTS.index(lay) + 4 * SPLIT_SHAPES.index(shape)
    p = _exact(M, N, K, lay, ab, cd, EPIS[i % 4], *SCALARS[(i // 4) % 4], key=(127, i))
    if i % 3 == 0:
        p = replace(p, transform_c="relu")          # the C transform runs in the finishing step
    x = synth.make_inputs(p)
    print(p.label(), flush=True)
    D, pl = run(p, x)
    ve = 8
    aligned = ((lay[0] == "N" or M % ve == 0) and (lay[1] == "T" or N % ve == 0))
    if aligned:
        assert "gemm_fast_256x256 " in pl.describe() and " ksplit " in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)
    # an unaligned pointer: the operands are copied and the product runs whole, same result
    D2, _ = run(p, x, offset=1)
    check(p, x, D2, reference(p, x), exact=True)


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("lay", LAYOUTS)
def test_fast_k_split_int8_exact(lay, shape, monkeypatch):
    # int8 -> int32: int32 partial sums, the integer finishing kernel (bias, beta in {0, 1},
    # ReLU); K doubled so that every chunk is a whole int8 slab of 128
    monkeypatch.setitem(FORCE, "algo", "split")
    M, N, K = shape
    K *= 2
    i = LAYOUTS.index(lay) + 4 * SPLIT_SHAPES.index(shape)
    p = _exact(M, N, K, lay, "i8", "i32", EPIS[i % 4], 1.0, 1.0 if i % 2 else 0.0, key=(130, i))
    x = synth.make_inputs(p)
    print(p.label(), flush=True)
    D, pl = run(p, x)
    aligned = ((lay[0] == "N" or M % 16 == 0) and (lay[1] == "T" or N % 16 == 0))
    if aligned:
        assert "gemm_fast_256x256 " in pl.describe() and " ksplit " in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("shape", [(16, 4096, 4096), (5, 1000, 2048), (64, 520, 1024),
                                   (33, 4096, 8192)])
@pytest.mark.parametrize("lay", LAYOUTS)
def test_fast_k_split_short_int8_exact(lay, shape):
    # the plan's own choice for short int8 products: the 128x128 tiles with K split into chunks
    # of 4 slabs or more, int32 partial sums, the integer finishing kernel; bias, beta = 1, ReLU
    M, N, K = shape
    i = LAYOUTS.index(lay) + 4 * [(16, 4096, 4096), (5, 1000, 2048), (64, 520, 1024),
                                  (33, 4096, 8192)].index(shape)
    p = _exact(M, N, K, lay, "i8", "i32", EPIS[i % 4], 1.0, 1.0 if i % 2 else 0.0, key=(131, i))
    x = synth.make_inputs(p)
    print(p.label(), flush=True)
    D, pl = run(p, x)
    if lay == "NT" and M <= 32:
        # B transposed, up to 32 rows: the memory-bound kernel takes it
        assert pl.describe().startswith("gemm_skinny"), pl.describe()
    else:
        assert pl.describe().startswith("gemm_fast_128x128 ") and " ksplit " in pl.describe() + " ", \
            pl.describe()
    check(p, x, D, reference(p, x), exact=True)


@pytest.mark.parametrize("shape", [(16, 4096, 4096), (5, 1000, 2048), (64, 520, 1024)])
@pytest.mark.parametrize("lb", ["N", "T"])
@pytest.mark.parametrize("ab,cd", [("f16", "f16"), ("bf16", "f32")])
def test_fast_k_split_short_transposed_a_exact(ab, cd, lb, shape):
    # short 16-bit products with A transposed (no skinny kernel): the plan's K split over the
    # 128x128 tiles
    M, N, K = shape
    i = (lb == "T") + 2 * [(16, 4096, 4096), (5, 1000, 2048), (64, 520, 1024)].index(shape)
    p = _exact(M, N, K, "T" + lb, ab, cd, EPIS[i % 4], *SCALARS[i % 4], key=(132, i))
    x = synth.make_inputs(p)
    print(p.label(), flush=True)
    D, pl = run(p, x)
    assert pl.describe().startswith("gemm_fast_128x128 ") and " ksplit " in pl.describe(), pl.describe()
    check(p, x, D, reference(p, x), exact=True)


def test_fast_k_split_graph_capture(monkeypatch):
    # no workspace yet inside the first capture: that run is not split; after an eager run the
    # captured runs split; every replay gives the eager result bit for bit
    monkeypatch.setitem(FORCE, "algo", "split")
    p = _exact(520, 300, 640, "NT", "bf16", "f32", "bias_relu", 2.0, -1.0, key=(128, 0))
    x = synth.make_inputs(p)
    ref = reference(p, x)
    from gpu_helpers import to_dev, to_host
    A, B = to_dev(p.ab, x["A"]), to_dev(p.ab, x["B"])
    C, bias = to_dev(p.cd, x["C"]), to_dev(p.bias_dt, x["bias"])
    import tiled_gemm_epilogues_amd as tge
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                  algo=FORCE["algo"], tile=FORCE["tile"])
    assert " ksplit " in pl.describe(), pl.describe()
    D = torch.zeros(p.M * p.ldc, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(s):
        g0 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g0, stream=s):
            pl.run(A, B, C, D, bias, p.alpha, p.beta)
        graphs.append(g0)
        pl.run(A, B, C, D, bias, p.alpha, p.beta)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=s):
            pl.run(A, B, C, D, bias, p.alpha, p.beta)
        graphs.append(g1)
    torch.cuda.synchronize()
    D0 = to_host(p.cd, D).reshape(p.M, p.ldc).copy()
    check(p, x, D0, ref, exact=True)
    for _ in range(3):
        for g in graphs:
            D.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_host(p.cd, D).reshape(p.M, p.ldc), D0)
            pl.run(A, B, C, D, bias, p.alpha, p.beta)
            torch.cuda.synchronize()


@pytest.mark.parametrize("lay", ["NN", "TT"])
def test_fast_k_split_full_size_points(lay):
    # the plan's own choice at 2048 x 2048 x 8192 (64 tiles of 256x256, K split 4 ways) and
    # 2048 x 2048 x 4096 (256 tiles of 128x128, K split in two), random fp16 inputs, bias + ReLU:
    # sampled outputs against the oracle's per-point reference
    K, kern, split = (8192, "gemm_fast_256x256 ", "ksplit 4") if lay == "NN" else (4096, "gemm_fast_128x128 ", "ksplit 2")
    p = synth.Problem(2048, 2048, K, lay[0], lay[1], "f16", "f16", "bias_relu", 1.0, 0.0,
                      key=(129, lay == "TT"))
    x = synth.make_inputs(p)
    D, pl = run(p, x)
    assert pl.describe().startswith(kern) and split in pl.describe(), pl.describe()
    check_points(p, x, D)


# ---- the plan's own choice over a wide range of sizes ------------------------------------------
# Seeded draws: M and N log-uniform up to 4096, K up to 8192 (at most 2^33 multiply-adds), half
# of them rounded up to whole 16-byte chunks and 128-deep slabs, a quarter with padded leading
# dimensions, so that the automatic routes are met (general kernel, skinny kernel, 128-wide fast
# tiles, the 256-wide tiles' K split, aligned copies): exact inputs, bit-exact against the oracle.
@pytest.mark.parametrize("case", range(40))
def test_auto_route_random_sizes_exact(case):
    rng = np.random.default_rng(np.random.SeedSequence([183, case]))
    pairs = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("i8", "i32")]
    ab, cd = pairs[case % len(pairs)]
    lay = LAYOUTS[int(rng.integers(4))]
    while True:
        M, N = (int(round(float(np.exp(rng.uniform(0.0, np.log(4096)))))) for _ in range(2))
        K = int(round(float(np.exp(rng.uniform(0.0, np.log(8192))))))
        if M * N * K <= 1 << 33:
            break
    if rng.random() < 0.5:
        M, N, K = -(-M // 16) * 16, -(-N // 16) * 16, -(-K // 128) * 128
    epi = EPIS[int(rng.integers(4))]
    alpha, beta = SCALARS[int(rng.integers(4))]
    p = _exact(M, N, K, lay, ab, cd, epi, alpha, beta, key=(184, case))
    if rng.random() < 0.25:
        pa, pb, pc = (int(v) for v in rng.integers(1, 10, size=3))
        p = replace(p, lda=p.lda + pa, ldb=p.ldb + pb, ldc=p.ldc + pc)
    offset = int(rng.integers(2))
    x = synth.make_inputs(p)
    D, pl = run(p, x, offset=offset)
    print(p.label(), "lda", p.lda, "ldb", p.ldb, "ldc", p.ldc, "offset", offset, "->", pl.describe(),
          flush=True)
    check(p, x, D, reference(p, x, threads=16), exact=True)
