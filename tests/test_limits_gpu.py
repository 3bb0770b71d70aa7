"""GPU parity at the size limits of the kernels: operands whose stored span comes within a few
bytes of 2^31 (the largest the plan accepts: the kernels address inside one matrix with 32-bit
offsets), and a strided batch whose last product starts more than 4 GiB past the first (64-bit
batch offsets).  Exact-integer inputs, so the result must equal the oracle's bit for bit; the
large spans come from leading dimensions far wider than the rows, which keeps the oracle's
work small."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import FORCE, check, reference, reference_batched, run, run_batched

pytestmark = pytest.mark.gpu

LIM = 1 << 31


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _widest_ld(rows, cols, esize, mult):
    """Largest leading dimension, a multiple of `mult`, with a stored span (rows - 1) * ld + cols
    below 2^31 bytes."""
    ld = (LIM // esize - cols - 1) // (rows - 1)
    return ld - ld % mult


# kernel, layout, ld multiple (1 with an odd ld: "fast" copies the operands into aligned rows
# first, "staged" reads them in place with the register-staged variant)
CASES = [("fast", "NN", 8), ("fast", "TN", 1), ("staged", "TN", 1), ("general", "TT", 8)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_operand_spans_just_below_2_gib(case, monkeypatch):
    kern, lay, mult = CASES[case]
    monkeypatch.setitem(FORCE, "algo", kern)
    M, N, K = 300, 264, 200
    p = synth.exact_integer_problem(M, N, K, lay[0], lay[1], "f16", "f32", "bias_relu", 1.0, 1.0,
                                    key=(140, case))
    ra, ca = (M, K) if lay[0] == "N" else (K, M)
    rb, cb = (K, N) if lay[1] == "N" else (N, K)
    p.lda = _widest_ld(ra, ca, 2, mult)
    p.ldb = _widest_ld(rb, cb, 2, mult)
    p.ldc = _widest_ld(M, N, 4, mult)
    if mult == 1:
        p.lda -= 1 - p.lda % 2; p.ldb -= 1 - p.ldb % 2; p.ldc -= 1 - p.ldc % 2   # odd
    for rows, cols, ld, e in ((ra, ca, p.lda, 2), (rb, cb, p.ldb, 2), (M, N, p.ldc, 4)):
        span = ((rows - 1) * ld + cols) * e
        assert LIM - (1 << 20) < span < LIM, span
    # the operands' values depend on the problem's key, not on its leading dimensions: the
    # oracle runs on the tightly stored copy
    tight = synth.exact_integer_problem(M, N, K, lay[0], lay[1], "f16", "f32", "bias_relu", 1.0,
                                        1.0, key=(140, case))
    xt = synth.make_inputs(tight)
    ref = reference(tight, xt)
    x = synth.make_inputs(p)
    print(p.label(), "lda", p.lda, "ldb", p.ldb, "ldc", p.ldc, flush=True)
    D, pl = run(p, x)
    assert ("gemm_fast" in pl.describe()) == (kern != "general"), pl.describe()
    check(p, xt, D, ref, exact=True)


def test_batch_offsets_beyond_4_gib(monkeypatch):
    # product 1 of A starts 4 GiB + 16 bytes after product 0; B is shared
    monkeypatch.setitem(FORCE, "algo", "fast")
    M, N, K = 264, 256, 192
    p = synth.exact_integer_problem(M, N, K, "N", "N", "f16", "f16", "bias", 1.0, 1.0,
                                    key=(141, 0), batch=2, stride_a=(1 << 31) + 8, stride_b=0,
                                    stride_bias=N)
    x = synth.make_inputs(p)
    print(p.label(), "stride_a", p.stride_a, flush=True)
    D, pl = run_batched(p, x)
    assert "gemm_fast" in pl.describe() and "batch 2" in pl.describe(), pl.describe()
    got = D
    ref = reference_batched(p, x)
    import oracle
    for b in range(2):
        Db = got[b * p.stride_c: b * p.stride_c + M * p.ldc].reshape(M, p.ldc)[:, :N]
        want = oracle.round_to(p.cd, ref[b])
        assert np.array_equal(oracle.decode(p.cd, Db), oracle.decode(p.cd, want)), f"product {b}"
