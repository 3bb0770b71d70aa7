"""Shared helpers for the GPU parity tests: upload the raw synthetic arrays, run one plan through
the C ABI, download D, and compare with the oracle."""
import numpy as np
import torch

import oracle
import synth
import tiled_gemm_epilogues_amd as tge

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
            "i32": torch.int32}
# kernel route pinned by a test (gemm_algo_t name, tile); the plans built here take it
FORCE = {"algo": "auto", "tile": 0}
TOL = 2e-3          # max|D-ref| / (K * max|op(A)| * max|op(B)|) for float outputs
DEV = "cuda:0"


def to_dev(dtype, raw, offset=0):
    """Raw numpy storage -> device tensor of the storage type; `offset` extra leading elements
    shift the data pointer (to test unaligned pointers)."""
    flat = np.ascontiguousarray(raw).reshape(-1)
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(flat.view(np.int16).copy()).view(TORCH_DT[dtype])
    else:
        t = torch.from_numpy(flat.copy())
    if offset:
        t = torch.cat([torch.zeros(offset, dtype=t.dtype), t])
    t = t.to(DEV)
    return t[offset:] if offset else t


def to_host(dtype, t):
    t = t.detach().cpu().contiguous()
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sentinel(dtype):
    return {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0),
            "i32": np.int32(-0x5A5A5A5A)}[dtype]


def run(p, x, offset=0, d_rows_extra=0, c_is_d=False, stream=None, plan=None):
    """Run problem p with inputs x on the GPU; returns the raw D storage (rows M + extra, ldc)
    initialised with a sentinel, so untouched elements are visible."""
    A = to_dev(p.a_store, x["A"], offset)
    B = to_dev(p.b_store, x["B"], offset)
    rows = p.M + d_rows_extra
    Dinit = np.full(rows * p.ldc, sentinel(p.cd), dtype=synth.RAW_NP[p.cd])
    if c_is_d:
        Dinit[: p.M * p.ldc] = x["C"].reshape(-1)
    D = to_dev(p.cd, Dinit, offset)
    C = D if c_is_d else (to_dev(p.cd, x["C"], offset) if x["C"] is not None else None)
    bias = to_dev(p.bias_dt, x["bias"], offset) if x["bias"] is not None else None
    pl = plan or tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                          transform_a=p.transform_a, transform_b=p.transform_b,
                          transform_c=p.transform_c, kind_a=p.kind_a, kind_b=p.kind_b,
                          algo=FORCE["algo"], tile=FORCE["tile"])
    pl.run(A, B, C, D, bias, p.alpha, p.beta, stream=stream)
    torch.cuda.synchronize()
    return to_host(p.cd, D).reshape(rows, p.ldc), pl


def reference(p, x, rows=None, threads=None):
    return oracle.gemm(p.M, p.N, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, p.ab, C=x["C"],
                       ldc=p.ldc, cd=p.cd, bias=x["bias"], alpha=p.alpha, beta=p.beta, relu=p.relu,
                       rows=rows, threads=threads, transform_a=p.transform_a,
                       transform_b=p.transform_b, transform_c=p.transform_c, kind_a=p.kind_a,
                       kind_b=p.kind_b)


def normaliser(p, x):
    ma = (float(np.abs(oracle.decode(p.ab, x["A"])).max()) if p.kind_a == "diagonal"
          else oracle.max_abs_op(p.ab, x["A"], p.op_a, p.M, p.K, p.lda, p.transform_a))
    mb = (float(np.abs(oracle.decode(p.ab, x["B"])).max()) if p.kind_b == "diagonal"
          else oracle.max_abs_op(p.ab, x["B"], p.op_b, p.K, p.N, p.ldb, p.transform_b))
    return p.K * ma * mb


def check(p, x, Draw, ref, rows=slice(None), exact=False):
    """Compare D (raw, rows x ldc) with the exact reference of those rows.  Returns the
    normalised error (float outputs) or 0 (integer outputs)."""
    Dv = Draw[rows, : p.N]
    if p.cd == "i32":
        assert np.array_equal(Dv.astype(np.int64), ref), "int32 result differs from the oracle"
        return 0.0
    got = oracle.decode(p.cd, Dv)
    assert np.isfinite(got).all(), "non-finite output"
    if exact:
        want = oracle.decode(p.cd, oracle.round_to(p.cd, ref))
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} elements differ, first at {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"
        return 0.0
    den = normaliser(p, x)
    if den == 0:
        want = oracle.decode(p.cd, oracle.round_to(p.cd, ref))
        assert np.array_equal(got, want)
        return 0.0
    err = float(np.max(np.abs(got - ref)) / den)
    assert err <= TOL, f"normalised error {err:.3e} > {TOL}"
    return err


def check_points(p, x, Draw, n=2000, seed=0):
    """Sampled comparison for full-size problems: n random output points plus the four corners."""
    g = np.random.default_rng(seed)
    ii = np.concatenate([g.integers(0, p.M, n), [0, 0, p.M - 1, p.M - 1]])
    jj = np.concatenate([g.integers(0, p.N, n), [0, p.N - 1, 0, p.N - 1]])
    ref = oracle.points(ii, jj, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, p.ab, C=x["C"],
                        ldc=p.ldc, cd=p.cd, bias=x["bias"], alpha=p.alpha, beta=p.beta, relu=p.relu)
    Dv = Draw[ii, jj]
    if p.cd == "i32":
        assert np.array_equal(Dv.astype(np.int64), ref)
        return 0.0
    got = oracle.decode(p.cd, Dv)
    den = normaliser(p, x)
    err = float(np.max(np.abs(got - ref)) / den)
    assert err <= TOL, f"normalised error {err:.3e} > {TOL}"
    return err


def run_batched(p, x, offset=0):
    """Run the strided-batched problem p (flat inputs x) through a batched plan; returns the raw
    flat D storage (initialised with a sentinel, gaps between products included)."""
    A = to_dev(p.a_store, x["A"], offset)
    B = to_dev(p.b_store, x["B"], offset)
    nD = max(p.batch - 1, 0) * p.stride_c + max(p.batch2 - 1, 0) * p.stride2_c + p.M * p.ldc
    D = to_dev(p.cd, np.full(nD, sentinel(p.cd), dtype=synth.RAW_NP[p.cd]), offset)
    C = to_dev(p.cd, x["C"], offset) if x["C"] is not None else None
    bias = to_dev(p.bias_dt, x["bias"], offset) if x["bias"] is not None else None
    pl = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                  batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, stride_c=p.stride_c,
                  stride_bias=p.stride_bias, transform_a=p.transform_a,
                  transform_b=p.transform_b, transform_c=p.transform_c, kind_a=p.kind_a,
                  kind_b=p.kind_b, algo=FORCE["algo"], tile=FORCE["tile"], batch2=p.batch2,
                  stride2_a=p.stride2_a, stride2_b=p.stride2_b, stride2_c=p.stride2_c,
                  stride2_bias=p.stride2_bias)
    pl.run(A, B, C, D, bias, p.alpha, p.beta)
    torch.cuda.synchronize()
    return to_host(p.cd, D).reshape(-1), pl


def reference_batched(p, x):
    """Exact results of every product, (batch * batch2) x M x N, product b = b1 * batch2 + b2."""
    return _reference_batched(p, x).reshape(-1, p.M, p.N)


def batch_offset(p, b):
    """Element offset of product b's C / D (b = b1 * batch2 + b2)."""
    b1, b2 = divmod(b, max(p.batch2, 1))
    return b1 * p.stride_c + b2 * p.stride2_c


def _reference_batched(p, x):
    return oracle.gemm_batched(p.M, p.N, p.K, p.op_a, p.op_b, x["A"], p.lda, x["B"], p.ldb, p.ab,
                               C=x["C"], ldc=p.ldc, cd=p.cd, bias=x["bias"], alpha=p.alpha,
                               beta=p.beta, relu=p.relu, batch=p.batch, stride_a=p.stride_a,
                               stride_b=p.stride_b, stride_c=p.stride_c,
                               stride_bias=p.stride_bias, transform_a=p.transform_a,
                               transform_b=p.transform_b, transform_c=p.transform_c,
                               kind_a=p.kind_a, kind_b=p.kind_b, batch2=p.batch2,
                               stride2_a=p.stride2_a, stride2_b=p.stride2_b,
                               stride2_c=p.stride2_c, stride2_bias=p.stride2_bias)
