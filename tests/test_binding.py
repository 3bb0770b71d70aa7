"""The Python binding on the CPU: tensors are checked against the plan before anything reaches
the C ABI (dtype, contiguity, row length, the span of elements the plan touches), and the
synthetic inputs the tests and the bench upload fit the plans built for them."""
import numpy as np
import pytest
import torch

import synth
import tiled_gemm_epilogues_amd as tge


def _t(n, dtype=torch.float16):
    return torch.zeros(n, dtype=dtype)


def test_spans_of_every_layout():
    p = tge.Plan(30, 20, 10, "N", "N", lda=12, ldb=24, ldc=21)
    sp = p.spans()
    assert sp["A"] == (29 * 12 + 10, 12)
    assert sp["B"] == (9 * 24 + 20, 24)
    assert sp["C"] == sp["D"] == (29 * 21 + 20, 21)
    assert sp["bias"] == (20, None)
    p = tge.Plan(30, 20, 10, "T", "T", lda=31, ldb=11, ldc=20)
    assert p.spans()["A"] == (9 * 31 + 30, 31)      # stored K x M
    assert p.spans()["B"] == (19 * 11 + 10, 11)     # stored N x K


def test_batched_spans_include_the_strides():
    p = tge.Plan(8, 16, 32, "N", "N", batch=3, stride_a=300, stride_b=0, stride_c=200,
                 stride_bias=16, epilogue="bias")
    sp = p.spans()
    assert sp["A"][0] == 2 * 300 + 7 * 32 + 32
    assert sp["B"][0] == 31 * 16 + 16               # shared between the products
    assert sp["D"][0] == 2 * 200 + 7 * 16 + 16
    assert sp["bias"][0] == 2 * 16 + 16


def test_diagonal_operand_span_is_its_vector():
    p = tge.Plan(64, 48, 64, "N", "N", kind_a="diagonal")
    assert p.spans()["A"] == (64, None)


def test_short_tensor_rejected():
    p = tge.Plan(30, 20, 10, lda=12)
    need = p.spans()["A"][0]
    p.check("A", _t(need))
    with pytest.raises(ValueError, match="spans"):
        p.check("A", _t(need - 1))
    with pytest.raises(ValueError, match="spans"):
        p.check("D", _t(30 * 20 - 1))


def test_wrong_dtype_rejected():
    p = tge.Plan(16, 16, 16, ab="bf16", cd="f32", epilogue="bias")
    with pytest.raises(TypeError):
        p.check("A", _t(256, torch.float16))
    with pytest.raises(TypeError):
        p.check("D", _t(256, torch.float16))
    with pytest.raises(TypeError):
        p.check("bias", _t(16, torch.int32))
    q = tge.Plan(16, 16, 128, ab="i8", cd="i32", epilogue="bias")
    q.check("bias", _t(16, torch.int32))


def test_non_contiguous_rejected():
    p = tge.Plan(16, 16, 16)
    big = torch.zeros(16, 32, dtype=torch.float16)
    with pytest.raises(ValueError, match="contiguous"):
        p.check("A", big[:, ::2])


def test_row_length_must_be_the_leading_dimension():
    p = tge.Plan(16, 24, 32, "N", "N")        # lda 32, ldb 24, ldc 24
    p.check("A", torch.zeros(16, 32, dtype=torch.float16))
    with pytest.raises(ValueError, match="leading dimension"):
        p.check("A", torch.zeros(32, 16, dtype=torch.float16))   # same size, transposed shape
    p.check("B", torch.zeros(32, 24, dtype=torch.float16))
    p.check("D", torch.zeros(16, 24, dtype=torch.float16))
    with pytest.raises(ValueError, match="leading dimension"):
        p.check("D", torch.zeros(24, 16, dtype=torch.float16))


def test_run_rejects_host_tensors_before_the_library():
    p = tge.Plan(16, 16, 16)
    with pytest.raises(ValueError, match="device tensor"):
        p.run(_t(256), _t(256), None, _t(256))


def _stored_sizes(p):
    """Elements (numbers for complex / dual types) of the arrays synth.make_inputs stores for p,
    and of the D buffer the tests and the bench allocate."""
    more = lambda stride: stride * (p.batch - 1) if p.batch > 1 and stride > 0 else 0
    more2 = lambda stride: stride * (p.batch2 - 1) if p.batch2 > 1 and stride > 0 else 0
    a = p.M if p.kind_a == "diagonal" else p.a_shape()[0] * p.lda
    b = p.N if p.kind_b == "diagonal" else p.b_shape()[0] * p.ldb
    c = p.M * p.ldc
    return {"A": a + more(p.stride_a) + more2(p.stride2_a),
            "B": b + more(p.stride_b) + more2(p.stride2_b),
            "C": c + more(p.stride_c) + more2(p.stride2_c),
            "D": c + max(p.batch - 1, 0) * p.stride_c + max(p.batch2 - 1, 0) * p.stride2_c,
            "bias": p.N + more(p.stride_bias) + more2(p.stride2_bias)}


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_synthetic_inputs_fit_their_plans(name):
    """Every workload's stored arrays cover the spans its plan checks (shape-level only: the
    arrays are not generated at full size)."""
    for p in synth.WORKLOADS[name]():
        plan = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                        batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b,
                        stride_c=p.stride_c, stride_bias=p.stride_bias, transform_a=p.transform_a,
                        transform_b=p.transform_b, transform_c=p.transform_c, kind_a=p.kind_a,
                        kind_b=p.kind_b, batch2=p.batch2, stride2_a=p.stride2_a,
                        stride2_b=p.stride2_b, stride2_c=p.stride2_c, stride2_bias=p.stride2_bias)
        sizes = _stored_sizes(p)
        sp = plan.spans()
        for what in ("A", "B", "D"):
            assert sizes[what] >= sp[what][0], (name, what, sizes[what], sp[what])
        if p.beta != 0:
            assert sizes["C"] >= sp["C"][0]
        if p.has_bias:
            assert sizes["bias"] >= sp["bias"][0]


def test_small_inputs_fit_their_plans():
    """Generated arrays (not only their sizes) of ragged, padded and batched problems."""
    probs = [synth.exact_integer_problem(37, 29, 70, "T", "N", "f16", "f32", "bias", 2.0, -1.0,
                                         key=(1, 0), ld_pad=3),
             synth.exact_integer_problem(37, 29, 70, "N", "T", "bf16", "bf16", "bias_relu", 1.0,
                                         1.0, key=(1, 1)),
             synth.exact_integer_problem(8, 40, 64, "N", "N", "f16", "f16", "bias", 1.0, 1.0,
                                         key=(1, 2), batch=3, stride_a=8 * 64 + 5, stride_b=0,
                                         stride_c=8 * 40 + 8, stride_bias=40)]
    for p in probs:
        x = synth.make_inputs(p)
        plan = tge.Plan(p.M, p.N, p.K, p.op_a, p.op_b, p.lda, p.ldb, p.ldc, p.ab, p.cd, p.epi,
                        batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b,
                        stride_c=p.stride_c, stride_bias=p.stride_bias)
        for what, key in (("A", "A"), ("B", "B"), ("C", "C"), ("bias", "bias")):
            if x[key] is None:
                continue
            dt = plan.dtype_of(what)
            flat = np.ascontiguousarray(x[key]).reshape(-1)
            t = (torch.from_numpy(flat.view(np.int16)).view(
                {"f16": torch.float16, "bf16": torch.bfloat16}[dt]) if dt in ("f16", "bf16")
                else torch.from_numpy(flat))
            plan.check(what, t)
