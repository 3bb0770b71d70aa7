"""The oracle's pins must catch plausible mistakes: each case plants one mistake in a copy of
oracle.c (on the CPU), builds it, and checks that the pin suite fails against that build."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "drop_last_k": ("k < K; ++k", "k + 1 < K; ++k"),
    "transposed_gather": ("out[r * cols + c] = op ? X[c * ldx + r] : X[r * ldx + c];",
                          "out[r * cols + c] = op ? X[r * ldx + c] : X[r * ldx + c];"),
    "bias_by_row": ("if (bias) t += bias[j];\n            if (relu && !(t > 0.0))",
                    "if (bias) t += bias[i % N];\n            if (relu && !(t > 0.0))"),
    "beta_sign": ("if (beta != 0.0) t += beta * C[i * N + j];",
                  "if (beta != 0.0) t -= beta * C[i * N + j];"),
    "alpha_scales_bias": ("if (bias) t += bias[j];\n            if (relu && !(t > 0.0))",
                          "if (bias) t += alpha * bias[j];\n            if (relu && !(t > 0.0))"),
    "f16_exponent_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "relu_threshold": ("if (relu && !(t > 0.0)) t = 0.0;\n            out[i * N + j] = t;",
                       "if (relu && t < -0.25) t = 0.0;\n            out[i * N + j] = t;"),
    "round_truncates": ("double m = rint(a / ldexp(1.0, ue - 10));",
                        "double m = floor(a / ldexp(1.0, ue - 10));"),
    "points_b_index": ("oracle_elem_f64(ab_dt, B, opb ? j * ldb + k : k * ldb + j)",
                       "oracle_elem_f64(ab_dt, B, opb ? k * ldb + j : k * ldb + j)"),
    "tile_skips_rows": ("for (int64_t i = m; i < me; ++i) {\n                    double a",
                        "for (int64_t i = m + (me - m > 1); i < me; ++i) {\n                    double a"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert old in src, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    c = tmp_path / "oracle_mut.c"
    c.write_text(mutated)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                    str(so), str(c), "-lpthread", "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"


# planted mistakes in the Python side of the oracle (the tolerance normaliser)
PY_MUTANTS = {
    "t_rows_cols_swapped": ("    else:\n        idx_ok = (np.arange(d.size) % ld) < rows",
                            "    else:\n        idx_ok = (np.arange(d.size) % ld) < cols"),
    "padding_included": ("    if op == \"N\":\n        idx_ok = (np.arange(d.size) % ld) < cols",
                         "    if op == \"N\":\n        idx_ok = (np.arange(d.size) % ld) < ld"),
    "span_one_short": ("d = decode(dtype, _raw(dtype, X)[: _span(op, rows, cols, ld)])",
                       "d = decode(dtype, _raw(dtype, X)[: _span(op, rows, cols, ld) - 1])"),
    "whole_storage": ("d = decode(dtype, _raw(dtype, X)[: _span(op, rows, cols, ld)])",
                      "d = decode(dtype, _raw(dtype, X))"),
    "sign_kept": ("return float(np.max(np.abs(d[idx_ok]))) if idx_ok.any() else 0.0",
                  "return float(np.max(d[idx_ok])) if idx_ok.any() else 0.0"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_normaliser_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    import importlib.util

    import oracle
    from test_oracle import check_max_abs_op_pins

    old, new = PY_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert old in src, f"mutation anchor for {name} not found"
    path = tmp_path / "oracle_mut.py"
    path.write_text(src.replace(old, new))
    # the mutated module uses the same C library as the real one
    monkeypatch.setenv("ORACLE_LIB", oracle._LIB_PATH)
    spec = importlib.util.spec_from_file_location("oracle_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        check_max_abs_op_pins(mod)


# planted mistakes in the type-converting load transform
CONV_MUTANTS = {
    "no_rounding": ("    x = np.ascontiguousarray(x, np.float64)\n    return decode(ab, round_to(ab, x))",
                    "    x = np.ascontiguousarray(x, np.float64)\n    return x"),
    "rounds_via_f32_truncation": ("    x = np.ascontiguousarray(x, np.float64)\n    return decode(ab, round_to(ab, x))",
                                  "    x = np.ascontiguousarray(x, np.float64)\n    return decode(ab, round_to(ab, np.trunc(x * 1024) / 1024))"),
    "conversion_skipped_in_gemm": ("    vals = decode(st, _raw(st, raw)[span_start: span_start + span_len]).astype(np.float64)\n    return convert_to(ab, vals)",
                                   "    vals = decode(st, _raw(st, raw)[span_start: span_start + span_len]).astype(np.float64)\n    return vals"),
}


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conversion_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    import importlib.util

    import oracle
    from test_oracle import check_conversion_pins

    old, new = CONV_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert old in src, f"mutation anchor for {name} not found"
    path = tmp_path / "oracle_mut.py"
    path.write_text(src.replace(old, new))
    monkeypatch.setenv("ORACLE_LIB", oracle._LIB_PATH)
    spec = importlib.util.spec_from_file_location("oracle_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        check_conversion_pins(mod)


# planted mistakes in the two-mode batch
BATCH2_MUTANTS = {
    "a_moves_with_b_stride": ("_raw_store(transform_a, ab, A)[b2 * stride2_a:]",
                              "_raw_store(transform_a, ab, A)[b2 * stride2_b:]"),
    "c_second_mode_dropped": ("C=_raw(cd, C)[b2 * stride2_c:]", "C=_raw(cd, C)[0:]"),
    "modes_swapped_in_result": ("np.stack(out, axis=1)", "np.stack(out, axis=0)"),
}


@pytest.mark.parametrize("name", sorted(BATCH2_MUTANTS))
def test_two_mode_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    import importlib.util

    import oracle
    from test_oracle import check_two_mode_pins

    old, new = BATCH2_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert old in src, f"mutation anchor for {name} not found"
    path = tmp_path / "oracle_mut.py"
    path.write_text(src.replace(old, new))
    monkeypatch.setenv("ORACLE_LIB", oracle._LIB_PATH)
    spec = importlib.util.spec_from_file_location("oracle_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        check_two_mode_pins(mod)
