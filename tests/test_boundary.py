"""The C-ABI library on the CPU: it loads, exports every function include/gemm.h declares, and
its host-side validation returns the documented status codes.  None of these calls reaches the
GPU (plan creation is host-only; the rejected or empty runs return before any launch)."""
import ctypes
import os
import re

import pytest

import tiled_gemm_epilogues_amd as tge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "gemm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(tge.EXPORTED)
    lib = tge.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(6):
        assert tge.gemm_status_string(s).startswith("GEMM_STATUS_")
    assert tge.gemm_status_string(tge.STATUS_SCRATCH_LIMIT) == "GEMM_STATUS_SCRATCH_LIMIT"
    assert tge.gemm_status_string(99) == "GEMM_STATUS_UNKNOWN"


def _create(**kw):
    a = dict(M=64, N=64, K=64, op_a="N", op_b="N", lda=64, ldb=64, ldc=64, ab_type="f16",
             cd_type="f16", epilogue="none")
    a.update(kw)
    return tge.gemm_plan_create(**a)


@pytest.mark.parametrize("kw", [dict(M=-1), dict(N=-1), dict(K=-1), dict(lda=63), dict(ldb=63),
                                dict(ldc=63), dict(op_a="T", lda=63), dict(op_b="T", ldb=63),
                                dict(op_a=2), dict(ab_type=9), dict(cd_type=-1), dict(epilogue=4),
                                dict(M=0, N=0, K=0, lda=0, ldb=0, ldc=0)])
def test_invalid_values(kw):
    st, h = _create(**kw)
    assert st == tge.STATUS_INVALID_VALUE and h is None


@pytest.mark.parametrize("ab,cd", [("f16", "bf16"), ("bf16", "f16"), ("i8", "f32"), ("f32", "f16"),
                                   ("i32", "i32"), ("i8", "i8"), ("f16", "i32"), ("cf16", "df32"),
                                   ("cf32", "cf32"), ("df16", "f32"), ("f16", "cf32")])
def test_unsupported_pairs(ab, cd):
    st, h = _create(ab_type=ab, cd_type=cd)
    assert st == tge.STATUS_NOT_SUPPORTED and h is None


def test_span_limit():
    st, _ = _create(M=40000, N=40000, K=64, ldb=40000, ldc=40000, cd_type="f32", ab_type="f16")
    assert st == tge.STATUS_NOT_SUPPORTED


@pytest.mark.parametrize("ab,cd", [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"),
                                   ("bf16", "f32"), ("i8", "i32")])
@pytest.mark.parametrize("lay", ["NN", "NT", "TN", "TT"])
def test_supported_pairs_and_describe(ab, cd, lay):
    p = tge.Plan(300, 200, 100, lay[0], lay[1], ab=ab, cd=cd, epilogue="bias_relu")
    d = p.describe()
    assert f"{ab}->{cd} {lay}" in d and "grid" in d


def test_null_out_pointer():
    lib = tge.lib()
    lib.gemm_plan_create.restype = ctypes.c_int
    st = lib.gemm_plan_create(None, ctypes.c_int64(1), ctypes.c_int64(1), ctypes.c_int64(1), 0, 0,
                              ctypes.c_int64(1), ctypes.c_int64(1), ctypes.c_int64(1), 1, 1, 0)
    assert st == tge.STATUS_INVALID_VALUE


def test_run_rejections_before_launch():
    assert tge.gemm_run(None, 1, 1, None, 1, None, 1.0, 0.0, None) == tge.STATUS_INVALID_VALUE
    st, h = _create(epilogue="bias")
    try:
        # D missing
        assert tge.gemm_run(h, 16, 16, None, None, 16, 1.0, 0.0, None) == tge.STATUS_INVALID_VALUE
        # bias missing for a bias epilogue
        assert tge.gemm_run(h, 16, 16, None, 16, None, 1.0, 0.0, None) == tge.STATUS_INVALID_VALUE
        # C missing with beta != 0
        assert tge.gemm_run(h, 16, 16, None, 16, 16, 1.0, 0.5, None) == tge.STATUS_INVALID_VALUE
        # A missing with K > 0
        assert tge.gemm_run(h, None, 16, None, 16, 16, 1.0, 0.0, None) == tge.STATUS_INVALID_VALUE
        # NaN scalar
        assert tge.gemm_run(h, 16, 16, None, 16, 16, float("nan"), 0.0, None) == tge.STATUS_INVALID_VALUE
    finally:
        tge.gemm_plan_destroy(h)
    st, h = _create(ab_type="i8", cd_type="i32")
    try:
        assert tge.gemm_run(h, 16, 16, None, 16, None, 2.0, 0.0, None) == tge.STATUS_NOT_SUPPORTED
        assert tge.gemm_run(h, 16, 16, 16, 16, None, 1.0, 0.5, None) == tge.STATUS_NOT_SUPPORTED
    finally:
        tge.gemm_plan_destroy(h)


def test_empty_problem_returns_without_launch():
    st, h = _create(M=0, lda=64)
    assert st == tge.STATUS_SUCCESS
    try:
        assert tge.gemm_run(h, None, None, None, None, None, 1.0, 0.0, None) == tge.STATUS_SUCCESS
    finally:
        tge.gemm_plan_destroy(h)


def test_destroy_null_is_noop():
    assert tge.gemm_plan_destroy(None) == tge.STATUS_SUCCESS


def test_forced_tile():
    for t in (256, 128, 64):
        assert f"tile {t}x{t}" in tge.Plan(100, 100, 100, tile=t).describe()


def test_plans_ignore_the_environment(monkeypatch):
    # the kernel choice comes from the description only: no environment variable steers it
    base = tge.Plan(8192, 8192, 8192).describe()
    for var in ("TGE_FORCE_KERNEL", "TGE_FORCE_TILE"):
        monkeypatch.setenv(var, "general" if var.endswith("KERNEL") else "64")
    assert tge.Plan(8192, 8192, 8192).describe() == base


@pytest.mark.parametrize("kw", [dict(algo=8), dict(algo=-1), dict(tile=32), dict(tile=-256)])
def test_invalid_algo_or_tile(kw):
    st, h = tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, "f16", "f16", "none", **kw)
    assert st == tge.STATUS_INVALID_VALUE and h is None


def test_single_hip_runtime_in_process():
    # the library must bind to the HIP runtime torch loaded, never bring a second one
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths


# ---- strided batch and the full description ---------------------------------------------------

def _create_batched(**kw):
    a = dict(M=64, N=64, K=64, op_a="N", op_b="N", lda=64, ldb=64, ldc=64, ab_type="f16",
             cd_type="f16", epilogue="none", batch=4, stride_a=64 * 64, stride_b=64 * 64,
             stride_c=64 * 64, stride_bias=0)
    a.update(kw)
    return tge.gemm_plan_create_batched(**a)


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(stride_a=-1), dict(stride_b=-2),
                                dict(stride_c=-1), dict(stride_bias=-1),
                                dict(stride_c=64 * 63 + 63), dict(stride_c=0)])
def test_batched_invalid_values(kw):
    st, h = _create_batched(**kw)
    assert st == tge.STATUS_INVALID_VALUE and h is None


def test_batched_valid_and_described():
    st, h = _create_batched(stride_c=64 * 63 + 64, stride_a=0)
    assert st == tge.STATUS_SUCCESS
    assert "batch 4" in tge.gemm_plan_describe(h)[1]
    tge.gemm_plan_destroy(h)
    # batch 1 ignores the strides, batch 0 is a valid empty launch
    for b in (0, 1):
        st, h = _create_batched(batch=b, stride_c=0)
        assert st == tge.STATUS_SUCCESS
        tge.gemm_plan_destroy(h)


def test_batched_grid_limit():
    st, _ = _create_batched(M=4096, N=4096, K=64, lda=64, ldb=4096, ldc=4096, batch=1 << 24,
                            stride_a=0, stride_b=0, stride_c=4096 * 4096)
    assert st == tge.STATUS_NOT_SUPPORTED


def test_batch_zero_run_returns_without_launch():
    p = tge.Plan(64, 64, 64, batch=0, stride_c=64 * 64)
    assert tge.gemm_run(p.handle, None, None, None, 1, None, 1.0, 0.0, None) == tge.STATUS_SUCCESS


def test_desc_validation_and_transforms_described():
    st, h = tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, "f16", "f16", "none",
                                      transform_a="relu", transform_c="relu")
    assert st == tge.STATUS_SUCCESS and "relu-in AC" in tge.gemm_plan_describe(h)[1]
    tge.gemm_plan_destroy(h)
    for bad in (dict(transform_a=4), dict(transform_b=-1), dict(transform_c=7), dict(transform_c=2)):
        st, h = tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, "f16", "f16", "none",
                                          **bad)
        assert st == tge.STATUS_INVALID_VALUE and h is None
    lib = tge.lib()
    lib.gemm_plan_create_desc.restype = ctypes.c_int
    out = ctypes.c_void_p()
    assert lib.gemm_plan_create_desc(ctypes.byref(out), None) == tge.STATUS_INVALID_VALUE
    assert out.value is None


def test_desc_matches_the_plain_create():
    a = tge.gemm_plan_create_desc(300, 200, 100, "T", "N", 300, 200, 200, "bf16", "f32", "bias")
    b = tge.gemm_plan_create(300, 200, 100, "T", "N", 300, 200, 200, "bf16", "f32", "bias")
    assert a[0] == b[0] == tge.STATUS_SUCCESS
    assert tge.gemm_plan_describe(a[1])[1] == tge.gemm_plan_describe(b[1])[1]


@pytest.mark.parametrize("ab,cd", [("cf16", "cf32"), ("cf16", "cf16"), ("df16", "df32"),
                                   ("df16", "df16")])
def test_complex_dual_plans(ab, cd):
    st, h = _create(ab_type=ab, cd_type=cd, op_b="T")
    assert st == tge.STATUS_SUCCESS
    d = tge.gemm_plan_describe(h)[1]
    assert ("gemm_dual" if ab.startswith("d") else "gemm_complex") in d and f"{ab}->{cd} NT" in d
    tge.gemm_plan_destroy(h)
    # only the plain product: no bias / ReLU epilogue, transforms or diagonal operands
    for epi in ("relu", "bias", "bias_relu"):
        assert _create(ab_type=ab, cd_type=cd, epilogue=epi)[0] == tge.STATUS_NOT_SUPPORTED
    assert tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, ab, cd, "none",
                                     transform_a="relu")[0] == tge.STATUS_NOT_SUPPORTED
    assert tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, ab, cd, "none",
                                     kind_a="diagonal")[0] == tge.STATUS_NOT_SUPPORTED


# ---- kernel choice (host logic: the plan's description names the kernel it will launch) -----

@pytest.mark.parametrize("shape,lay,ab,cd,want,extra", [
    # aligned large product: the direct-load fast kernel
    ((8192, 8192, 8192), "NN", "f16", "f16", "gemm_fast_256x256 ", None),
    # odd leading dimensions (4095 x 3073 x 2047 stored tightly): both operands are copied
    # into aligned rows, then the direct-load kernel runs on the copies
    ((4095, 3073, 2047), "NN", "bf16", "f32", "gemm_fast_256x256 ", " repack AB"),
    ((4095, 3073, 2047), "TT", "bf16", "f32", "gemm_fast_256x256 ", " repack AB"),
    # aligned ld but N off the 16-byte grid with B not transposed: B is copied (rows padded)
    ((4096, 4100, 4096), "NN", "f16", "f16", "gemm_fast_256x256 ", " repack B"),
    # the same with B transposed (K-contiguous): the direct loads take it
    ((4096, 4100, 4096), "NT", "f16", "f16", "gemm_fast_256x256 ", None),
    # fp32 has no fast path; a short product takes the skinny kernel with K split 4 ways
    ((8192, 8192, 8192), "NN", "f32", "f32", "gemm_mfma_256x256", None),
    ((16, 4096, 4096), "NN", "f16", "f16", "gemm_skinny_m16", None),
])
def test_kernel_choice(shape, lay, ab, cd, want, extra):
    M, N, K = shape
    p = tge.Plan(M, N, K, lay[0], lay[1], ab=ab, cd=cd)
    assert want in p.describe() + " ", p.describe()
    assert (extra in p.describe()) if extra else ("repack" not in p.describe()), p.describe()


@pytest.mark.parametrize("shape,lay", [((4095, 3073, 2047), "NN"), ((4095, 3073, 2047), "TN"),
                                       ((4096, 4100, 4096), "NN")])
def test_kernel_choice_register_staged(shape, lay):
    # algorithm "staged": the register-staged variant reads such operands in place
    M, N, K = shape
    d = tge.Plan(M, N, K, lay[0], lay[1], ab="bf16", cd="f32", algo="staged").describe()
    assert "gemm_fast_256x256_rs" in d and "repack" not in d, d


def test_repack_only_what_the_direct_loads_cannot_read():
    # only the operand off the grid is copied: B with an odd ld; A with an M extent off the grid
    # when stored transposed; a K-contiguous operand's K tail needs no copy
    assert tge.Plan(4096, 4096, 4096, "N", "N", 4096, 4097, 4096).describe().endswith("repack B")
    assert tge.Plan(4100, 4096, 4096, "T", "N").describe().endswith("repack A (A to K-major)")
    d = tge.Plan(4096, 4096, 4100, "N", "T", 4104, 4104, 4096).describe()
    assert "gemm_fast_256x256 " in d and "repack" not in d, d
    # a strided batch whose A stride breaks alignment copies A per product
    d = tge.Plan(2048, 2048, 2048, "N", "N", batch=4, stride_a=2048 * 2048 + 1,
                 stride_b=2048 * 2048, stride_c=2048 * 2048).describe()
    assert "repack A" in d and "batch 4" in d, d


def test_kmajor_copy_of_a_transposed_a():
    # A stored transposed and B not: A is copied into K-contiguous rows (and the kernel of the
    # non-transposed layout runs) when N is wide enough to repay the copy, always with the
    # kmajor algorithm, never with fast; the other layouts never copy for it
    d = tge.Plan(5000, 5000, 5000, "T", "N", ab="bf16", cd="f32").describe()
    assert "gemm_fast_256x256 " in d and d.endswith("repack A (A to K-major)"), d
    d = tge.Plan(5000, 5000, 5000, "T", "N", ab="bf16", cd="f32", algo="fast").describe()
    assert "gemm_fast_256x256 " in d and "repack" not in d, d
    for n in (1024, 2048):
        d = tge.Plan(4096, n, 4096, "T", "N").describe()
        assert "repack" not in d, d
    d = tge.Plan(1024, 1024, 1024, "T", "N", algo="kmajor").describe()
    assert "gemm_fast_256x256 " in d and "(A to K-major)" in d, d
    for lay in ("NN", "NT", "TT"):
        d = tge.Plan(4096, 4096, 4096, lay[0], lay[1], algo="kmajor").describe()
        assert "gemm_fast_256x256 " in d and "repack" not in d, d
    # an A that has to be copied anyway (M off the 16-byte grid) is copied transposed
    d = tge.Plan(4100, 1024, 4096, "T", "N", algo="fast").describe()
    assert d.endswith("repack A (A to K-major)"), d


def test_fast128_tiles_chosen_for_mid_size_products():
    # 128x128 tiles of the fast kernel where 256x256 ones would leave half the CUs idle or more
    # (16-bit inputs read in place, no load transforms); an explicit tile of 128 pins them
    for (M, N, K) in [(1024, 1024, 1024), (2048, 2048, 2048), (4096, 2048, 2048), (1024, 4096, 1024),
                      (512, 512, 512), (256, 1024, 4096)]:
        assert tge.Plan(M, N, K).describe().startswith("gemm_fast_128x128 "), (M, N, K)
    for (M, N, K) in [(3072, 3072, 3072), (4096, 4096, 4096), (512, 512, 32)]:
        assert not tge.Plan(M, N, K).describe().startswith("gemm_fast_128x128 "), (M, N, K)
    assert tge.Plan(2048, 2048, 2048, ab="bf16", cd="f32", op_a="T").describe().startswith("gemm_fast_128x128 ")
    assert tge.Plan(2048, 2048, 2048, ab="i8", cd="i32").describe().startswith("gemm_fast_128x128 ")
    # load transforms and operands off the 16-byte grid: the 128-wide tiles on the copies
    for kw, shows in [(dict(transform_a="relu"), "repack A"), (dict(lda=2049), "repack A"),
                      (dict(ldb=2050, op_b="T"), "repack B"), (dict(op_a="T", M=2044), "repack A (A to K-major)")]:
        args = dict(M=2048, N=2048, K=2048)
        args.update(kw)
        d = tge.Plan(**args).describe()
        assert d.startswith("gemm_fast_128x128 ") and shows in d, (kw, d)
    # below about 2^31 multiply-adds the copy costs more than the tiles gain: the general kernel
    for kw in [dict(M=1024, N=1024, K=1024, lda=1025), dict(M=17, N=1, K=1161, op_a="T", lda=18),
               dict(M=1024, N=1024, K=1024, transform_a="relu")]:
        assert tge.Plan(**kw).describe().startswith("gemm_mfma_"), kw
    # (pinned, the 128-wide tiles take the copies at any size)
    d = tge.Plan(1024, 1024, 1024, lda=1025, algo="fast", tile=128).describe()
    assert d.startswith("gemm_fast_128x128 ") and "repack A" in d, d
    # not for the general algorithm, or a long K that splits
    assert not tge.Plan(1024, 1024, 1024, lda=1025, algo="general").describe().startswith("gemm_fast")
    assert " ksplit " in tge.Plan(2048, 2048, 8192).describe()
    # short products (64 < M <= 256) from 64 slabs of K split it over the 128-wide tiles
    for (M, N, K) in [(96, 4096, 4096), (256, 4096, 4096), (128, 8192, 8192)]:
        d = tge.Plan(M, N, K).describe()
        assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d
    d = tge.Plan(128, 4096, 2048).describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit" not in d, d
    assert tge.Plan(64, 4096, 4096).describe().startswith("gemm_skinny")
    d = tge.Plan(3072, 3072, 3072, algo="fast", tile=128).describe()
    assert d.startswith("gemm_fast_128x128 ") and "grid 576" in d, d
    assert not tge.Plan(2048, 2048, 2048, algo="general").describe().startswith("gemm_fast")


def test_skinny_split_k_described():
    # 64 column blocks fill a quarter of the chip: K is split 4 ways (8 chunks per wave); short K
    # is not split
    assert "ksplit 4" in tge.Plan(16, 4096, 4096, "N", "N").describe()
    assert "ksplit" not in tge.Plan(16, 4096, 512, "N", "N").describe()
    assert "ksplit" not in tge.Plan(16, 16384, 4096, "N", "N").describe()
    # GEMM_ALGO_NOSPLIT keeps the skinny kernel and drops its split
    d = tge.Plan(16, 4096, 4096, "N", "N", algo="nosplit").describe()
    assert "gemm_skinny_m16 " in d and "ksplit" not in d, d


def test_skinny_narrow_blocks_described():
    # B transposed, M <= 16: 16-column blocks when they make one round of 192-256 workgroups
    # (no k split); otherwise the 64-column blocks, split over K when they are too few
    d = tge.Plan(16, 4096, 4096, "N", "T").describe()
    assert "gemm_skinny_m16_n16" in d and "ksplit" not in d, d
    d = tge.Plan(16, 4096, 4096, "N", "N").describe()
    assert "gemm_skinny_m16 " in d and "ksplit 4" in d, d
    for shape in [(32, 4096, 4096), (7, 4104, 8192), (16, 1000, 2048)]:
        d = tge.Plan(*shape, "N", "T").describe()
        assert "_n16" not in d, d


def test_diagonal_kernels_described():
    d = tge.Plan(4096, 4096, 4096, "N", "N", kind_a="diagonal").describe()
    assert "gemm_diag_rows" in d and "diag A" in d, d
    d = tge.Plan(4096, 4096, 4096, "N", "T", kind_a="diagonal").describe()
    assert "gemm_diag_cols" in d, d
    d = tge.Plan(4096, 4096, 4096, "T", "N", kind_b="diagonal").describe()
    assert "gemm_diag_cols" in d and "diag B" in d, d
    d = tge.Plan(512, 512, 512, "N", "N", kind_a="diagonal", kind_b="diagonal").describe()
    assert "gemm_diag_rows" in d and "diag AB" in d, d


def test_transform_copies_only_for_the_fast_kernel():
    # the fast path copies an operand to apply its load transform; a skinny plan applies it in
    # its own kernel (also when a batch makes the fast kernel eligible too)
    d = tge.Plan(8192, 8192, 8192, "N", "N", transform_a="relu", transform_c="relu").describe()
    assert "gemm_fast_256x256 " in d and "repack A " in d and "relu-in AC" in d, d
    d = tge.Plan(64, 4096, 4096, "N", "N", batch=64, stride_a=64 * 4096, stride_b=0,
                 stride_c=64 * 4096, transform_a="relu").describe()
    assert "gemm_skinny" in d and "repack" not in d, d
    # only C transformed: nothing to copy
    d = tge.Plan(8192, 8192, 8192, "N", "N", transform_c="relu").describe()
    assert "repack" not in d, d


def test_fast_k_split_described():
    # few 256x256 tiles (more 128x128 ones than CUs) and K >= 4096: K cut into chunks of at least
    # 16 slabs, tiles x S >= 128
    d = tge.Plan(2048, 3072, 4096, "N", "N").describe()
    assert "gemm_fast_256x256 " in d and "ksplit 2" in d, d
    d = tge.Plan(2560, 2560, 8192, "N", "T").describe()
    assert "gemm_fast_256x256 " in d and "ksplit 2" in d, d
    # one 128x128 tile per CU and 64 to 127 slabs: those tiles split in two
    for (M, N, K, ab, cd) in [(2048, 2048, 4096, "f16", "f16"), (4096, 1024, 4096, "bf16", "f32"),
                              (2048, 2048, 8192, "i8", "i32")]:
        d = tge.Plan(M, N, K, ab=ab, cd=cd).describe()
        assert d.startswith("gemm_fast_128x128 ") and "ksplit 2" in d, (M, N, K, ab, d)
    assert "ksplit" not in tge.Plan(2048, 2048, 3072).describe()
    # from 128 slabs the 256-wide tiles' split (chunks of 32 slabs)
    d = tge.Plan(2048, 2048, 8192).describe()
    assert d.startswith("gemm_fast_256x256 ") and "ksplit 4" in d, d
    # fewer 128x128 tiles than CUs and at least 48 slabs: those tiles split K instead (about one
    # workgroup per CU, chunks of at least 4 slabs)
    for (M, N, K, lay, ab, cd, S) in [(1024, 1024, 8192, "NT", "bf16", "f32", 4), (512, 512, 8192, "NN", "f16", "f16", 16),
                                      (768, 768, 3072, "TN", "f16", "f16", 6), (288, 416, 7168, "NN", "f16", "f32", 16),
                                      (512, 512, 6144, "NN", "i8", "i32", 12)]:
        d = tge.Plan(M, N, K, lay[0], lay[1], ab=ab, cd=cd).describe()
        assert d.startswith("gemm_fast_128x128 ") and f"ksplit {S}" in d, d
    # at most one workgroup per CU: S is the largest divisor of the slabs with tiles x S <= 256
    for (M, N, K, S) in [(768, 768, 4096, 4), (640, 896, 4096, 4), (1536, 1024, 3072, 2), (512, 512, 8192, 16)]:
        d = tge.Plan(M, N, K).describe()
        t128 = ((M + 127) // 128) * ((N + 127) // 128)
        assert f"ksplit {S}" in d and t128 * S <= 256, (M, N, K, d)
    # empty products with the split pinned plan without a split (no launch)
    for (M, N) in [(0, 512), (512, 0)]:
        assert "ksplit" not in tge.Plan(M, N, 4096, algo="split", tile=128).describe()
    # 32 slabs: unsplit
    d = tge.Plan(640, 640, 2048).describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit" not in d, d
    # 2048^3 (K = 2048) stays on the general kernel; enough tiles: no split
    assert "ksplit" not in tge.Plan(2048, 2048, 2048, "N", "N").describe()
    assert "ksplit" not in tge.Plan(8192, 8192, 8192, "N", "N").describe()
    # no split with load transforms on A/B
    assert "ksplit" not in tge.Plan(2048, 2048, 8192, "N", "N", transform_a="relu").describe()
    # int8: 64 slabs of 128 from K = 8192
    d = tge.Plan(2048, 3072, 8192, "N", "N", ab="i8", cd="i32").describe()
    assert "gemm_fast_256x256 " in d and "ksplit 2" in d, d
    assert "ksplit" not in tge.Plan(2048, 2048, 4096, "N", "N", ab="i8", cd="i32").describe()
    # short int8 products (no skinny kernel): the 128x128 tiles split K from 8 slabs
    d = tge.Plan(16, 4096, 4096, "N", "N", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit 8" in d, d
    d = tge.Plan(64, 8192, 4096, "N", "T", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit 4" in d, d
    d = tge.Plan(16, 4096, 1024, "N", "N", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit 2" in d, d
    assert "ksplit" not in tge.Plan(16, 4096, 512, "N", "N", ab="i8", cd="i32").describe()
    # ... and short 16-bit products with A transposed (the skinny kernel needs A not transposed)
    d = tge.Plan(16, 4096, 4096, "T", "N").describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit 8" in d, d
    # int8 with B transposed up to 32 rows: the memory-bound kernel (int32 partial sums when it
    # splits K; a batch runs unsplit)
    d = tge.Plan(16, 4096, 4096, "N", "T", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_skinny_m16_n16 "), d
    d = tge.Plan(32, 8192, 4096, "N", "T", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_skinny_m32 ") and "ksplit 2" in d, d
    d = tge.Plan(40, 8192, 4096, "N", "T", ab="i8", cd="i32").describe()
    assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d
    d = tge.Plan(32, 4096, 4096, "N", "T", ab="i8", cd="i32", batch=3, stride_a=32 * 4096,
                 stride_b=0, stride_c=32 * 4096, stride_bias=0).describe()
    assert d.startswith("gemm_skinny") and "ksplit" not in d, d
    # the 256-wide tiles' split of short products, pinned: chunks down to 2 slabs
    d = tge.Plan(16, 4096, 4096, "N", "N", ab="i8", cd="i32", algo="split").describe()
    assert "gemm_fast_256x256 " in d and " ksplit " in d, d
    assert "gemm_skinny" in tge.Plan(16, 4096, 4096, "N", "N").describe()
    # an operand off the 16-byte grid is copied first, then split as well
    d = tge.Plan(2048, 2048, 8192, "N", "N", 8193, 2048, 2048).describe()
    assert "ksplit 4" in d and "repack A" in d, d
    d = tge.Plan(2048, 2048, 4096, "N", "N", 4097, 2048, 2048).describe()
    assert d.startswith("gemm_fast_128x128 ") and "ksplit 2" in d and "repack A" in d, d
    d = tge.Plan(2048, 3072, 4096, "N", "N", 4097, 3072, 3072).describe()
    assert d.startswith("gemm_fast_256x256 ") and "ksplit 2" in d and "repack A" in d, d
    assert "ksplit" not in tge.Plan(2048, 2048, 8192, "N", "N", algo="nosplit").describe()
    # the plan's own choice of kernel and tile otherwise
    for (M, N, K) in [(2048, 2048, 2048), (512, 512, 8192), (8192, 8192, 8192)]:
        d_auto, d_ns = tge.Plan(M, N, K).describe(), tge.Plan(M, N, K, algo="nosplit").describe()
        assert d_ns.split(" grid ")[0] == d_auto.split(" grid ")[0] and "ksplit" not in d_ns, (d_auto, d_ns)


def test_noalloc_rejects_runs_beyond_the_scratch_before_any_device_call():
    # the sizing pass runs on the host only: with fake (never dereferenced) pointers a run whose
    # aligned copy of A needs 8192 x 8200 x 2 bytes > 64 MiB is rejected before any HIP call
    assert tge.NOALLOC_SCRATCH_BYTES == 64 << 20
    st, h = tge.gemm_plan_create(8192, 8192, 8192, "N", "N", 8193, 8192, 8192, "f16", "f16", "none")
    assert st == tge.STATUS_SUCCESS and "repack A" in tge.gemm_plan_describe(h)[1]
    fake = 1 << 40
    assert tge.gemm_run_noalloc(h, fake, fake, None, fake, None, 1.0, 0.0, None) == \
        tge.STATUS_SCRATCH_LIMIT
    # argument errors come first, as in gemm_run
    assert tge.gemm_run_noalloc(h, fake, fake, None, None, None, 1.0, 0.0, None) == \
        tge.STATUS_INVALID_VALUE
    assert tge.gemm_run_noalloc(None, fake, fake, None, fake, None, 1.0, 0.0, None) == \
        tge.STATUS_INVALID_VALUE
    tge.gemm_plan_destroy(h)


def test_conversion_plans_validate():
    # conversions need a 16-bit input type and dense operands; none on C
    ok = tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, "f16", "f16", "none",
                                   transform_a="from_f32")
    assert ok[0] == tge.STATUS_SUCCESS
    tge.gemm_plan_destroy(ok[1])
    for kw, st in [(dict(ab_type="i8", cd_type="i32", transform_b="from_f32"), tge.STATUS_NOT_SUPPORTED),
                   (dict(transform_c="from_f32"), tge.STATUS_INVALID_VALUE),
                   (dict(transform_a=4), tge.STATUS_INVALID_VALUE),
                   (dict(transform_a="from_i8", kind_a="diagonal"), tge.STATUS_NOT_SUPPORTED)]:
        a = dict(ab_type="f16", cd_type="f16")
        a.update(kw)
        ab, cd = a.pop("ab_type"), a.pop("cd_type")
        got = tge.gemm_plan_create_desc(64, 64, 64, "N", "N", 64, 64, 64, ab, cd, "none", **a)
        assert got[0] == st and got[1] is None, (kw, got)


def test_short_products_split_only_from_eight_slabs():
    # four slabs of K (fp16 K = 256, int8 K = 512) stay on the general kernel, which measured
    # faster there; eight and more split
    for shape, ab in [((16, 256, 256), "f16"), ((64, 8192, 256), "f16"), ((64, 8192, 512), "i8")]:
        d = tge.Plan(*shape, "T", "N", ab=ab, cd="i32" if ab == "i8" else "f16").describe()
        assert "ksplit" not in d, d
    for shape, ab in [((32, 1024, 1024), "f16"), ((16, 4096, 1024), "i8"), ((64, 1024, 512), "f16")]:
        d = tge.Plan(*shape, "T", "N", ab=ab, cd="i32" if ab == "i8" else "f16").describe()
        assert d.startswith("gemm_fast_128x128 ") and " ksplit " in d, d


def test_empty_skinny_shapes_plan_and_run_without_launch():
    # found by the sanitizer build: an empty N (or batch) on a shape the skinny kernel takes
    # divided by zero while choosing its K split
    for kw in (dict(N=0, ldb=8, ldc=8), dict(N=4096, batch=0, stride_c=16 * 4096)):
        a = dict(M=16, K=4096, op_a="N", op_b="N")
        a.update(kw)
        p = tge.Plan(**a)
        assert tge.gemm_run(p.handle, None, None, None, None, None, 1.0, 0.0, None) == \
            tge.STATUS_SUCCESS


def test_two_mode_batch_validation_and_description():
    base = dict(M=64, N=64, K=64, op_a="N", op_b="N", lda=64, ldb=64, ldc=64, ab_type="f16",
                cd_type="f16", epilogue="none", batch=2, stride_a=4096, stride_b=0,
                stride_c=4096, stride_bias=0)
    ok = tge.gemm_plan_create_desc(**base, batch2=3, stride2_a=0, stride2_b=4096,
                                   stride2_c=2 * 4096)
    assert ok[0] == tge.STATUS_SUCCESS and "batch 2x3" in tge.gemm_plan_describe(ok[1])[1]
    tge.gemm_plan_destroy(ok[1])
    # the D blocks of the two modes must nest without overlap; negative values are invalid
    for kw in (dict(batch2=3, stride2_c=4096), dict(batch2=3, stride2_c=100),
               dict(batch2=-1), dict(batch2=2, stride2_a=-1)):
        st, h = tge.gemm_plan_create_desc(**base, **kw)
        assert st == tge.STATUS_INVALID_VALUE and h is None, kw
    # batch2 of 0 or 1 is a single mode; a conversion with two modes is not supported
    for b2 in (0, 1):
        st, h = tge.gemm_plan_create_desc(**base, batch2=b2, stride2_c=7)
        assert st == tge.STATUS_SUCCESS and "batch 2 " in tge.gemm_plan_describe(h)[1] + " "
        tge.gemm_plan_destroy(h)
    st, h = tge.gemm_plan_create_desc(**base, batch2=2, stride2_c=8192, transform_a="from_f32")
    assert st == tge.STATUS_NOT_SUPPORTED


def test_two_mode_spans_in_the_binding():
    p = tge.Plan(8, 16, 32, batch=2, stride_a=300, stride_c=200, batch2=3, stride2_a=0,
                 stride2_b=600, stride2_c=500)
    sp = p.spans()
    assert sp["A"][0] == 300 + 7 * 32 + 32
    assert sp["B"][0] == 31 * 16 + 16 + 2 * 600
    assert sp["D"][0] == 200 + 2 * 500 + 7 * 16 + 16
