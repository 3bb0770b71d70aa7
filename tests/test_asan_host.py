"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code, on the CPU:

* the oracle (oracle.c) built with the sanitizers and preloaded into a Python process that runs
  the oracle's pins (tests/test_oracle.py) against it;
* the plan and run logic of the C ABI (gemm_api.cpp, host side, sanitizers on the host pass
  only) linked with host-only kernel stand-ins (tests/asan/kernel_stubs.cpp) and driven over a
  grid of problem descriptions (tests/asan/plan_driver.cpp) and out-of-range enum values from C
  (tests/asan/enum_calls.c); no kernel is launched.
Either run fails on the first sanitizer report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None, reason="no ASan")
def test_oracle_pins_under_asan(tmp_path):
    so = tmp_path / "liboracle_asan.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=undefined", "-o", str(so),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lpthread", "-lm"], check=True)
    pre = " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    env = dict(os.environ, ORACLE_LIB=str(so), LD_PRELOAD=pre,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANGXX), reason="no hipcc")
def test_plan_logic_under_asan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    common = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), *san, "-c"]
    objs = []
    for src in (os.path.join(ROOT, "tiled_gemm_epilogues_amd", "csrc", "gemm_api.cpp"),
                os.path.join(ROOT, "tests", "asan", "kernel_stubs.cpp"),
                os.path.join(ROOT, "tests", "asan", "plan_driver.cpp")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.run(common + [src, "-o", str(obj)], check=True, capture_output=True, timeout=600)
        objs.append(str(obj))
    # the out-of-range enum calls are C (where an enum argument is any int)
    cobj = tmp_path / "enum_calls.o"
    subprocess.run([os.path.join(os.path.dirname(CLANGXX), "clang"), "-std=c11", "-O1", "-g",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-c",
                    os.path.join(ROOT, "tests", "asan", "enum_calls.c"), "-o", str(cobj)], check=True)
    objs.append(str(cobj))
    exe = tmp_path / "plan_driver"
    # clang's own sanitizer runtimes match the objects hipcc built
    subprocess.run([CLANGXX, "-fsanitize=address,undefined", "-o", str(exe), *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True,
                   capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "0 failures" in r.stdout, r.stdout
