"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU).

- the oracle (plain C, gcc) run over every function on small seeded inputs by
  tests/sanitize/oracle_driver.c;
- the C ABI's host side (capi.cpp: validation, the overlap checker, error
  formatting) with its host pass instrumented, linked with the built kernel
  objects and driven by tests/sanitize/capi_driver.c through calls that all
  fail validation (no device is touched).

Any out-of-bounds access, leak or undefined behaviour aborts the driver; the
test asserts a clean exit and no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "_build")
ROCM = "/opt/rocm"
KERNEL_OBJS = ["lcs_idx_score.hip.o", "lcs_topk.hip.o", "lcs_sparse_mla.hip.o",
               "lcs_cache.hip.o", "lcs_cp.hip.o"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600, **kw)
    assert r.returncode == 0, "%s\n-> rc %d\n%s" % (" ".join(cmd), r.returncode, r.stdout)
    return r.stdout


def _run_driver(exe, expect):
    env = dict(os.environ, **SAN_ENV)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300, env=env)
    out = r.stdout
    assert r.returncode == 0, "driver rc %d\n%s" % (r.returncode, out)
    for marker in ("AddressSanitizer", "LeakSanitizer", "runtime error", "SUMMARY:"):
        assert marker not in out, out
    assert expect in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    gcc_san = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off"]
    _run(gcc_san + [os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    _run_driver(exe, "oracle sanitizer driver ok")


def test_capi_host_validation_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.skip("kernel objects not built (run __graft_entry__.build()): %s" % missing)
    capi_o = str(tmp_path / "capi_san.o")
    drv_o = str(tmp_path / "capi_driver.o")
    exe = str(tmp_path / "capi_asan")
    # host pass only: the instrumentation flags go through -Xarch_host one by one
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
         ["-c", os.path.join(ROOT, "long_context_sparse_12_amd", "csrc", "capi.cpp"),
          "-o", capi_o])
    clang_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([clang, "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer"] + clang_san +
         ["-c", os.path.join(SAN, "capi_driver.c"), "-o", drv_o])
    _run([clang + "++"] + clang_san + [drv_o, capi_o] + objs +
         ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    _run_driver(exe, "capi sanitizer driver ok")
