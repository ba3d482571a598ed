"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): a
sanitized build of the library (device code unchanged) and a C++ driver that calls every entry
point on its argument-error paths and the host planners (row and state sizes, workspace plans
for every operation and layer kind, paged and contiguous caches).  A sanitizer report, or an
entry point returning another status than the driver expects, fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_host_code_is_clean_under_asan_and_ubsan():
    from long_context_attention_11_amd import build as B
    tmp = tempfile.mkdtemp(prefix="csa_san_")
    try:
        lib = B.build(out=os.path.join(tmp, "libcsa_san.so"), host_sanitize=True, jobs=6)
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, "the library is not instrumented"
        exe = os.path.join(tmp, "abi_driver")
        cmd = [CLANG, "-std=c++17", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-fno-omit-frame-pointer", "-g", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
               "-I", "/opt/rocm/include", DRIVER, "-o", exe, "-L", tmp, "-l:libcsa_san.so", "-L", "/opt/rocm/lib",
               "-lamdhip64", f"-Wl,-rpath,{tmp}", "-Wl,-rpath,/opt/rocm/lib"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "0 failures" in r.stdout
        assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
