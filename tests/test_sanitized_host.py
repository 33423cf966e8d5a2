"""The host code of the library (argument validation of every entry point,
workspace plans, the global-KV file parser) under AddressSanitizer and UBSan:
the checked build (host pass only) runs the CPU tests of the C ABI, the file
format and the binding in a child process with the sanitizer runtime
preloaded; any report aborts the child."""

import os
import shutil
import subprocess
import sys

import pytest

from compressed_sparse_attention_04_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan():
    runtime = B.sanitizer_runtime()
    if runtime is None or not os.path.exists(B.HIPCC) or shutil.which("nm") is None:
        pytest.skip("no clang sanitizer runtime / hipcc in this image")
    lib = B.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms      # the host code is instrumented
    env = dict(os.environ, CSA_LIB_PATH=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_abi_host.py", "test_kvio_host.py", "test_binding_host.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
