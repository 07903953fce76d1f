"""The host-side code of the library (argument checks, closed-form sizes, status
strings, launch set-up up to the first HIP call) under AddressSanitizer and
UndefinedBehaviorSanitizer: the ABI tests run again, in a child interpreter with
the ASan runtime preloaded, against a sanitized build.  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_checks_under_host_sanitizers():
    from swa_memory_anchor_amd import build_sanitized as S

    lib = S.build_sanitized()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_handle_" in nm, "library is not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = S.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import swa_memory_anchor_amd as R\n"
            "R.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py")))
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=600, cwd=ROOT)
    finally:
        shutil.rmtree(os.path.dirname(lib), ignore_errors=True)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
