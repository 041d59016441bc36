"""The C-ABI checks of test_abi.py against the host-sanitized build of the library
(libmla_asan.so: AddressSanitizer and UndefinedBehaviorSanitizer on the host code, that is the
argument validation, the split planning and the launch set-up). Runs in a child process with the
compiler's ASan runtime preloaded; any sanitizer report fails the test. Skipped when the sanitized
library has not been built (python mla_decode_decoupled_amd/build.py --sanitize)."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_decode_decoupled_amd")
ASAN_LIB = os.path.join(PKG, "libmla_asan.so")


def _asan_runtime():
    spec = importlib.util.spec_from_file_location("_mla_build_for_asan", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b.asan_runtime()


@pytest.mark.skipif(not os.path.exists(ASAN_LIB), reason="libmla_asan.so not built (build.py --sanitize)")
def test_abi_checks_under_address_and_ub_sanitizers():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["MLA_LIB_PATH"] = ASAN_LIB
    # the Python interpreter and the HIP runtime are not instrumented: leak reports would be theirs
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not ceilings"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    # the child really loaded the sanitized build
    probe = subprocess.run([sys.executable, "-c", "from mla_decode_decoupled_amd import _lib; print(_lib.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == ASAN_LIB, probe.stdout + probe.stderr
