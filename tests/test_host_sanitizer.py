"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

api.cpp (argument validation, workspace layouts, the no-allocation scratch
set-up) is rebuilt with host-side ASan + UBSan (build.py build_sanitized), and
the ABI validation tests run against that build in a child process with the
shared ASan runtime preloaded.  Every call there is rejected on the host before
any HIP call, so no GPU is needed; any sanitizer report fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "activation_sparse_transformer_bf16_amd"))


def _hipcc_present():
    return os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc") is not None


@pytest.mark.skipif(not _hipcc_present(), reason="hipcc is needed to build the sanitizer variant")
def test_abi_validation_clean_under_asan_and_ubsan():
    import build as twell_build
    lib = twell_build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": twell_build.asan_runtime(),
        "TWELL_LIBRARY": lib,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    # the child processes load the sanitizer build
    r = subprocess.run([sys.executable, "-c", "import activation_sparse_transformer_bf16_amd as t; print(t.LIB_PATH)"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
