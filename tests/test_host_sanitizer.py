"""The host side of the library (validation, layout, page bookkeeping and
rollback in duo_api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: the host ABI tests run in a child process against
a build whose host code is instrumented, with the sanitizer runtime
preloaded.  No GPU: every call there either fails validation, needs no device
work, or (without a device) fails at its first launch."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs the host tests, which expect a host without a HIP device")
    from kv_cache_duo_amd import build as b
    lib = b.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "DUO_LIBRARY": lib,
        "LD_PRELOAD": b.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    report = out
    for marker in ("ERROR: AddressSanitizer", "runtime error:"):
        at = out.find(marker)
        if at >= 0:
            report = out[max(0, at - 200):at + 3000]
            break
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, report
    assert " passed" in out
