"""The oracle and the host C++ of the library (scheduler, table checks,
status text) built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc/g++, host code only: no device code is built with a sanitizer) and run
through their CPU tests in a child process: the oracle's pins, the scheduler
against its ownership model, and the table checker's accept and reject
cases.  Any out-of-bounds access, use after free or undefined behaviour
aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc has no AddressSanitizer runtime")
def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    from paged_kv_cache_193_amd import build as pbuild
    olib = obuild.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    hlib = pbuild.build_host_sanitized(str(tmp_path / "libpkvhost_asan.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime("libasan.so"),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PKV_ORACLE_LIB": olib,
        "PKV_HOST_LIB": hlib,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "tests/test_oracle_pins.py", "tests/test_scheduler.py", "tests/test_host_checks.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
