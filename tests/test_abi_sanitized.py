"""The CPU ABI tests again, against the library whose host code (argument
checks, workspace planning, packing) is built with AddressSanitizer and
UndefinedBehaviorSanitizer (libbmoe_hostsan.so, made by the package build).
The interpreter is not instrumented, so the sanitizer runtime is preloaded in
a child process; any report fails that process."""
import os
import subprocess
import sys

import pytest

from compressed_mixture_experts_amd import build as bbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_under_host_sanitizers():
    rt = bbuild.sanitizer_runtime()
    if not os.path.exists(bbuild.LIB_HOSTSAN) or not rt:
        pytest.skip("libbmoe_hostsan.so or the sanitizer runtime is missing (build with the package build)")
    env = dict(os.environ)
    env.update({
        "BMOE_LIBRARY": bbuild.LIB_HOSTSAN,
        "LD_PRELOAD": rt,
        # the interpreter's own allocations are not checked for leaks; any
        # memory error or undefined behaviour in the library aborts
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": env.get("HIP_VISIBLE_DEVICES", ""),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
