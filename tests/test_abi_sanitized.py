"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with both sanitizers on its host side (the checking build
of ``block_drafting_sd_amd.build``; device code unchanged), then runs the
whole ABI suite (``tests/test_abi.py``: exports, argument validation of every
entry point, workspace sizing, binding checks) in a child process that loads
that build with the sanitizer runtime preloaded.  Any heap, stack or global
overflow, use after free or undefined behaviour in the validation layer
aborts the child.  No GPU is needed: validation never touches a device.
"""
import os
import subprocess
import sys

from block_drafting_sd_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers():
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update(SD_LIB_PATH=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and \
        "runtime error" not in r.stderr, tail
