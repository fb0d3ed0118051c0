"""The ABI's CPU tests (argument validation and every rejection path of
tests/test_abi_cpu.py) rerun against a build whose host code in attn_api.hip
is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(non-recoverable), in a child process with the sanitizer runtime preloaded.
A memory error or undefined behaviour in the host validation aborts it."""

import os
import subprocess
import sys

import pytest

from online_softmax_exact_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    res = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_under_asan_and_ubsan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    if not all(os.path.exists(os.path.join(B.OUT_DIR, os.path.basename(s)[:-4] + ".o"))
               for s in B.sources()):
        B.build()
    lib = B.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, ATTN_MI355X_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # The child maps the instrumented library and the sanitizer runtime.
    probe = ("from online_softmax_exact_amd import _lib; _lib.load_library(); "
             "maps = open('/proc/self/maps').read(); "
             f"assert {lib!r} in maps, 'sanitized library not loaded'; "
             "assert 'libclang_rt.asan' in maps, 'sanitizer runtime not loaded'; print('ok')")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0 and "ok" in res.stdout, res.stdout + res.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "passed" in res.stdout and "failed" not in res.stdout
