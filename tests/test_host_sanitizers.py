"""The library's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

libpakv_hostsan.so is libpakv.so with its host-only sources (the C ABI's
argument checks, the layer map, the page pools, the decode-step set-up)
compiled with -fsanitize=address,undefined.  The CPU suites that drive those
paths through the C ABI (test_abi_cpu.py, test_page_pool.py) run again in a
child process that loads it, with the ASan runtime preloaded (the Python
interpreter itself is not instrumented); any report aborts the child.  No GPU
is used: those suites make no device calls.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_logic_is_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from full_attention_amd.build import asan_runtime, library_path
    lib = library_path("hostsan")
    rt = asan_runtime()
    if not os.path.exists(lib) or rt is None:
        pytest.skip("libpakv_hostsan.so or the ASan runtime is missing (__graft_entry__.build() builds it)")
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, PAKV_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_page_pool.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
