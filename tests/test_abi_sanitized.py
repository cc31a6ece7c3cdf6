"""The host-side C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library variant built with api.cpp instrumented (build(variant="san"),
host code only) runs tests/test_abi.py in a child process with the clang ASan
runtime preloaded; any memory error or undefined behaviour in argument
validation, workspace sizing or the other host paths aborts that run.  No GPU
is needed: nothing in test_abi.py reaches a kernel launch.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers():
    sys.path.insert(0, ROOT)
    from block_sparse_attention_meanpool_amd import build as b
    lib = b.build(variant="san")
    rt = b.san_runtime()
    if not os.path.exists(rt):
        pytest.skip(f"clang ASan runtime not found ({rt})")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out
    # the child loaded the sanitized build, and it is instrumented
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm
