"""The C ABI's host code under AddressSanitizer (CPU only).

Builds libdropkv_asan.so (the host code of every source compiled with
-fsanitize=address for the host only; device code unchanged), then runs the
host-side ABI tests (argument validation, workspace sizing, error text,
symbol exports) against it in a child process with the clang ASan runtime
preloaded. Any heap or stack error in the host code fails the child.
"""

import os
import subprocess
import sys

import pytest

from kv_cache_eviction_pass1_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan():
    try:
        rt = build.asan_runtime()
        build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build(variant="asan")
    assert b"__asan_report" in subprocess.run(["nm", "-D", lib], capture_output=True).stdout
    # the ASan runtime must come first; anything already preloaded stays after it
    pre = rt + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    env = dict(os.environ, LD_PRELOAD=pre, DROPKV_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
