"""The host C++ of the library (tree compile and node budget) under AddressSanitizer and
UndefinedBehaviorSanitizer: the host-library tests, including every invalid-spec and
short-buffer case, run against a sanitized CPU-only build of csrc/tree_compile.cpp in a
child process with the ASan runtime preloaded.  Any report fails the test.

[M7.2] §0x06D asks that a step validate everything before it mutates anything; the tree
compiler does index-heavy work on caller buffers, which is what the sanitizers watch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CHILD = """
import sys
sys.path.insert(0, {root!r})
import medusa_tree_attention_amd._binding as B
B.LIBRARY = {lib!r}
B._SIGNATURES = {{k: v for k, v in B._SIGNATURES.items() if k in ("medusa_tree_compile", "medusa_tree_budget")}}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py", "tests/test_budget.py",
                      "-k", "not every_declared_symbol"]))
"""


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_library_is_clean_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("the ASan runtime is not installed")
    from medusa_tree_attention_amd import build
    lib = build.build_host_sanitized(verbose=False)
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in out, out[-4000:]
