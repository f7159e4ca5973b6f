"""The C-ABI front end under host AddressSanitizer and UndefinedBehaviorSanitizer.

The library is built again with its host code instrumented, and the host-side
ABI checks (argument validation, workspace queries, the split plans, tuning,
the binding's shape checks, the no-alloc entry point's refusal) run against it
in a child process with the ASan runtime preloaded. Any sanitizer report stops
the child with a non-zero status. No GPU is needed.
"""
import os
import subprocess
import sys

import pytest

from full_gqa_attention_layer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
from full_gqa_attention_layer_amd import hgqa
hgqa.load_library({lib!r})
import pytest
sys.exit(pytest.main(['-q', '-s', '-m', 'not gpu', '-p', 'no:cacheprovider',
                      'tests/test_abi.py', 'tests/test_zz_no_alloc.py']))
"""


def test_abi_checks_under_host_sanitizers(tmp_path):
    rt = build.asan_runtime()
    if not rt:
        pytest.skip("the clang ASan runtime is not installed")
    lib = build.build_sanitized(str(tmp_path / "libhgqa_sanitized.so"))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
