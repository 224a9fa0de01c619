"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer: the
CPU ABI tests (validation of every entry point, exact capacity, sizing and workspace
layout, the replica plan, the allocation-free entry point's refusals) run in a child
process against a library whose abi.hip host code is instrumented; any sanitizer report
aborts the child and fails this test. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "expert_routing_amd"))


def test_abi_checks_clean_under_asan_ubsan():
    import build_sanitized as BS
    if BS.runtime_library() is None:
        pytest.skip("no ASan runtime next to the ROCm clang")
    lib = BS.build_sanitized()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=BS.runtime_env(lib), cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail
