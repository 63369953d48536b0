"""The oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: builds both with sanitized host code and runs the
oracle pins and the C-ABI validation tests against those builds in a child
process (tests/run_sanitized.py).  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_cpu_checks_clean_under_asan_ubsan():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "run_sanitized.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert "runtime error" not in r.stdout + r.stderr, tail  # UBSan's report prefix
    assert " passed" in r.stdout, tail
