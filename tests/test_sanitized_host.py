"""The CPU tier again, on the library's host code built with AddressSanitizer
and UndefinedBehaviorSanitizer (head_heterogeneous_block_amd/build_sanitize.py):
any sanitizer report aborts the child run and fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.sanitize


def test_cpu_tier_clean_under_sanitizers():
    if not shutil.which("hipcc") and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "head_heterogeneous_block_amd", "build_sanitize.py"), "-x"],
                       cwd=ROOT, capture_output=True, text=True, timeout=1500)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-40:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
