"""Host check (no GPU) of the invariant-divisor division the kernels use for their block indices:
compiles tests/host/fastdiv_check.cpp against the kernels' header with the host C++ compiler and
runs it (edge and pseudo-random numerator/divisor pairs against integer division)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_decode_attention_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp")


def test_fast_div_matches_integer_division():
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "fastdiv_check")
        subprocess.run([cxx, "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe], check=True, capture_output=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "equal to integer division" in r.stdout
