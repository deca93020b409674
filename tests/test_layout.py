"""Host-side check of the LDS layout / MFMA operand address math (no GPU).

Compiles tests/layout_check.cpp against the kernels' own layout header with the
host C++ compiler and runs it: every lane of every fragment read must receive
exactly the elements its MFMA operand needs, with no LDS bank conflicts.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layout_math(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "layout_check"
    subprocess.run([cxx, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "io_aware_exact_fwd_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK" in r.stdout
