"""Host logic of packed launches: the grid bound covers every real block.

Batches of up to 512 packed sequences are launched over their real blocks
only; the host sizes the grid by heads * (ceil(T / BS) + B) when that is
smaller than the plain (sequence, head, block) grid.  `packed_grid_check.cpp`
checks the bound on 4000 seeded boundary tables (up to 700 sequences, empty
ones included, three block sizes) with the library's own header; this test
compiles and runs it with the host compiler.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_packed_grid_covers_every_real_block(tmp_path):
    exe = tmp_path / "packed_grid_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
                    "-I", os.path.join(ROOT, "io_aware_exact_fwd_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "packed_grid_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:")
