"""The direct global -> LDS loads write M0 from inline assembly (the LDS
destination of ``global_load_lds_dwordx4`` is M0 plus the lane offset).  M0 is
a register the compiler also allocates for its own purposes (indexed register
moves, some messages), and it cannot protect a value written behind its back:
a compiler-generated use of M0 between the asm's write and its load, or one
that expects M0 to survive the asm, would silently corrupt LDS addresses.

This test builds every kernel source for gfx950 to device assembly, exactly
as the library is built, and checks that M0 appears in one form only: the
``s_mov_b32 m0, <sgpr>`` of a TileLoader asm block, followed in the same
block by its ``global_load_lds_dwordx4``.  Any other mention of M0 fails the
test, so a compiler update or a new code path that starts using M0 is caught
before it reaches a GPU.
"""
import os
import re
import subprocess
import tempfile

import pytest

from io_aware_exact_fwd_amd import build as B

KERNEL_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [B.hipcc(), *B.DEVICE, *B.COMMON, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def m0_violations(asm: str):
    """Lines mentioning m0 outside the allowed asm-block pattern."""
    bad = []
    lines = asm.splitlines()
    in_asm = False
    pending_m0 = False      # an asm block set m0 and has not issued its load yet
    for n, raw in enumerate(lines, 1):
        line = raw.split(";", 1)[0].strip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm, pending_m0 = True, False
            continue
        if raw.strip().startswith(";;#ASMEND"):
            if pending_m0:
                bad.append((n, "asm block set m0 without a following global_load_lds_dwordx4"))
            in_asm = False
            continue
        if not line:
            continue
        mentions_m0 = re.search(r"\bm0\b", line) is not None
        if in_asm:
            if re.match(r"s_mov_b32\s+m0,\s*s\d+$", line):
                pending_m0 = True
            elif line.startswith("global_load_lds_dwordx4"):
                if not pending_m0:
                    bad.append((n, "global_load_lds_dwordx4 without its m0 write in the same block"))
                pending_m0 = False
            elif mentions_m0:
                bad.append((n, line))
        elif mentions_m0:
            bad.append((n, line))
    return bad


@pytest.fixture(scope="module")
def asm_by_source():
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(4) as ex:
        return dict(zip(KERNEL_SOURCES, ex.map(lambda s: device_asm(s, d), KERNEL_SOURCES)))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_m0_only_in_tile_loader_blocks(asm_by_source, src):
    asm = asm_by_source[src]
    assert "global_load_lds_dwordx4" in asm, f"{src}: no direct loads found (pattern changed?)"
    bad = m0_violations(asm)
    assert bad == [], f"{src}: m0 used outside the TileLoader asm blocks: {bad[:5]}"


def test_checker_flags_a_compiler_m0_use():
    """The checker itself: a compiler-generated m0 write, an asm block with a
    stray m0 use, and a load with no m0 write are all reported."""
    good = ";;#ASMSTART\n\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n;;#ASMEND\n"
    assert m0_violations(good) == []
    assert m0_violations(good + "\ts_mov_b32 m0, -1\n")
    assert m0_violations(";;#ASMSTART\n\ts_mov_b32 m0, s4\n\tv_movrels_b32 v0, v1\n;;#ASMEND\n")
    assert m0_violations(";;#ASMSTART\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n;;#ASMEND\n")
    assert m0_violations(";;#ASMSTART\n\ts_mov_b32 m0, s4\n;;#ASMEND\n")
