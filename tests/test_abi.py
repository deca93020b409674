"""The C ABI without a GPU: the library loads, exports what include/attn.h
declares, and rejects bad arguments before it makes any HIP call.

Pointers passed here are fake but aligned addresses.  Every call outside the
no-device test fails validation before a pointer could be used; the calls
whose arguments are all valid run only where no GPU exists.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def L():
    import io_aware_exact_fwd_amd as attn
    return attn.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes",
                                           "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq",
                                           "attn_bwd_grads", "attn_strerror",
                                           "attn_device_check", "attn_fwd_window",
                                           "attn_bwd_window", "attn_bwd_grads_window",
                                           "attn_fwd_decode",
                                           "attn_fwd_decode_workspace_bytes", "attn_fwd_varlen",
                                           "attn_bwd_varlen", "attn_bwd_grads_varlen", "attn_fwd_fp8",
                                           "attn_bwd_varlen_workspace_bytes",
                                           "attn_bwd_varlen_split_workspace_bytes",
                                           "attn_fwd_decode_static"])


def test_library_exports_every_declared_symbol(L):
    import io_aware_exact_fwd_amd as attn
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(attn.EXPORTED) == set(declared_functions())


def test_exports_nothing_else():
    """Only the declared C entry points are visible (the rest is hidden)."""
    import subprocess
    import io_aware_exact_fwd_amd as attn
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in syms if s.startswith("attn_")} == set(declared_functions())


A = 0x10000           # aligned fake address
MIS = 0x10008         # 8-byte aligned only


def fwd(L, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=16, d=64, causal=1, scale=0.125):
    return L.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, None)


def bwd(L, ws_bytes=None, ws=A, B=1, Hq=2, Hkv=2, N=16, d=64, scale=0.125, **ptr):
    p = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A)
    p.update(ptr)
    if ws_bytes is None:
        ws_bytes = 1 << 20
    return L.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                      ws, ws_bytes, B, Hq, Hkv, N, d, 1, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fwd_null(L, which):
    assert fwd(L, **{which: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0), dict(Hkv=0), dict(N=0), dict(N=-5), dict(d=0),
                                dict(Hq=3, Hkv=2), dict(N=1 << 25, d=128)])
def test_fwd_shape(L, kw):
    assert fwd(L, **kw) == 2


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=32), dict(q=MIS), dict(v=MIS), dict(lse=0x10004)])
def test_fwd_unsupported(L, kw):
    assert fwd(L, **kw) == 3


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan")])
def test_fwd_scale(L, scale):
    assert fwd(L, scale=scale) == 5


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null(L, which):
    assert bwd(L, **{which: None}) == 1
    assert bwd(L, ws=None) == 1


def test_bwd_workspace(L):
    # one fp32 D per query row, rounded up to 256 bytes: O(N), not O(N^2)
    assert L.attn_bwd_workspace_bytes(1, 8, 8, 32768, 128) == 8 * 32768 * 4
    assert L.attn_bwd_workspace_bytes(1, 3, 3, 10, 64) == 256
    assert L.attn_bwd_workspace_bytes(4, 8, 4, 2048, 128) == 4 * 8 * 2048 * 4
    # with the head split, S fp32 partial dK and dV per key row after D:
    # 32 query heads over 1 K/V head split 16 ways, 8 over 2 (B=2) 4 ways
    assert L.attn_bwd_workspace_bytes(1, 32, 1, 8192, 128) == 32 * 8192 * 4 + 16 * 2 * 8192 * 128 * 4
    need = L.attn_bwd_workspace_bytes(2, 8, 2, 1000, 128)
    assert need == 2 * 8 * 1000 * 4 + 4 * 2 * (2 * 2 * 1000) * 128 * 4
    assert bwd(L, B=2, Hq=8, Hkv=2, N=1000, d=128, ws_bytes=need - 1) == 4


def _splits(L, B, Hq, Hkv, N, d):
    """The head split count the workspace size encodes (the most either mask takes)."""
    delta = (B * Hq * N * 4 + 255) // 256 * 256
    extra = L.attn_bwd_workspace_bytes(B, Hq, Hkv, N, d) - delta
    per_split = 2 * B * Hkv * N * d * 4
    assert extra % per_split == 0
    return max(1, extra // per_split)


def test_bwd_head_split_rule(L):
    """The split count: causal, the divisor S of G = Hq/Hkv minimising
    S + 16G/(B*Hkv*S), at most 2048 key blocks once 256 are reached; otherwise
    the fewest splits giving 256 blocks of 128 keys."""
    assert _splits(L, 1, 32, 1, 8192, 128) == 16      # 16 and 32 tie: the smaller
    assert _splits(L, 1, 8, 1, 32768, 128) == 8
    assert _splits(L, 1, 32, 4, 8192, 128) == 4
    assert _splits(L, 1, 31, 1, 8192, 128) == 31      # prime group: all or nothing
    assert _splits(L, 1, 64, 8, 16384, 128) == 2      # 4 would pass 2048 blocks
    assert _splits(L, 4, 32, 8, 4096, 128) == 1       # 1 and 2 tie
    assert _splits(L, 1, 8, 8, 32768, 128) == 1       # no grouping
    assert _splits(L, 1, 32, 1, 8192, 64) == 16       # the same at d = 64
    assert _splits(L, 2, 16, 2, 4096, 128) == 4       # causal 4, full 2: the larger
    assert L.attn_bwd_workspace_bytes(1, 3, 2, 10, 64) == 0      # invalid problem -> 0


def test_bwd_shape_and_scale(L):
    assert bwd(L, Hq=4, Hkv=3) == 2
    assert bwd(L, d=80) == 3
    assert bwd(L, dk=MIS) == 3
    assert bwd(L, scale=float("nan")) == 5


def test_stage_argument_errors(L):
    assert L.attn_bwd_preprocess(None, A, A, 1, 2, 16, 64, None) == 1
    assert L.attn_bwd_preprocess(A, A, A, 1, 2, 16, 96, None) == 3
    assert L.attn_bwd_preprocess(A, A, A, 1, 0, 16, 64, None) == 2
    assert L.attn_bwd_preprocess(A, MIS, A, 1, 2, 16, 64, None) == 3
    args = [A] * 8
    assert L.attn_bwd_dkdv(*args, 1, 4, 3, 16, 128, 1, 0.1, None) == 2
    assert L.attn_bwd_dkdv(*args[:6], None, A, 1, 4, 2, 16, 128, 1, 0.1, None) == 1
    assert L.attn_bwd_dkdv(*args, 1, 4, 2, 16, 128, 1, -0.1, None) == 5
    assert L.attn_bwd_dq(*args[:7], 1, 4, 2, 16, 128, 1, float("inf"), None) == 5
    assert L.attn_bwd_dq(*args[:6], MIS, 1, 4, 2, 16, 128, 1, 0.1, None) == 3
    assert L.attn_bwd_dq(A, A, A, A, None, A, A, 1, 4, 2, 16, 128, 1, 0.1, None) == 1
    args = [A] * 9
    assert L.attn_bwd_grads(*args, 1, 4, 3, 16, 128, 1, 0.1, None) == 2
    assert L.attn_bwd_grads(*args[:8], None, 1, 4, 2, 16, 128, 1, 0.1, None) == 1
    assert L.attn_bwd_grads(*args[:7], MIS, A, 1, 4, 2, 16, 128, 1, 0.1, None) == 3
    assert L.attn_bwd_grads(*args, 1, 4, 2, 16, 100, 1, 0.1, None) == 3
    assert L.attn_bwd_grads(*args, 1, 4, 2, 16, 128, 1, 0.0, None) == 5


def test_strerror(L):
    for code in range(0, 8):
        s = L.attn_strerror(code)
        assert s and len(s) > 1
    assert b"unknown" in L.attn_strerror(99)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_hip_error(L):
    """All arguments valid, no GPU: the device check fails with ATTN_ERR_HIP or
    ATTN_ERR_UNSUPPORTED -- it never falls back to another path.  The pointers
    are fake, so these calls run only where no device exists (where one does,
    they would reach a launch)."""
    rc = fwd(L)
    assert rc in (3, 6)
    assert L.attn_device_check(0) in (3, 6)
    #                      q  k  v  o  lse cu B  T    max Hq Hkv d  causal win scale
    assert L.attn_fwd_varlen(A, A, A, A, A, A, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) in (3, 6)
    assert L.attn_bwd_varlen(*([A] * 10), A, 4 * 100 * 4, 2, 100, 60, 4, 2, 64, 1, -1, 0.1,
                             None) in (3, 6)
    assert L.attn_bwd_grads_varlen(*([A] * 10), 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) in (3, 6)
    #                     q  k  v  qd kd vd o  lse B  Hq Hkv N   d   causal scale
    assert L.attn_fwd_fp8(A, A, A, A, A, A, A, A, 1, 4, 2, 64, 128, 1, 0.1, None) in (3, 6)


def test_window_entry_points_validate(L):
    """Windowed calls: the plain calls' checks plus window >= 0, all before any
    device work."""
    # negative window
    assert L.attn_fwd_window(A, A, A, A, A, 1, 2, 2, 16, 64, 1, -1, 0.1, None) == 2
    assert L.attn_bwd_window(A, A, A, A, A, A, A, A, A, A, 1 << 20, 1, 2, 2, 16, 64, 1, -3, 0.1, None) == 2
    assert L.attn_bwd_grads_window(*([A] * 9), 1, 2, 2, 16, 64, 1, -1, 0.1, None) == 2
    # the plain checks still apply
    assert L.attn_fwd_window(None, A, A, A, A, 1, 2, 2, 16, 64, 1, 4, 0.1, None) == 1
    assert L.attn_fwd_window(A, A, A, A, A, 1, 3, 2, 16, 64, 1, 4, 0.1, None) == 2
    assert L.attn_fwd_window(A, A, A, A, A, 1, 2, 2, 16, 96, 1, 4, 0.1, None) == 3
    assert L.attn_fwd_window(A, A, A, A, A, 1, 2, 2, 16, 64, 1, 4, 0.0, None) == 5
    assert L.attn_bwd_window(A, A, A, A, A, A, A, A, A, A, 0, 1, 2, 2, 16, 64, 1, 4, 0.1, None) == 4
    assert L.attn_bwd_grads_window(*([A] * 8), MIS, 1, 2, 2, 16, 64, 1, 4, 0.1, None) == 3


def test_decode_validation_and_workspace(L):
    """Decode: shape rules (Nq <= Nk), workspace sizing, errors before device work."""
    ws = L.attn_fwd_decode_workspace_bytes
    # automatic split count: the workspace holds (d + 1) floats per row per chunk
    n = ws(2, 8, 2, 1, 4096, 128, 0)
    assert n > 0 and n % (2 * 8 * 1 * 129 * 4) == 0
    chunks = n // (2 * 8 * 1 * 129 * 4)
    assert 1 <= chunks <= 4096 // 128
    assert ws(1, 4, 4, 3, 1000, 64, 1) == 1 * 4 * 3 * 65 * 4          # one chunk
    assert ws(1, 4, 4, 3, 1000, 64, 100) == 8 * 4 * 3 * 65 * 4        # at most one chunk per tile
    assert ws(1, 4, 4, 5, 4, 64, 0) == 0                               # Nq > Nk
    assert ws(1, 4, 3, 1, 4, 64, 0) == 0                               # Hq % Hkv
    args = [A] * 5
    assert L.attn_fwd_decode(*args, 1, 4, 4, 5, 4, 64, 1, -1, 0.1, 0, A, 1 << 20, None) == 2
    assert L.attn_fwd_decode(*args, 1, 4, 4, 1, 64, 96, 1, -1, 0.1, 0, A, 1 << 20, None) == 3
    assert L.attn_fwd_decode(*args, 1, 4, 4, 1, 64, 64, 1, -1, 0.1, 0, None, 1 << 20, None) == 1
    assert L.attn_fwd_decode(*args, 1, 4, 4, 1, 64, 64, 1, -1, 0.1, 0, A, 16, None) == 4
    assert L.attn_fwd_decode(*args, 1, 4, 4, 1, 64, 64, 1, -1, -1.0, 0, A, 1 << 20, None) == 5
    assert L.attn_fwd_decode(A, A, MIS, A, A, 1, 4, 4, 1, 64, 64, 1, -1, 0.1, 0, A, 1 << 20, None) == 3



def test_decode_static_validation(L):
    """The decode call without a workspace: the same argument checks as
    attn_fwd_decode, and a problem whose partials exceed the static scratch is
    refused (ATTN_ERR_SCRATCH) before any device work."""
    f = L.attn_fwd_decode_static
    ws = L.attn_fwd_decode_workspace_bytes
    #        q  k  v  o  lse B   Hq  Hkv Nq  Nk    d    causal win scale splits
    assert f(A, A, A, A, None, 1, 4, 4, 1, 64, 64, 1, -1, 0.1, 0, None) == 1
    assert f(A, A, A, A, A, 1, 4, 4, 5, 4, 64, 1, -1, 0.1, 0, None) == 2           # Nq > Nk
    assert f(A, A, A, A, A, 1, 4, 3, 1, 64, 64, 1, -1, 0.1, 0, None) == 2          # Hq % Hkv
    assert f(A, A, A, A, A, 1, 4, 4, 1, 64, 96, 1, -1, 0.1, 0, None) == 3          # d
    assert f(A, A, MIS, A, A, 1, 4, 4, 1, 64, 64, 1, -1, 0.1, 0, None) == 3        # alignment
    assert f(A, A, A, A, A, 1, 4, 4, 1, 64, 64, 1, -1, -1.0, 0, None) == 5         # scale
    big = (64, 64, 64, 16, 4096, 128)
    assert ws(*big, 32) > 32 << 20
    assert f(A, A, A, A, A, *big, 1, -1, 0.1, 32, None) == 7                       # scratch too small
    assert b"static" in L.attn_strerror(7) or b"STATIC" in L.attn_strerror(7)


def test_varlen_validation_and_workspace(L):
    """Packed batches: shape rules, the empty batch, workspace size, all
    before any device work."""
    assert L.attn_bwd_varlen_workspace_bytes(8, 1000, 128) == 8 * 1000 * 4
    assert L.attn_bwd_varlen_workspace_bytes(8, 1000, 96) == 0
    assert L.attn_bwd_varlen_workspace_bytes(0, 1000, 128) == 0
    # the size that allows the head split: D rounded to 256 bytes, then S
    # partial dK/dV planes [2, Hkv, total, d] fp32 -- 32 heads over 1 K/V head,
    # 8192 packed rows in sequences of at most 4096 (two at that length): 16
    sp = L.attn_bwd_varlen_split_workspace_bytes
    assert sp(4, 8192, 4096, 32, 1, 128) == 32 * 8192 * 4 + 16 * 2 * 8192 * 128 * 4
    assert sp(4, 8192, 4096, 8, 8, 128) == 8 * 8192 * 4          # no grouping: no split
    assert sp(2, 1000, 600, 3, 3, 64) == (3 * 1000 * 4 + 255) // 256 * 256
    assert sp(2, 100, 200, 4, 2, 64) == 0                         # max_seqlen > total
    assert sp(2, 100, 60, 4, 2, 96) == 0                          # d
    f = L.attn_fwd_varlen
    #         q  k  v  o  lse cu   B  T    max Hq Hkv d  causal win scale
    assert f(A, A, A, A, A, A, 0, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 2        # B = 0
    assert f(A, A, A, A, A, A, 2, 100, 101, 4, 2, 64, 1, -1, 0.1, None) == 2       # max > total
    assert f(A, A, A, A, A, A, 2, 100, 0, 4, 2, 64, 1, -1, 0.1, None) == 2         # max = 0 < total
    assert f(A, A, A, A, A, A, 2, 100, 60, 4, 3, 64, 1, -1, 0.1, None) == 2        # Hq % Hkv
    assert f(A, A, A, A, A, A, 2, 100, 60, 4, 2, 96, 1, -1, 0.1, None) == 3        # d
    assert f(A, A, A, A, A, None, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 1     # no table
    assert f(A, A, MIS, A, A, A, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 3      # alignment
    assert f(A, A, A, A, A, A, 2, 100, 60, 4, 2, 64, 1, -1, 0.0, None) == 5        # scale
    assert f(None, None, None, None, None, None, 3, 0, 0, 4, 2, 64, 1, -1, 0.1, None) == 0  # empty batch
    assert f(A, A, A, A, A, A, 2, 1 << 25, 60, 4, 2, 128, 1, -1, 0.1, None) == 2   # total * d > 2^31
    b = L.attn_bwd_varlen
    ptrs = [A] * 10
    assert b(*ptrs, A, 4 * 100 * 4 - 1, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 4
    assert b(*ptrs[:9], None, A, 1 << 20, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 1
    assert b(*ptrs, A, 1 << 20, 2, 100, 200, 4, 2, 64, 1, -1, 0.1, None) == 2
    assert b(*([None] * 10), None, 0, 2, 0, 0, 4, 2, 64, 1, -1, 0.1, None) == 0
    g = L.attn_bwd_grads_varlen
    assert g(*([A] * 9), None, 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 1
    assert g(*([A] * 10), 2, 100, 60, 4, 2, 64, 1, -1, -2.0, None) == 5
    assert g(*([A] * 5), MIS, *([A] * 4), 2, 100, 60, 4, 2, 64, 1, -1, 0.1, None) == 3


def test_fp8_validation(L):
    f = L.attn_fwd_fp8
    #         q  k  v  qd kd vd o  lse B  Hq Hkv N   d   causal scale
    assert f(A, A, A, A, A, A, A, A, 1, 4, 2, 64, 64, 1, 0.1, None) == 3         # d = 64: 8-bit path is d = 128
    assert f(A, A, A, None, A, A, A, A, 1, 4, 2, 64, 128, 1, 0.1, None) == 1     # descale missing
    assert f(A, A, A, A, A, A, A, A, 1, 4, 3, 64, 128, 1, 0.1, None) == 2        # Hq % Hkv
    assert f(A, MIS, A, A, A, A, A, A, 1, 4, 2, 64, 128, 1, 0.1, None) == 3      # alignment
    assert f(A, A, A, A, A, A, A, A, 1, 4, 2, 64, 128, 1, float("nan"), None) == 5


def test_library_imports_no_allocation_or_copy():
    """The library's only device work is kernel launches: it imports no
    allocator and no copy or fill routine (host or device), so every buffer is
    the caller's and no call hides an allocation or a transfer."""
    import shutil
    import subprocess

    import io_aware_exact_fwd_amd as attn
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", attn.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    names = [line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()]
    assert "hipLaunchKernel" in names
    bad = [n for n in names if re.search(r"(?i)alloc|free|memcpy|memset|hostregister|mmap", n)]
    assert bad == [], bad


def test_autograd_entry_points_reject_host_tensors():
    """The differentiable wrappers validate like the direct calls: host tensors
    are refused before anything reaches the library."""
    import io_aware_exact_fwd_amd as attn
    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attention(q, q, q)
    qp = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attention_varlen(qp, qp, qp, [0, 3, 8], 5)
