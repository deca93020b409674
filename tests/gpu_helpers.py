"""Helpers shared by the GPU parity tests (no attention arithmetic here).

Every comparison made through ``max_abs`` or ``rel_maxnorm`` is also logged,
not gated: the mean error, the error against the oracle rounded to the
output's storage type (bf16 for O and the gradients, fp32 for LSE), and that
rounding's own size, the floor no kernel can go below.  ``conftest`` prints
the worst of them per test file at the end of the session and, when
``ATTN_PARITY_LOG`` names a file, writes every record there as JSON lines.
"""
import os
import sys

import numpy as np
import torch

from synth_inputs import bf16_bits_to_f64

# Tolerances of the parity bar: max |O_gpu - O_ref| <= 1e-2, max |LSE_gpu - LSE_ref|
# <= 1e-3, and max |G_gpu - G_ref| / max |G_ref| <= 2e-2 for G in dQ, dK, dV.
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD_REL = 2e-2


def say(msg: str) -> None:
    """Name the case about to run on the GPU, flushed, so a crash points at it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 CUDA tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_f64(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bf16_bits_to_f64(bits))


def dev_f64(t: torch.Tensor) -> torch.Tensor:
    return t.detach().float().cpu().double()


ERROR_LOG: list = []


def _storage_round(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """b rounded to a's storage type: bf16 if every value of a is a bf16 value, else fp32."""
    if a.numel() and bool((a.to(torch.bfloat16).double() == a).all()):
        return b.to(torch.bfloat16).double()
    return b.float().double()


def _log(kind: str, a: torch.Tensor, b: torch.Tensor, scale: float) -> None:
    if a.numel() == 0:
        return
    diff = (a - b).abs()
    rb = _storage_round(a, b)
    ERROR_LOG.append({
        "test": os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0],
        "kind": kind, "n": a.numel(),
        "max": float(diff.max()) / scale, "mean": float(diff.mean()) / scale,
        "max_vs_rounded_oracle": float((a - rb).abs().max()) / scale,
        "rounding_floor": float((rb - b).abs().max()) / scale,
    })


def max_abs(a: torch.Tensor, b: torch.Tensor) -> float:
    _log("abs", a, b, 1.0)
    return float((a - b).abs().max())


def rel_maxnorm(a: torch.Tensor, b: torch.Tensor, floor: float = 0.0) -> float:
    """max |a - b| / max |b|, the denominator floored at ``floor``.

    A gradient that is exactly zero in the mathematics (dQ and dK when every
    row sees a single key) has max |b| = 0; the floor -- 1e-3 times the largest
    gradient of the same problem -- keeps the ratio meaningful there and is
    far below max |b| in every other case.
    """
    den = max(float(b.abs().max()), floor, 1e-30)
    _log("rel", a, b, den)
    return float((a - b).abs().max() / den)


def bwd_head_split(attn, B: int, Hq: int, Hkv: int, N: int, d: int) -> bool:
    """Whether attn_bwd shares each K/V head's query heads out over several
    workgroups for this shape: its workspace then holds partial sums beyond the
    one fp32 D per query row (rounded up to 256 bytes)."""
    delta = (B * Hq * N * 4 + 255) // 256 * 256
    return attn.bwd_workspace_bytes(B, Hq, Hkv, N, d) > delta


def assert_same_sum_to_bf16_ulp(a: torch.Tensor, b: torch.Tensor) -> None:
    """a and b are bf16 roundings of one fp32 sum taken in two orders: each
    element may differ by one bf16 unit in the last place (at most 2^-7 of its
    magnitude), plus fp32 reassociation error (floored at 1e-4 of max |b|)."""
    x, y = a.float(), b.float()
    bound = 2.0 ** -7 * torch.maximum(x.abs(), y.abs()) + 1e-4 * float(y.abs().max())
    assert bool(((x - y).abs() <= bound).all()), float(((x - y).abs() - bound).max())


def varlen_head_split(attn, B: int, T: int, max_seqlen: int, Hq: int, Hkv: int, d: int) -> bool:
    """Whether bwd_varlen, given its default (split-size) workspace, shares each
    K/V head's query heads out over several workgroups for some mask."""
    delta = (Hq * T * 4 + 255) // 256 * 256
    return attn.bwd_varlen_split_workspace_bytes(B, T, max_seqlen, Hq, Hkv, d) > delta
