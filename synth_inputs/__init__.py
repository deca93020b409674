"""Seeded synthetic inputs shared by the CPU oracle, the tests and the bench.

This module holds no attention arithmetic: it only draws normal samples, scales
them and rounds them to bfloat16.  Both the oracle and the GPU library consume
the exact same bf16 values that come out of here, so a parity test compares the
two implementations of one function on one input.

Recipe (per workload, per seed):
  * generator  ``numpy.random.Generator(numpy.random.PCG64(seed))``;
  * draw order ``Q, K, V[, dO]``, each ``standard_normal(shape, dtype=float32)``
    in C order over ``[B, H, N, d]`` (Q and dO use H = H_q, K and V use H_kv);
  * multiply by the workload's input scale (1.0, or 0.5 -- exact in binary);
  * round fp32 -> bf16 to nearest, ties to even, with integer bit operations.

Packed variable-length batches draw the same way over ``[H, T, d]`` (T the
packed token count; identical values to the ``[1, H, T, d]`` draw) and add
``cu_seqlens``; their sequence lengths come from ``pack_lengths``: a
generator ``PCG64(seed)`` draws ``exp(uniform(ln lo, ln hi))`` rounded to an
integer, one length at a time, until the pack holds T tokens (the last length
is cut to fit).

8-bit inputs (OCP E4M3) draw the same fp32 values, then per (batch, head):
``descale = max|x| / 448`` (fp32) and ``code = E4M3(x / descale)``, rounded to
the nearest representable value, ties to even (``f32_to_e4m3_bits``).

Very large inputs (tensors of several GiB, drawn where they are used) come
from ``hashed_bf16_bits``: element i of a stream with seed s is the SplitMix64
output for state s + (i + 1) * 0x9E3779B97F4A7C15, whose low 16 bits give a
sign, a power of two in [1/8, 1] and 7 mantissa bits.  It uses integer
operations only, so a GPU and the CPU produce the same bits for any slice.

The bf16 payload is returned as ``uint16`` bit patterns; ``bf16_bits_to_f32``
and ``bf16_bits_to_f64`` decode them exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "draw_normal_f32",
    "make_inputs",
    "make_custom_inputs",
    "pack_lengths",
    "cu_from_lengths",
    "f32_to_e4m3_bits",
    "make_fp8_inputs",
    "hashed_bf16_bits",
    "splitmix64_reference",
]


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, input scale, seed and masking."""

    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: Tuple[bool, ...]
    seed: int
    in_scale: float = 1.0
    with_grad: bool = False
    note: str = ""
    window: Optional[int] = None    # sliding window |i - j| <= window, or none
    nq: Optional[int] = None        # queries, when fewer than the N keys (decoding)
    # packed variable-length batch: N tokens split into sequences whose lengths
    # are drawn log-uniform in [lo, hi] (pack_lengths with this seed); B = 1
    pack: Optional[Tuple[int, int]] = None
    fp8: bool = False               # Q, K, V as E4M3 codes with per-head descales

    def lengths(self) -> List[int]:
        """Sequence lengths of a packed workload (one sequence of N otherwise)."""
        if self.pack is None:
            return [self.N]
        return pack_lengths(self.N, self.seed, *self.pack)

    def keys_per_query(self, causal: bool) -> int:
        """Visible keys summed over the query rows of one head (a count)."""
        if self.pack is not None:
            return sum(self._keys(n, causal) for n in self.lengths())
        return self._keys(self.N, causal)

    def _keys(self, n: int, causal: bool) -> int:
        w = self.window
        if self.nq is not None:
            if w is not None:
                raise ValueError("windowed decode workloads are not defined")
            m = self.nq      # queries at positions n - m .. n - 1
            return m * (n - m) + m * (m + 1) // 2 if causal else m * n
        if w is None or w >= n - 1:
            return n * (n + 1) // 2 if causal else n * n
        left = (w + 1) * (w + 2) // 2 + (n - w - 1) * (w + 1)     # keys j in [i - w, i]
        if causal:
            return left
        return 2 * left - n                                           # plus [i, i + w], i counted once

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def pairs(self, causal: bool) -> int:
        """Unmasked (query, key) pairs over all (batch, query head)."""
        return self.B * self.Hq * self.keys_per_query(causal)

    def fwd_flops(self, causal: bool) -> int:
        """Algorithmic matmul FLOPs of the forward: 2d for QK^T plus 2d for PV."""
        return 4 * self.d * self.pairs(causal)

    def bwd_flops(self, causal: bool) -> int:
        """Algorithmic matmul FLOPs of the backward: S, dP, dV, dQ and dK."""
        return 10 * self.d * self.pairs(causal)


# The five problems the benchmark and the parity suite are built around.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny", 1, 2, 2, 256, 64, (True, False), seed=0,
                 note="fp32 N(0,1) draws; the GPU sees their bf16 rounding"),
        Workload("fwd-2K", 4, 16, 16, 2048, 128, (True,), seed=1),
        Workload("fwd-8K", 1, 32, 32, 8192, 128, (True,), seed=2, in_scale=0.5),
        Workload("gqa-16K", 1, 64, 8, 16384, 128, (True,), seed=3),
        Workload("fb-32K", 1, 8, 8, 32768, 128, (True,), seed=4, with_grad=True),
        Workload("swa-32K", 1, 8, 8, 32768, 128, (True,), seed=5, with_grad=True, window=4096,
                 note="sliding-window causal attention, 4096 keys back"),
        Workload("decode-32K", 16, 32, 8, 32768, 128, (True,), seed=6, nq=1,
                 note="one new query per sequence against a 32768-key cache"),
        Workload("fp8-8K", 1, 32, 32, 8192, 128, (True,), seed=8, fp8=True,
                 note="E4M3 inputs with one descale per (batch, head)"),
        Workload("varlen-32K", 1, 8, 8, 32768, 128, (True,), seed=7, with_grad=True,
                 pack=(512, 16384),
                 note="32768 tokens packed from sequences of 512..16384 tokens (log-uniform)"),
    )
}


def pack_lengths(total: int, seed: int, lo: int, hi: int) -> List[int]:
    """Seeded sequence lengths, log-uniform in [lo, hi], that fill ``total``."""
    if not (1 <= lo <= hi) or total < 0:
        raise ValueError("need 1 <= lo <= hi and total >= 0")
    rng = np.random.Generator(np.random.PCG64(seed))
    out: List[int] = []
    left = total
    while left > 0:
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = min(max(n, 1), left)
        out.append(n)
        left -= n
    return out


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round values to OCP E4M3 (nearest, ties to even); return uint8 codes.

    Every value must round to at most 448 in magnitude (no saturation here).
    The rounding works on the format's grid: spacing 2^-9 below 2^-6, and
    2^(e-3) in the binade [2^e, 2^(e+1)).  The quotient by a power of two is
    exact in float64, and numpy's rint rounds half to even.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    neg = np.signbit(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))       # a = f * 2^ex, f in [0.5, 1)
    step = np.ldexp(1.0, ex - 1 - 3)
    q = np.rint(a / step) * step
    if bool((q > 448.0).any()):
        raise ValueError("value beyond the E4M3 range (448)")
    _, eq = np.frexp(np.where(q > 0, q, 1.0))
    e_field = np.where(q >= 2.0 ** -6, eq - 1 + 7, 0)
    mant = np.where(q >= 2.0 ** -6, q / np.ldexp(1.0, eq - 1 - 3) - 8, q / 2.0 ** -9)
    code = (e_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(q == 0, 0, code) | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def make_fp8_inputs(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int) -> Dict[str, np.ndarray]:
    """E4M3 codes for Q, K, V ([B, H, N, d] uint8) and their fp32 descales ([B, H])."""
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed, keep_f32=True)
    out: Dict[str, np.ndarray] = {}
    for name in ("q", "k", "v"):
        f = x[name + "_f32"]
        amax = np.abs(f).max(axis=(2, 3))
        descale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        out[name + "8"] = f32_to_e4m3_bits(f.astype(np.float64) / descale.astype(np.float64)[:, :, None, None])
        out[name + "_descale"] = descale
    return out


_GOLDEN = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1


def splitmix64_reference(seed: int, i: int) -> int:
    """SplitMix64 output number i (0-based) of a generator seeded with `seed`,
    in plain Python integers (the published definition)."""
    z = (seed + (i + 1) * _GOLDEN) & _M64
    z = ((z ^ (z >> 30)) * _MIX1) & _M64
    z = ((z ^ (z >> 27)) * _MIX2) & _M64
    return z ^ (z >> 31)


def _signed(c: int) -> int:
    return c - (1 << 64) if c >= (1 << 63) else c


def _lsr(z, s: int):
    """Logical right shift of int64 tensors (torch's >> is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def hashed_bf16_bits(start: int, count: int, seed: int, device="cpu", chunk: int = 1 << 26):
    """bf16 bit patterns (torch.int16) of stream elements start .. start+count-1.

    Low 16 bits h of the SplitMix64 output: sign = bit 15, exponent field
    124 + bits 7..8 (a power of two in [1/8, 1]), mantissa = bits 0..6.
    int64 arithmetic wraps identically on every device.
    """
    import torch
    out = torch.empty(count, dtype=torch.int16, device=device)
    g, m1, m2 = _signed(_GOLDEN), _signed(_MIX1), _signed(_MIX2)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        i = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=device)
        z = (i + 1) * g + _signed(seed & _M64)
        z = (z ^ _lsr(z, 30)) * m1
        z = (z ^ _lsr(z, 27)) * m2
        z = z ^ _lsr(z, 31)
        h = z & 0xFFFF
        bits = ((h >> 15) << 15) | ((124 + ((h >> 7) & 3)) << 7) | (h & 0x7F)
        out[c0:c0 + n] = (bits - ((bits >> 15) << 16)).to(torch.int16)   # as signed 16-bit
        del i, z, h, bits
    return out


def cu_from_lengths(lengths) -> np.ndarray:
    """Sequence boundaries [0, n0, n0 + n1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite.  The rounding adds 0x7FFF plus the lowest kept bit to the
    32-bit pattern and keeps the upper half, which is round-half-to-even on the
    16 discarded bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly to fp64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def draw_normal_f32(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_custom_inputs(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int,
                       in_scale: float = 1.0, with_grad: bool = False,
                       keep_f32: bool = False) -> Dict[str, np.ndarray]:
    """Draw Q, K, V (and dO) for an arbitrary shape with the recipe above.

    Returns ``{"q","k","v"[,"do"]}`` as uint16 bf16 bit arrays; with
    ``keep_f32`` also ``"q_f32"`` ... holding the unrounded fp32 draws.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = {"q": (B, Hq, N, d), "k": (B, Hkv, N, d), "v": (B, Hkv, N, d)}
    if with_grad:
        shapes["do"] = (B, Hq, N, d)
    out: Dict[str, np.ndarray] = {}
    for name in ("q", "k", "v", "do"):
        if name not in shapes:
            continue
        x = draw_normal_f32(rng, shapes[name], in_scale)
        out[name] = f32_to_bf16_bits(x)
        if keep_f32:
            out[name + "_f32"] = x
        del x
    return out


def make_inputs(workload: str | Workload, seed: Optional[int] = None,
                keep_f32: bool = False) -> Dict[str, np.ndarray]:
    """Inputs of a named workload (its own seed unless ``seed`` is given)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    sd = w.seed if seed is None else seed
    if w.fp8:
        return make_fp8_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, sd)
    if w.pack is not None:
        # packed batch: [H, T, d] tensors (the [1, H, T, d] draw) plus the boundaries
        x = make_custom_inputs(1, w.Hq, w.Hkv, w.N, w.d, sd, in_scale=w.in_scale,
                               with_grad=w.with_grad, keep_f32=keep_f32)
        x = {name: a[0] for name, a in x.items()}
        x["cu_seqlens"] = cu_from_lengths(w.lengths())
        return x
    x = make_custom_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, sd, in_scale=w.in_scale,
                           with_grad=w.with_grad, keep_f32=keep_f32)
    if w.nq is not None:
        # decoding: the N keys are the cache; the queries are a separate draw of nq rows
        xq = make_custom_inputs(w.B, w.Hq, w.Hkv, w.nq, w.d, sd + 1, in_scale=w.in_scale,
                                keep_f32=keep_f32)
        for name in [n for n in xq if n.startswith("q")]:
            x[name] = xq[name]
    return x
