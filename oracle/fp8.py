"""8-bit floating-point (OCP E4M3) attention inputs -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run anything in ``oracle/``; the GPU library never
calls this code.

Setting: page "6.1 2023 年代：長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力"
(cccbook), §2.3, names a low-bit path as one of FlashAttention-3's additions,
and the same section stresses that the method stays exact.  The pages give no
format, scaling or error model, so the reading taken here is:

  * Q, K and V arrive as 8-bit codes in the OCP E4M3 format (1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m/8 * 2^-6; the codes S.1111.111 are NaN and there is no
    infinity; the largest finite value is 448), each head with its own
    descale factor: the value of element x of head (b, h) is
    decode(code) * descale[b, h];
  * the exact result is attention (``oracle.attention``) of those values --
    the low-bit path changes the inputs' precision, not what is computed.

A fast kernel rounds more than this (it feeds the probabilities to the 8-bit
matrix unit); the tests hold it to a bound derived from its documented
rounding, against this exact result.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from .attention import attention_forward, to_f64

__all__ = ["e4m3_to_f64", "dequantize", "fp8_attention_forward", "E4M3_MAX"]

E4M3_MAX = 448.0


def e4m3_to_f64(codes) -> torch.Tensor:
    """uint8 E4M3 codes -> float64 values (NaN for S.1111.111), by the format's
    definition: (-1)^s * 2^(e-7) * (1 + m/8) for e >= 1, (-1)^s * 2^-6 * m/8 for e = 0."""
    c = torch.as_tensor(codes).to(torch.int64)
    if c.numel() and (int(c.min()) < 0 or int(c.max()) > 255):
        raise ValueError("E4M3 codes are bytes")
    sign = torch.where((c >> 7) & 1 == 1, -1.0, 1.0).to(torch.float64)
    e = ((c >> 3) & 0xF).to(torch.float64)
    m = (c & 0x7).to(torch.float64)
    normal = sign * torch.pow(2.0, e - 7.0) * (1.0 + m / 8.0)
    subnormal = sign * (2.0 ** -6) * (m / 8.0)
    out = torch.where(e == 0, subnormal, normal)
    return torch.where((c & 0x7F) == 0x7F, torch.full_like(out, float("nan")), out)


def dequantize(codes, descale) -> torch.Tensor:
    """[B, H, N, d] codes with a [B, H] descale per head -> float64 values."""
    x = e4m3_to_f64(codes)
    s = to_f64(descale)
    if x.dim() != 4 or tuple(s.shape) != tuple(x.shape[:2]):
        raise ValueError("codes are [B, H, N, d] with one descale per (batch, head)")
    return x * s[:, :, None, None]


def fp8_attention_forward(q8, k8, v8, q_descale, k_descale, v_descale, causal: bool,
                          scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O [B,H_q,N,d] and LSE [B,H_q,N] (float64) of attention over the dequantized inputs."""
    q, k, v = dequantize(q8, q_descale), dequantize(k8, k_descale), dequantize(v8, v_descale)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if bool(torch.isnan(t).any()):
            raise ValueError(f"{name} holds a NaN code")
    return attention_forward(q, k, v, causal, scale)
