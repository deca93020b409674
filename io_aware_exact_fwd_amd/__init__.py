"""Python binding of the gfx950 attention library (``libattn.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI in ``include/attn.h``.  PyTorch provides device
memory and the current stream; nothing here computes attention, and there is
no CPU or PyTorch fallback -- a missing library or an unsupported device
raises.

    o, lse = fwd(q, k, v, causal=True)           # q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o, lse = fwd_varlen(q, k, v, cu_seqlens)     # packed q [Hq,T,d], k/v [Hkv,T,d]
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch  # loads the HIP runtime that libattn.so then binds to

__all__ = [
    "AttnError", "fwd", "bwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "bwd_grads", "fwd_decode",
    "decode_workspace_bytes", "fwd_decode_static", "DECODE_STATIC_SCRATCH_BYTES", "fwd_varlen", "bwd_varlen", "bwd_varlen_workspace_bytes",
    "bwd_varlen_split_workspace_bytes",
    "bwd_grads_varlen", "fwd_fp8", "attention", "attention_varlen",
    "bwd_workspace_bytes",
    "device_check", "strerror", "lib", "LIB_PATH", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
            "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_grads", "attn_strerror",
            "attn_device_check", "attn_fwd_window", "attn_bwd_window", "attn_bwd_grads_window",
            "attn_fwd_decode", "attn_fwd_decode_workspace_bytes", "attn_fwd_varlen",
            "attn_bwd_varlen", "attn_bwd_varlen_workspace_bytes", "attn_bwd_grads_varlen",
            "attn_bwd_varlen_split_workspace_bytes",
            "attn_fwd_fp8", "attn_fwd_decode_static")

ATTN_OK = 0
# bytes of the static decode scratch behind attn_fwd_decode_static (include/attn.h)
DECODE_STATIC_SCRATCH_BYTES = 32 << 20


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: attn error {code}: {strerror(code)}")


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load ``libattn.so`` (built by ``io_aware_exact_fwd_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m io_aware_exact_fwd_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd.restype = i
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, vp]
    L.attn_bwd_preprocess.restype = i
    L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_bwd_dkdv.restype = i
    L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_bwd_dq.restype = i
    L.attn_bwd_grads.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_bwd_grads.restype = i
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_window.restype = i
    L.attn_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
    L.attn_bwd_window.restype = i
    L.attn_bwd_grads_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.attn_bwd_grads_window.restype = i
    L.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_fwd_decode.restype = i
    L.attn_fwd_decode_static.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd_decode_static.restype = i
    L.attn_fwd_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_fwd_decode_workspace_bytes.restype = sz
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_varlen.restype = i
    L.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i,
                                  i, i, f, vp]
    L.attn_bwd_varlen.restype = i
    L.attn_bwd_grads_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                        i, i, f, vp]
    L.attn_bwd_grads_varlen.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_bwd_varlen_workspace_bytes.argtypes = [i, i, i]
    L.attn_bwd_varlen_workspace_bytes.restype = sz
    L.attn_bwd_varlen_split_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_varlen_split_workspace_bytes.restype = sz
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_strerror.argtypes = [i]
    L.attn_strerror.restype = ctypes.c_char_p
    L.attn_device_check.argtypes = [i]
    L.attn_device_check.restype = i
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().attn_strerror(int(code)).decode()


def device_check(device: int = 0) -> int:
    return int(lib().attn_device_check(int(device)))


def bwd_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_bf16(name: str, t: torch.Tensor, shape) -> None:
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(q: torch.Tensor, k: torch.Tensor) -> Tuple[int, int, int, int, int]:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, stream=None,
        window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O = softmax(scale*QK^T + mask)V (bf16) and LSE (fp32 [B,Hq,N]) on the GPU.

    window: None, or the sliding window (keys with |i - j| <= window).
    """
    B, Hq, Hkv, N, d = _dims(q, k)
    _check_bf16("q", q, (B, Hq, N, d))
    _check_bf16("k", k, (B, Hkv, N, d))
    _check_bf16("v", v, (B, Hkv, N, d))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, (B, Hq, N, d))
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, Hq, N))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if window is None:
        rc = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                            B, Hq, Hkv, N, d, int(bool(causal)), tau, _stream(stream))
    else:
        rc = lib().attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   B, Hq, Hkv, N, d, int(bool(causal)), int(window), tau,
                                   _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd" if window is None else "attn_fwd_window")
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
        lse: torch.Tensor, do: torch.Tensor, causal: bool = True,
        scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None,
        stream=None, window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV (bf16) of L = sum(dO * O), recomputing scores from the LSE.

    window: None, or the sliding window the forward used.
    """
    B, Hq, Hkv, N, d = _dims(q, k)
    for name, t, shp in (("q", q, (B, Hq, N, d)), ("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d)),
                         ("o", o, (B, Hq, N, d)), ("do", do, (B, Hq, N, d))):
        _check_bf16(name, t, shp)
    _check_f32("lse", lse, (B, Hq, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dq", dq, (B, Hq, N, d))
    _check_bf16("dk", dk, (B, Hkv, N, d))
    _check_bf16("dv", dv, (B, Hkv, N, d))
    need = bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ws_bytes = workspace.numel() * workspace.element_size()
    if window is None:
        rc = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                            _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                            B, Hq, Hkv, N, d, int(bool(causal)), tau, _stream(stream))
    else:
        rc = lib().attn_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                   B, Hq, Hkv, N, d, int(bool(causal)), int(window), tau,
                                   _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd" if window is None else "attn_bwd_window")
    return dq, dk, dv


def _check_f32(name: str, t: torch.Tensor, shape) -> None:
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {tuple(shape)}")


def _check_workspace(t: torch.Tensor) -> None:
    """A caller-supplied workspace must be device memory in one piece (its size
    is checked by the library against what the call needs)."""
    if not torch.is_tensor(t) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")


def bwd_preprocess(o: torch.Tensor, do: torch.Tensor, delta: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """delta [B,Hq,N] fp32 = rowsum(dO * O): the first stage of bwd."""
    B, Hq, N, d = o.shape
    _check_bf16("o", o, (B, Hq, N, d))
    _check_bf16("do", do, (B, Hq, N, d))
    if delta is None:
        delta = torch.empty((B, Hq, N), dtype=torch.float32, device=o.device)
    _check_f32("delta", delta, (B, Hq, N))
    rc = lib().attn_bwd_preprocess(_ptr(o), _ptr(do), _ptr(delta), B, Hq, N, d, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_preprocess")
    return delta


def _stage_checks(q, k, v, do, lse, delta):
    B, Hq, Hkv, N, d = _dims(q, k)
    for name, t, shp in (("q", q, (B, Hq, N, d)), ("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d)),
                         ("do", do, (B, Hq, N, d))):
        _check_bf16(name, t, shp)
    _check_f32("lse", lse, (B, Hq, N))
    _check_f32("delta", delta, (B, Hq, N))
    return B, Hq, Hkv, N, d


def bwd_dkdv(q, k, v, do, lse, delta, causal: bool = True, scale: Optional[float] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """dK, dV (bf16) from the inputs, lse and delta: the second stage of bwd."""
    B, Hq, Hkv, N, d = _stage_checks(q, k, v, do, lse, delta)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dk", dk, (B, Hkv, N, d))
    _check_bf16("dv", dv, (B, Hkv, N, d))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dk),
                             _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_dkdv")
    return dk, dv


def bwd_dq(q, k, v, do, lse, delta, causal: bool = True, scale: Optional[float] = None,
           dq: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dQ (bf16) from the inputs, lse and delta: the third stage of bwd."""
    B, Hq, Hkv, N, d = _stage_checks(q, k, v, do, lse, delta)
    dq = torch.empty_like(q) if dq is None else dq
    _check_bf16("dq", dq, (B, Hq, N, d))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dq),
                           B, Hq, Hkv, N, d, int(bool(causal)), tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_dq")
    return dq


def bwd_grads(q, k, v, do, lse, delta, causal: bool = True, scale: Optional[float] = None,
              dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
              dv: Optional[torch.Tensor] = None, stream=None,
              window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV (bf16) in one launch: what bwd_dkdv and bwd_dq give, bitwise."""
    B, Hq, Hkv, N, d = _stage_checks(q, k, v, do, lse, delta)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dq", dq, (B, Hq, N, d))
    _check_bf16("dk", dk, (B, Hkv, N, d))
    _check_bf16("dv", dv, (B, Hkv, N, d))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if window is None:
        rc = lib().attn_bwd_grads(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d,
                                  int(bool(causal)), tau, _stream(stream))
    else:
        rc = lib().attn_bwd_grads_window(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                                         _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv,
                                         N, d, int(bool(causal)), int(window), tau,
                                         _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_grads" if window is None else "attn_bwd_grads_window")
    return dq, dk, dv


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                           num_splits: int = 0) -> int:
    return int(lib().attn_fwd_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, int(num_splits)))


def fwd_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
               scale: Optional[float] = None, window: Optional[int] = None, num_splits: int = 0,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode forward: q [B,Hq,Nq,d] against the cache k, v [B,Hkv,Nk,d] (Nq <= Nk,
    queries at the last Nq positions).  Returns O (bf16) and LSE (fp32 [B,Hq,Nq])."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check_bf16("q", q, (B, Hq, Nq, d))
    _check_bf16("k", k, (B, Hkv, Nk, d))
    _check_bf16("v", v, (B, Hkv, Nk, d))
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, (B, Hq, Nq, d))
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, Hq, Nq))
    need = decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk,
                               d, int(bool(causal)), -1 if window is None else int(window), tau,
                               int(num_splits), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_decode")
    return out, lse



def fwd_decode_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                      scale: Optional[float] = None, window: Optional[int] = None,
                      num_splits: int = 0, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fwd_decode without a workspace (attn_fwd_decode_static): the per-chunk
    partials live in the library's static per-GPU scratch, so with ``out`` and
    ``lse`` given nothing is allocated.  Calls that may overlap on one GPU race
    on that scratch (see include/attn.h)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check_bf16("q", q, (B, Hq, Nq, d))
    _check_bf16("k", k, (B, Hkv, Nk, d))
    _check_bf16("v", v, (B, Hkv, Nk, d))
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, (B, Hq, Nq, d))
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, Hq, Nq))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_fwd_decode_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv,
                                      Nq, Nk, d, int(bool(causal)),
                                      -1 if window is None else int(window), tau, int(num_splits),
                                      _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_decode_static")
    return out, lse


# ---------------------------------------------------------------------------
# Packed variable-length batches
# ---------------------------------------------------------------------------
def _packing(cu_seqlens, max_seqlen: Optional[int], total: int, device) -> Tuple[torch.Tensor, int, int]:
    """(int32 device boundaries, B, max_seqlen).  A host table, or a missing
    max_seqlen, is checked here (it must rise from 0 to total); a device table
    with max_seqlen given is passed on unread (the library clamps every
    access, see include/attn.h)."""
    if not torch.is_tensor(cu_seqlens):
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int32)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 boundaries")
    if not cu_seqlens.is_cuda or max_seqlen is None:
        cu = cu_seqlens.cpu().tolist()
        if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
            raise ValueError(f"cu_seqlens must rise from 0 to {total}")
        longest = max(b - a for a, b in zip(cu, cu[1:]))
        if max_seqlen is None:
            max_seqlen = longest
        elif max_seqlen < longest:
            raise ValueError(f"max_seqlen {max_seqlen} < longest sequence {longest}")
    return cu_seqlens.to(device).contiguous(), cu_seqlens.numel() - 1, int(max_seqlen)


def bwd_varlen_workspace_bytes(Hq: int, total: int, d: int) -> int:
    return int(lib().attn_bwd_varlen_workspace_bytes(Hq, total, d))


def bwd_varlen_split_workspace_bytes(B: int, total: int, max_seqlen: int, Hq: int, Hkv: int,
                                     d: int) -> int:
    """Workspace bytes with which bwd_varlen may split query heads over workgroups."""
    return int(lib().attn_bwd_varlen_split_workspace_bytes(B, total, max_seqlen, Hq, Hkv, d))


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
               max_seqlen: Optional[int] = None, causal: bool = True,
               scale: Optional[float] = None, window: Optional[int] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Packed batch: q [Hq, T, d], k/v [Hkv, T, d] bf16, sequence b = rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1.  Returns O [Hq, T, d] and LSE [Hq, T]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q and k must be [H, T, d]")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    _check_bf16("q", q, (Hq, T, d))
    _check_bf16("k", k, (Hkv, T, d))
    _check_bf16("v", v, (Hkv, T, d))
    cu, B, max_seqlen = _packing(cu_seqlens, max_seqlen, T, q.device)
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, (Hq, T, d))
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (Hq, T))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu), B, T,
                               max_seqlen, Hq, Hkv, d, int(bool(causal)),
                               -1 if window is None else int(window), tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_varlen")
    return out, lse


def bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
               lse: torch.Tensor, do: torch.Tensor, cu_seqlens, max_seqlen: Optional[int] = None,
               causal: bool = True, scale: Optional[float] = None, window: Optional[int] = None,
               dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
               dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ [Hq, T, d], dK and dV [Hkv, T, d] of a packed batch (see fwd_varlen)."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q and k must be [H, T, d]")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    for name, t, shp in (("q", q, (Hq, T, d)), ("k", k, (Hkv, T, d)), ("v", v, (Hkv, T, d)),
                         ("o", o, (Hq, T, d)), ("do", do, (Hq, T, d))):
        _check_bf16(name, t, shp)
    _check_f32("lse", lse, (Hq, T))
    cu, B, max_seqlen = _packing(cu_seqlens, max_seqlen, T, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dq", dq, (Hq, T, d))
    _check_bf16("dk", dk, (Hkv, T, d))
    _check_bf16("dv", dv, (Hkv, T, d))
    if workspace is None:
        need = bwd_varlen_split_workspace_bytes(B, T, max_seqlen, Hq, Hkv, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(cu), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), B, T, max_seqlen,
                               Hq, Hkv, d, int(bool(causal)), -1 if window is None else int(window),
                               tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_varlen")
    return dq, dk, dv


def bwd_grads_varlen(q, k, v, do, lse, delta, cu_seqlens, max_seqlen: Optional[int] = None,
                     causal: bool = True, scale: Optional[float] = None,
                     window: Optional[int] = None, dq=None, dk=None, dv=None,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The gradient stage of bwd_varlen given delta = rowsum(dO * O) [Hq, T]
    (bwd_preprocess over the packed rows)."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q and k must be [H, T, d]")
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    for name, t, shp in (("q", q, (Hq, T, d)), ("k", k, (Hkv, T, d)), ("v", v, (Hkv, T, d)),
                         ("do", do, (Hq, T, d))):
        _check_bf16(name, t, shp)
    _check_f32("lse", lse, (Hq, T))
    _check_f32("delta", delta, (Hq, T))
    cu, B, max_seqlen = _packing(cu_seqlens, max_seqlen, T, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dq", dq, (Hq, T, d))
    _check_bf16("dk", dk, (Hkv, T, d))
    _check_bf16("dv", dv, (Hkv, T, d))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_bwd_grads_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu), B, T, max_seqlen, Hq,
                                     Hkv, d, int(bool(causal)),
                                     -1 if window is None else int(window), tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_grads_varlen")
    return dq, dk, dv


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_descale: torch.Tensor,
            k_descale: torch.Tensor, v_descale: torch.Tensor, causal: bool = True,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """8-bit forward: q8 [B,Hq,N,128], k8/v8 [B,Hkv,N,128] E4M3 codes (uint8 or
    float8_e4m3fn), descales fp32 [B,Hq] / [B,Hkv].  Returns O (bf16) and LSE (fp32)."""
    if q8.dim() != 4 or k8.dim() != 4:
        raise ValueError("q8 and k8 must be [B, H, N, d]")
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    for name, t, shp in (("q8", q8, (B, Hq, N, d)), ("k8", k8, (B, Hkv, N, d)), ("v8", v8, (B, Hkv, N, d))):
        if t.element_size() != 1 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{name} must be a contiguous 1-byte CUDA tensor of shape {shp}")
    _check_f32("q_descale", q_descale, (B, Hq))
    _check_f32("k_descale", k_descale, (B, Hkv))
    _check_f32("v_descale", v_descale, (B, Hkv))
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device)
    _check_bf16("out", out, (B, Hq, N, d))
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    _check_f32("lse", lse, (B, Hq, N))
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_descale), _ptr(k_descale),
                            _ptr(v_descale), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d,
                            int(bool(causal)), tau, _stream(stream))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_fp8")
    return out, lse


# ---------------------------------------------------------------------------
# Autograd entry points: the forward keeps O and the LSE for the backward,
# which recomputes the scores from them (nothing N x N is saved).  Both calls
# only route tensors to the functions above.
# ---------------------------------------------------------------------------
class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, window):
        o, lse = fwd(q, k, v, causal=causal, scale=scale, window=window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, scale, window)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        causal, scale, window = ctx.args
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), causal=causal, scale=scale, window=window)
        return dq, dk, dv, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
              scale: Optional[float] = None, window: Optional[int] = None,
              return_lse: bool = False):
    """Differentiable attention on [B, H, N, d] bf16 CUDA tensors (H_q a multiple
    of H_kv).  Returns O, or (O, LSE) with ``return_lse``; gradients reach q, k
    and v through attn_bwd (or attn_bwd_window)."""
    o, lse = _Attention.apply(q, k, v, bool(causal), scale, window)
    return (o, lse) if return_lse else o


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, causal, scale, window):
        o, lse = fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=causal, scale=scale, window=window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (cu_seqlens, max_seqlen, causal, scale, window)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        cu_seqlens, max_seqlen, causal, scale, window = ctx.args
        dq, dk, dv = bwd_varlen(q, k, v, o, lse, do.contiguous(), cu_seqlens, max_seqlen,
                                causal=causal, scale=scale, window=window)
        return dq, dk, dv, None, None, None, None, None


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
                     max_seqlen: Optional[int] = None, causal: bool = True,
                     scale: Optional[float] = None, window: Optional[int] = None,
                     return_lse: bool = False):
    """Differentiable attention over a packed batch: q [Hq, T, d], k/v [Hkv, T, d]
    bf16, sequences at cu_seqlens (as for fwd_varlen).  Returns O, or (O, LSE)."""
    o, lse = _AttentionVarlen.apply(q, k, v, cu_seqlens, max_seqlen, bool(causal), scale, window)
    return (o, lse) if return_lse else o
