"""CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run anything in ``oracle/``.  The GPU library never
calls it and shares no code with it; the seeded inputs both sides consume come
from ``synth_inputs``, which holds no attention arithmetic.

What it computes is the plain definition, in float64, with torch CPU ops used
only as dense linear-algebra and elementwise primitives:

    s_ij  = tau * q_i . k_j              for j in A(i)
    LSE_i = ln sum_{j in A(i)} exp(s_ij) (computed as m_i + ln sum exp(s_ij - m_i))
    P_ij  = exp(s_ij - LSE_i)  (0 outside A(i))
    O_i   = sum_j P_ij v_j

with A(i) = {0..N-1} (non-causal) or {0..i} (causal), optionally narrowed to a
sliding window of w keys on each side, |i - j| <= w, and the textbook softmax
Jacobian for the backward:

    dP_ij = dO_i . v_j
    c_i   = sum_k P_ik dP_ik
    dS_ij = P_ij (dP_ij - c_i)
    dQ_i  = tau * sum_j dS_ij k_j
    dK_j  = tau * sum_i dS_ij q_i   (summed over the query heads of the group)
    dV_j  = sum_i P_ij dO_i         (summed over the query heads of the group)

Sources, by page title and section:
  * [EVOL] "从“算力黑洞”到“效率革命”：大模型Attention的演进之路" (mhpn.cn):
      §2 (标准Attention) gives Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V;
      §3 (MLA, i.e. multi-query) and its GQA paragraph give K/V head sharing
      among groups of query heads; §6 (实战) gives ``is_causal=True`` as the
      triangular mask that stops a position from seeing later positions.
  * [LONGCTX] "6.1 2023 年代：長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力"
      (cccbook): §2.2 (分塊與重計算) -- the forward keeps the output and the
      per-row log-sum-exp statistic; §2.3 -- the result is exact, identical to
      standard softmax attention; §4 (稀疏注意力與線性注意力) -- sliding-window
      attention, where each query sees only a fixed number of tokens before and
      after it.
  * [LA2] "Lightning Attention-2 新一代注意力机制": the mask of a
      unidirectional (GPT-style) model is lower triangular.

Readings where the pages leave a step open:
  * the mask is additive minus infinity (masked probabilities are exactly 0);
    the literal elementwise-product form on the [LA2] page would leave weight
    on future keys, contradicting the "no future information" use in [EVOL] §6;
  * causal alignment is j <= i with one sequence length for queries and keys,
    so no row is ever fully masked;
  * a window w counts keys on each side of the query, excluding the query
    itself: A(i) narrows to i - w <= j <= i + w, intersected with j <= i under
    the causal mask; w = 0 leaves the query's own key only, w >= N - 1 changes
    nothing, and no row is ever empty;
  * with fewer queries than keys (N_q < N_k: decoding against a KV cache, the
    setting of [EVOL] §1 and §3 and [LONGCTX] §1.5) the queries are the last
    N_q positions of the sequence: query i sits at position i + N_k - N_q, and
    the causal mask and the window are taken between positions (bottom-right
    alignment), so query N_q - 1 sees every key;
  * LSE is the natural log over the *scaled* scores, masked keys excluded;
  * head h of the query reads K/V head floor(h / G), G = H_q / H_kv
    (contiguous groups);
  * the backward is the analytic derivative of the forward (the pages print no
    gradient formulas) and uses the textbook c_i, not the rowsum(dO * O)
    shortcut a fast kernel may take;
  * packed variable-length batches ([EVOL] §6, scenario 2: long-context
    training data is built by concatenating and packing documents into long
    sequences): each packed sequence is its own attention problem -- its
    queries see only its own keys, positions counted from its first token --
    so a packed batch is the definition above applied to every sequence on
    its own.  Layout [H, T, d]: sequence b is rows cu_seqlens[b] ..
    cu_seqlens[b+1] - 1 of every head (cu_seqlens[0] = 0, non-decreasing,
    cu_seqlens[B] = T; empty sequences allowed); LSE is [H_q, T].

Query rows are processed in blocks only to bound memory (a full 32K x 32K
fp64 score matrix is 8 GiB); every row is materialised over all N keys with
masked entries set to -inf, exactly as the naive three-pass method of [EVOL] §4
would, just on the CPU.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "default_scale",
    "attention_forward",
    "attention_backward",
    "attention_probs",
    "forward_rows",
    "probs_rows",
    "backward_dq_rows",
    "varlen_forward",
    "varlen_backward",
    "varlen_forward_rows",
    "check_cu_seqlens",
    "to_f64",
]

_ROW_BLOCK = 512


def default_scale(d: int) -> float:
    """tau = 1 / sqrt(d_k)  ([EVOL] §2)."""
    return 1.0 / math.sqrt(d)


def to_f64(x) -> torch.Tensor:
    """Any array-like -> contiguous float64 CPU tensor."""
    t = torch.as_tensor(x)
    return t.to(device="cpu", dtype=torch.float64).contiguous()


def _shapes(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positional: bool):
    """(B, H_q, H_kv, N_q, d, G).  With a positional mask (causal or window) the
    queries are the last N_q of N_k >= N_q positions; without one any N_k."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if positional and Nk < N:
        raise ValueError("a causal or windowed mask needs at least as many keys as queries")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return B, Hq, Hkv, N, d, Hq // Hkv


def _check_window(window: Optional[int]) -> None:
    if window is not None and int(window) < 0:
        raise ValueError("window must be >= 0 (or None for no window)")


def _row_probs(q_rows: torch.Tensor, k_head: torch.Tensor, rows: torch.Tensor,
               causal: bool, scale: float,
               window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Scores -> (P, LSE) for a set of query rows of one head, over all keys.

    q_rows [R, d], k_head [N, d], rows [R] = the sequence positions of q_rows.
    Returns P [R, N] (exact zeros where masked) and LSE [R].
    """
    N = k_head.shape[0]
    s = scale * (q_rows @ k_head.transpose(0, 1))              # s_ij, [R, N]
    keys = torch.arange(N, dtype=torch.int64)
    if causal:
        s = s.masked_fill(keys[None, :] > rows[:, None], -math.inf)
    if window is not None:
        dist = keys[None, :] - rows[:, None]                   # j - i
        s = s.masked_fill((dist < -int(window)) | (dist > int(window)), -math.inf)
    m = s.max(dim=1).values                                    # finite: key i is always in A(i)
    ell = torch.exp(s - m[:, None]).sum(dim=1)
    lse = m + torch.log(ell)
    p = torch.exp(s - lse[:, None])                            # exp(-inf) = 0 on masked keys
    return p, lse


def attention_forward(q, k, v, causal: bool, scale: Optional[float] = None,
                      row_block: int = _ROW_BLOCK,
                      window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O [B,H_q,N,d] and LSE [B,H_q,N], both float64."""
    _check_window(window)
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Hkv, N, d, G = _shapes(q, k, v, causal or window is not None)
    tau = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                rows = torch.arange(r0, r1, dtype=torch.int64) + (k.shape[2] - N)   # positions
                p, l_blk = _row_probs(q[b, h, r0:r1], k[b, g], rows, causal, tau, window)
                o[b, h, r0:r1] = p @ v[b, g]
                lse[b, h, r0:r1] = l_blk
    return o, lse


def attention_probs(q, k, causal: bool, scale: Optional[float] = None,
                    window: Optional[int] = None) -> torch.Tensor:
    """The full probability matrix P [B,H_q,N_q,N_k] (small inputs only)."""
    _check_window(window)
    q, k = to_f64(q), to_f64(k)
    B, Hq, Hkv, N, d, G = _shapes(q, k, k, causal or window is not None)
    tau = default_scale(d) if scale is None else float(scale)
    out = torch.empty((B, Hq, N, k.shape[2]), dtype=torch.float64)
    rows = torch.arange(N, dtype=torch.int64) + (k.shape[2] - N)               # positions
    for b in range(B):
        for h in range(Hq):
            out[b, h], _ = _row_probs(q[b, h], k[b, h // G], rows, causal, tau, window)
    return out


def forward_rows(q, k, v, causal: bool, scale: Optional[float], b: int, h: int,
                 rows: Sequence[int],
                 window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O and LSE of selected query rows of one (batch, query head).

    Used to check very large problems on sampled rows: each row is computed
    from the definition over all N keys, independently of the other rows.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    g = h // (Hq // Hkv)
    d = q.shape[-1]
    tau = default_scale(d) if scale is None else float(scale)
    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)
    _check_window(window)
    q_r = to_f64(q[b, h])[rows_t]
    k_g, v_g = to_f64(k[b, g]), to_f64(v[b, g])
    p, lse = _row_probs(q_r, k_g, rows_t + (k.shape[2] - q.shape[2]), causal, tau, window)
    return p @ v_g, lse


def probs_rows(q, k, causal: bool, scale: Optional[float], b: int, h: int,
               rows: Sequence[int]) -> torch.Tensor:
    """Rows of the probability matrix P [len(rows), N_k] of one (batch, query head)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = h // (Hq // Hkv)
    d = q.shape[-1]
    tau = default_scale(d) if scale is None else float(scale)
    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)
    p, _ = _row_probs(to_f64(q[b, h])[rows_t], to_f64(k[b, g]), rows_t + (k.shape[2] - q.shape[2]),
                      causal, tau, None)
    return p


def attention_backward(q, k, v, do, causal: bool, scale: Optional[float] = None,
                       row_block: int = _ROW_BLOCK, window: Optional[int] = None):
    """dQ [B,H_q,N,d], dK and dV [B,H_kv,N,d] of L = sum(dO * O), float64."""
    _check_window(window)
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, Hq, Hkv, N, d, G = _shapes(q, k, v, causal or window is not None)
    if tuple(do.shape) != tuple(q.shape):
        raise ValueError("dO must have the shape of Q")
    tau = default_scale(d) if scale is None else float(scale)
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                rows = torch.arange(r0, r1, dtype=torch.int64) + (k.shape[2] - N)   # positions
                q_blk, do_blk = q[b, h, r0:r1], do[b, h, r0:r1]
                p, _ = _row_probs(q_blk, k[b, g], rows, causal, tau, window)
                dp = do_blk @ v[b, g].transpose(0, 1)          # dP_ij = dO_i . v_j
                c = (p * dp).sum(dim=1)                        # c_i = sum_k P_ik dP_ik
                ds = p * (dp - c[:, None])                     # dS_ij
                dq[b, h, r0:r1] = tau * (ds @ k[b, g])
                dk[b, g] += tau * (ds.transpose(0, 1) @ q_blk)
                dv[b, g] += p.transpose(0, 1) @ do_blk
    return dq, dk, dv


def backward_dq_rows(q, k, v, do, causal: bool, scale: Optional[float], b: int,
                     h: int, rows: Sequence[int], window: Optional[int] = None) -> torch.Tensor:
    """dQ of selected query rows of one (batch, query head).

    dQ_i needs only row i of P and dP, so sampled rows of a large problem can
    be checked one by one.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    g = h // (Hq // Hkv)
    d = q.shape[-1]
    tau = default_scale(d) if scale is None else float(scale)
    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)
    _check_window(window)
    q_r = to_f64(q[b, h])[rows_t]
    do_r = to_f64(do[b, h])[rows_t]
    k_g, v_g = to_f64(k[b, g]), to_f64(v[b, g])
    p, _ = _row_probs(q_r, k_g, rows_t + (k.shape[2] - q.shape[2]), causal, tau, window)
    dp = do_r @ v_g.transpose(0, 1)
    c = (p * dp).sum(dim=1)
    ds = p * (dp - c[:, None])
    return tau * (ds @ k_g)


# ---------------------------------------------------------------------------
# Packed variable-length batches: every sequence on its own
# ---------------------------------------------------------------------------
def check_cu_seqlens(cu_seqlens, total: int) -> list:
    """Sequence boundaries as a list of ints; raises unless they start at 0,
    never decrease and end at the packed length ``total``."""
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError(f"cu_seqlens must rise from 0 to {total}: {cu}")
    return cu


def _packed_shapes(q, k, v):
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("packed tensors are [H, T, d]")
    if k.shape[1] != q.shape[1] or k.shape[2] != q.shape[2] or q.shape[0] % k.shape[0]:
        raise ValueError("packed K/V must be [H_kv, T, d] with H_q % H_kv == 0")


def varlen_forward(q, k, v, cu_seqlens, causal: bool, scale: Optional[float] = None,
                   window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O [H_q, T, d] and LSE [H_q, T] of a packed batch, float64."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    _packed_shapes(q, k, v)
    cu = check_cu_seqlens(cu_seqlens, q.shape[1])
    if scale is None:
        scale = default_scale(q.shape[2])
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:2], dtype=torch.float64)
    for s0, s1 in zip(cu, cu[1:]):
        if s1 == s0:
            continue
        ob, lb = attention_forward(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1],
                                   causal, scale, window=window)
        o[:, s0:s1] = ob[0]
        lse[:, s0:s1] = lb[0]
    return o, lse


def varlen_backward(q, k, v, do, cu_seqlens, causal: bool, scale: Optional[float] = None,
                    window: Optional[int] = None):
    """dQ [H_q, T, d], dK and dV [H_kv, T, d] of L = sum(dO * O) over a packed batch."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    _packed_shapes(q, k, v)
    cu = check_cu_seqlens(cu_seqlens, q.shape[1])
    if scale is None:
        scale = default_scale(q.shape[2])
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    for s0, s1 in zip(cu, cu[1:]):
        if s1 == s0:
            continue
        g = attention_backward(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1],
                               do[None, :, s0:s1], causal, scale, window=window)
        dq[:, s0:s1], dk[:, s0:s1], dv[:, s0:s1] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def varlen_forward_rows(q, k, v, cu_seqlens, causal: bool, scale: Optional[float], h: int,
                        rows: Sequence[int], window: Optional[int] = None):
    """O and LSE of selected packed rows (global row indices) of query head h,
    each computed within its own sequence."""
    cu = check_cu_seqlens(cu_seqlens, q.shape[1])
    outs, lses = [], []
    for r in rows:
        b = max(i for i in range(len(cu) - 1) if cu[i] <= r < cu[i + 1])
        s0, s1 = cu[b], cu[b + 1]
        ob, lb = forward_rows(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], causal,
                              scale, 0, h, [r - s0], window=window)
        outs.append(ob[0])
        lses.append(lb[0])
    return torch.stack(outs), torch.stack(lses)
