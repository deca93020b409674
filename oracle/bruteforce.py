"""Scalar brute-force attention -- TEST INFRASTRUCTURE ONLY.

Pure-Python loops over nested lists, ``math.exp`` and ``math.fsum`` (exactly
rounded sums).  It exists to pin ``oracle.attention`` on tiny inputs: it shares
no code with it, indexes every operand element by element (so a transposed
operand or a wrong head index in the vectorised oracle shows up), and sums with
``fsum`` so its own rounding error is far below the comparison tolerance.

It follows the same definitions, from the pages named in
``oracle/attention.py``: scaled dot-product softmax attention
([EVOL] §2, "从“算力黑洞”到“效率革命”：大模型Attention的演进之路"), causal keys
j <= i ([EVOL] §6), K/V head floor(h/G) for grouped queries ([EVOL] §3), the
natural-log log-sum-exp statistic ([LONGCTX] §2.2, cccbook ch. 6.1), the
sliding window of w keys on each side of a query ([LONGCTX] §4), queries that
are the last N_q of N_k positions when decoding against a KV cache ([EVOL] §1,
§3; [LONGCTX] §1.5), packed batches whose sequences never see each other
(``segments``: the sequence id of every position, [EVOL] §6 scenario 2), and
the analytic softmax gradients (N_q = N_k only).  Only use it for N * N * d up
to ~10^5.
"""
from __future__ import annotations

import math
from typing import List

__all__ = ["bf_forward", "bf_backward", "tolist4"]


def tolist4(x) -> List:
    """Array-like [B,H,N,d] -> nested Python lists of floats."""
    if hasattr(x, "tolist"):
        return x.tolist()
    return [[[[float(e) for e in row] for row in head] for head in bat] for bat in x]


def _visible(i: int, n: int, causal: bool, window=None, nq=None, segments=None) -> List[int]:
    """Keys (of n) that query i (of nq, default n) attends to, in increasing
    order.  With nq < n the queries are the last nq positions of the sequence;
    with segments, only keys of the query's own segment are seen."""
    pos = i + n - (n if nq is None else nq)
    out = []
    for j in range(n):
        if causal and j > pos:
            continue
        if window is not None and abs(pos - j) > window:
            continue
        if segments is not None and segments[j] != segments[pos]:
            continue
        out.append(j)
    return out


def _dot(a: List[float], b: List[float]) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def bf_forward(q, k, v, causal: bool, scale: float, window=None, segments=None):
    """Returns (O, LSE) as nested lists: O[b][h][i][t], LSE[b][h][i]."""
    q, k, v = tolist4(q), tolist4(k), tolist4(v)
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    O = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    L = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(N):
                keys = _visible(i, Nk, causal, window, N, segments)
                s = [scale * _dot(q[b][h][i], k[b][g][j]) for j in keys]
                m = max(s)
                lse = m + math.log(math.fsum(math.exp(x - m) for x in s))
                p = [math.exp(x - lse) for x in s]
                L[b][h][i] = lse
                for t in range(d):
                    O[b][h][i][t] = math.fsum(pj * v[b][g][j][t] for pj, j in zip(p, keys))
    return O, L


def bf_backward(q, k, v, do, causal: bool, scale: float, window=None, segments=None):
    """Returns (dQ, dK, dV) as nested lists for L = sum_{b,h,i,t} dO * O."""
    q, k, v, do = tolist4(q), tolist4(k), tolist4(v), tolist4(do)
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    dQ = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    # dK, dV collect every term and are summed exactly at the end.
    dK_terms = [[[[[] for _ in range(d)] for _ in range(N)] for _ in range(Hkv)] for _ in range(B)]
    dV_terms = [[[[[] for _ in range(d)] for _ in range(N)] for _ in range(Hkv)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(N):
                keys = _visible(i, N, causal, window, None, segments)
                s = [scale * _dot(q[b][h][i], k[b][g][j]) for j in keys]
                m = max(s)
                lse = m + math.log(math.fsum(math.exp(x - m) for x in s))
                p = [math.exp(x - lse) for x in s]
                dp = [_dot(do[b][h][i], v[b][g][j]) for j in keys]
                c = math.fsum(pj * dpj for pj, dpj in zip(p, dp))
                ds = [pj * (dpj - c) for pj, dpj in zip(p, dp)]
                for t in range(d):
                    dQ[b][h][i][t] = scale * math.fsum(dsj * k[b][g][j][t] for dsj, j in zip(ds, keys))
                for dsj, pj, j in zip(ds, p, keys):
                    for t in range(d):
                        dK_terms[b][g][j][t].append(scale * dsj * q[b][h][i][t])
                        dV_terms[b][g][j][t].append(pj * do[b][h][i][t])
    dK = [[[[math.fsum(c) for c in row] for row in head] for head in bat] for bat in dK_terms]
    dV = [[[[math.fsum(c) for c in row] for row in head] for head in bat] for bat in dV_terms]
    return dQ, dK, dV
