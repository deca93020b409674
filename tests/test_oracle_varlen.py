"""Pins of the oracle's packed variable-length batches (CPU only).

A packed batch is read as independent sequences ([EVOL] §6, scenario 2:
documents concatenated and packed into long training sequences, each its own
attention problem).  The pins hold it to things other than itself: the
scalar brute force run over the whole concatenation with a same-sequence
mask, the dense batched oracle when every length is equal, and the
permutation of whole sequences inside the pack.
"""
import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward, bf_backward, bf_forward,
                    check_cu_seqlens, varlen_backward, varlen_forward, varlen_forward_rows)


def rnd(seed, *shape):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape))


def packed(seed, lengths, Hq, Hkv, d):
    T = sum(lengths)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    q, k, v, do = rnd(seed, Hq, T, d), rnd(seed + 1, Hkv, T, d), rnd(seed + 2, Hkv, T, d), rnd(seed + 3, Hq, T, d)
    seg = [b for b, n in enumerate(lengths) for _ in range(n)]
    return q, k, v, do, cu, seg


T64 = torch.float64


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [None, 0, 2])
def test_varlen_matches_segment_masked_bruteforce(causal, window):
    """The concatenation with a block-diagonal (same-sequence) mask, computed by
    scalar loops, equals the per-sequence oracle -- forward and backward."""
    q, k, v, do, cu, seg = packed(80, [3, 0, 5, 1, 7], 4, 2, 8)
    o, lse = varlen_forward(q, k, v, cu, causal, 0.41, window=window)
    bo, bl = bf_forward(q[None], k[None], v[None], causal, 0.41, window=window, segments=seg)
    assert torch.allclose(o, torch.tensor(bo, dtype=T64)[0], atol=1e-12)
    assert torch.allclose(lse, torch.tensor(bl, dtype=T64)[0], atol=1e-12)
    g = varlen_backward(q, k, v, do, cu, causal, 0.41, window=window)
    bg = bf_backward(q[None], k[None], v[None], do[None], causal, 0.41, window=window, segments=seg)
    for x, y in zip(g, bg):
        assert torch.allclose(x, torch.tensor(y, dtype=T64)[0], atol=1e-11)


def test_equal_lengths_are_the_dense_batch():
    """With B sequences of one length N the pack is the dense [B, H, N, d]
    batch laid out as [H, B*N, d]."""
    B, Hq, Hkv, N, d = 3, 4, 2, 6, 8
    q, k, v, do = rnd(90, B, Hq, N, d), rnd(91, B, Hkv, N, d), rnd(92, B, Hkv, N, d), rnd(93, B, Hq, N, d)
    pack = lambda x: x.permute(1, 0, 2, 3).reshape(x.shape[1], B * N, d)
    cu = [i * N for i in range(B + 1)]
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, causal)
        po, pl = varlen_forward(pack(q), pack(k), pack(v), cu, causal)
        assert torch.allclose(po, pack(o), atol=1e-14)
        assert torch.allclose(pl, lse.permute(1, 0, 2).reshape(Hq, B * N), atol=1e-14)
        g = attention_backward(q, k, v, do, causal)
        pg = varlen_backward(pack(q), pack(k), pack(v), pack(do), cu, causal)
        for x, y in zip(pg, g):
            assert torch.allclose(x, pack(y), atol=1e-13)


def test_reordering_sequences_moves_their_rows():
    """Sequences do not interact: packing them in another order only moves
    each sequence's rows of O, LSE and the gradients."""
    lengths = [4, 2, 6, 3]
    q, k, v, do, cu, _ = packed(100, lengths, 2, 1, 4)
    order = [2, 0, 3, 1]
    idx = torch.cat([torch.arange(cu[b], cu[b + 1]) for b in order])
    cu2 = [0]
    for b in order:
        cu2.append(cu2[-1] + lengths[b])
    for causal in (True, False):
        o, lse = varlen_forward(q, k, v, cu, causal)
        o2, lse2 = varlen_forward(q[:, idx], k[:, idx], v[:, idx], cu2, causal)
        assert torch.allclose(o2, o[:, idx], atol=1e-14) and torch.allclose(lse2, lse[:, idx], atol=1e-14)
        g = varlen_backward(q, k, v, do, cu, causal)
        g2 = varlen_backward(q[:, idx], k[:, idx], v[:, idx], do[:, idx], cu2, causal)
        for x, y in zip(g2, g):
            assert torch.allclose(x, y[:, idx], atol=1e-13)


def test_first_row_of_every_causal_sequence_sees_only_itself():
    """Under the causal mask the first token of each sequence sees one key:
    O = its own v, LSE = tau q.k -- whatever precedes it in the pack."""
    q, k, v, _, cu, _ = packed(110, [5, 1, 4], 4, 2, 8)
    o, lse = varlen_forward(q, k, v, cu, True, 0.5)
    for s0 in cu[:-1]:
        for h in range(4):
            assert torch.allclose(o[h, s0], v[h // 2, s0], atol=1e-15)
            assert abs(float(lse[h, s0]) - 0.5 * float(q[h, s0] @ k[h // 2, s0])) < 1e-13


def test_sampled_rows_agree_with_the_whole_pack():
    q, k, v, _, cu, _ = packed(120, [7, 3, 9], 4, 2, 8)
    rows = [0, 6, 7, 9, 10, 18]
    for causal in (True, False):
        o, lse = varlen_forward(q, k, v, cu, causal, window=3)
        ro, rl = varlen_forward_rows(q, k, v, cu, causal, None, 3, rows, window=3)
        assert torch.allclose(ro, o[3, rows], atol=1e-14) and torch.allclose(rl, lse[3, rows], atol=1e-14)


@pytest.mark.parametrize("cu,total", [([1, 4], 4), ([0, 5, 3, 6], 6), ([0, 4], 5), ([0], 0)])
def test_bad_boundaries_are_rejected(cu, total):
    with pytest.raises(ValueError):
        check_cu_seqlens(cu, total)
