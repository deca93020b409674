"""Pins of the CPU oracle against things other than itself.

Each test fixes the oracle to brute force, a closed form, an invariant of the
mathematics or a library routine, so that a plausible slip in it (a dropped
term, a wrong sign or index, a transposed operand, a wrong head mapping, a
missing scale) fails at least one of them.  ``test_oracle_mutants.py`` plants
such slips in a copy of the oracle and checks that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward, attention_probs,
                    backward_dq_rows, bf_backward, bf_forward, default_scale,
                    forward_rows, probs_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rnd(seed, *shape, scale=1.0):
    g = np.random.default_rng(seed)
    return torch.from_numpy(g.standard_normal(shape) * scale)


def max_rel(a, b):
    a = torch.as_tensor(np.asarray(a, dtype=np.float64))
    b = torch.as_tensor(np.asarray(b, dtype=np.float64))
    return float((a - b).abs().max() / max(1.0, float(b.abs().max())))


# --------------------------------------------------------------------------
# hand-worked closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    q, k, v, do = (torch.tensor(case[n], dtype=torch.float64) for n in ("q", "k", "v", "do"))
    o, lse = attention_forward(q, k, v, case["causal"], case["scale"])
    dq, dk, dv = attention_backward(q, k, v, do, case["causal"], case["scale"])
    for got, name in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        want = torch.tensor(case[name], dtype=torch.float64)
        assert torch.allclose(got, want, rtol=0, atol=1e-13), (name, got, want)


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------
BF_SHAPES = [
    # B, Hq, Hkv, N, d
    (1, 1, 1, 1, 1),
    (1, 1, 1, 2, 4),
    (1, 2, 1, 3, 4),
    (1, 2, 2, 8, 16),
    (2, 4, 2, 17, 4),
    (1, 4, 1, 32, 16),
    (1, 2, 2, 9, 64),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", BF_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_matches_bruteforce(shape, causal):
    B, Hq, Hkv, N, d = shape
    q, k, v = rnd(1, B, Hq, N, d), rnd(2, B, Hkv, N, d), rnd(3, B, Hkv, N, d)
    tau = default_scale(d)
    o, lse = attention_forward(q, k, v, causal, tau, row_block=5)
    bo, bl = bf_forward(q, k, v, causal, tau)
    assert max_rel(o, bo) < 1e-12
    assert max_rel(lse, bl) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", BF_SHAPES[:6], ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_bruteforce(shape, causal):
    B, Hq, Hkv, N, d = shape
    q, k, v = rnd(4, B, Hq, N, d), rnd(5, B, Hkv, N, d), rnd(6, B, Hkv, N, d)
    do = rnd(7, B, Hq, N, d)
    tau = 0.37  # a scale that is not 1/sqrt(d) pins where tau enters
    dq, dk, dv = attention_backward(q, k, v, do, causal, tau, row_block=3)
    bq, bk, bv = bf_backward(q, k, v, do, causal, tau)
    assert max_rel(dq, bq) < 1e-11
    assert max_rel(dk, bk) < 1e-11
    assert max_rel(dv, bv) < 1e-11


def test_tiny_workload_one_head_bruteforce():
    """The 'tiny' workload (N=256, d=64, fp32 draws) against brute force on one head."""
    from synth_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"]
    x = make_inputs(w, keep_f32=True)
    q = torch.from_numpy(x["q_f32"][:, :1, :96].astype(np.float64))
    k = torch.from_numpy(x["k_f32"][:, :1, :96].astype(np.float64))
    v = torch.from_numpy(x["v_f32"][:, :1, :96].astype(np.float64))
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, causal)
        bo, bl = bf_forward(q, k, v, causal, 1 / 8)
        assert max_rel(o, bo) < 1e-12 and max_rel(lse, bl) < 1e-12


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_probability_rows(causal):
    q, k = rnd(8, 1, 3, 40, 8), rnd(9, 1, 3, 40, 8)
    p = attention_probs(q, k, causal)
    assert torch.allclose(p.sum(-1), torch.ones(1, 3, 40, dtype=torch.float64), atol=1e-14)
    assert bool((p >= 0).all())
    if causal:
        upper = torch.triu(torch.ones(40, 40, dtype=torch.bool), diagonal=1)
        assert bool((p[..., upper] == 0).all())
        assert bool((p[..., ~upper] > 0).all())


@pytest.mark.parametrize("causal", [True, False])
def test_constant_v(causal):
    q, k = rnd(10, 1, 2, 33, 8), rnd(11, 1, 2, 33, 8)
    c = torch.linspace(-2.0, 3.0, 8, dtype=torch.float64)
    v = c.expand(1, 2, 33, 8).clone()
    o, _ = attention_forward(q, k, v, causal)
    assert torch.allclose(o, v, atol=1e-13)
    do = rnd(12, 1, 2, 33, 8)
    dq, dk, _ = attention_backward(q, k, v, do, causal)
    assert float(dq.abs().max()) < 1e-12 and float(dk.abs().max()) < 1e-12


def test_single_unmasked_key():
    q, k, v = rnd(13, 1, 2, 10, 8), rnd(14, 1, 2, 10, 8), rnd(15, 1, 2, 10, 8)
    tau = 0.3
    o, lse = attention_forward(q, k, v, True, tau)
    assert torch.equal(o[:, :, 0], v[:, :, 0])          # P_00 = exp(0) = 1 exactly
    assert torch.allclose(lse[:, :, 0], tau * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-14)
    o1, l1 = attention_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], False, tau)
    assert torch.equal(o1, v[:, :, :1])
    assert torch.allclose(l1[..., 0], tau * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_give_uniform_attention(causal):
    N = 21
    q = torch.zeros(1, 2, N, 4, dtype=torch.float64)
    k, v = rnd(16, 1, 2, N, 4), rnd(17, 1, 2, N, 4)
    o, lse = attention_forward(q, k, v, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        assert torch.allclose(o[:, :, i], v[:, :, :n_vis].mean(2), atol=1e-14)
        assert abs(float(lse[0, 0, i]) - math.log(n_vis)) < 1e-14


def test_noncausal_permutation_invariance():
    q, k, v, do = rnd(18, 1, 2, 30, 8), rnd(19, 1, 1, 30, 8), rnd(20, 1, 1, 30, 8), rnd(21, 1, 2, 30, 8)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(30))
    o, lse = attention_forward(q, k, v, False)
    o2, lse2 = attention_forward(q, k[:, :, perm], v[:, :, perm], False)
    assert torch.allclose(o, o2, atol=1e-13) and torch.allclose(lse, lse2, atol=1e-13)
    dq, dk, dv = attention_backward(q, k, v, do, False)
    dq2, dk2, dv2 = attention_backward(q, k[:, :, perm], v[:, :, perm], do, False)
    assert torch.allclose(dq, dq2, atol=1e-12)
    assert torch.allclose(dk[:, :, perm], dk2, atol=1e-12)
    assert torch.allclose(dv[:, :, perm], dv2, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_key_shift(causal):
    q, k, v = rnd(22, 1, 2, 25, 8), rnd(23, 1, 2, 25, 8), rnd(24, 1, 2, 25, 8)
    u = rnd(25, 8)
    tau = 0.41
    o, lse = attention_forward(q, k, v, causal, tau)
    o2, lse2 = attention_forward(q, k + u, v, causal, tau)
    assert torch.allclose(o, o2, atol=1e-12)
    assert torch.allclose(lse2, lse + tau * (q @ u), atol=1e-12)


def test_causal_prefix_and_last_row():
    q, k, v = rnd(26, 1, 2, 40, 8), rnd(27, 1, 2, 40, 8), rnd(28, 1, 2, 40, 8)
    o, lse = attention_forward(q, k, v, True)
    for m in (1, 7, 23):
        om, lm = attention_forward(q[:, :, :m], k[:, :, :m], v[:, :, :m], True)
        assert torch.allclose(o[:, :, :m], om, atol=1e-14) and torch.allclose(lse[:, :, :m], lm, atol=1e-14)
    onc, lnc = attention_forward(q, k, v, False)
    assert torch.allclose(o[:, :, -1], onc[:, :, -1], atol=1e-14)
    assert torch.allclose(lse[:, :, -1], lnc[:, :, -1], atol=1e-14)


def test_lse_split_merge():
    """Natural-log LSE over scaled scores: halves of the keys merge exactly."""
    q, k, v = rnd(29, 1, 2, 24, 8), rnd(30, 1, 2, 24, 8), rnd(31, 1, 2, 24, 8)
    tau = 0.29
    o, lse = attention_forward(q, k, v, False, tau)
    oa, la = attention_forward(q, k[:, :, :11], v[:, :, :11], False, tau)   # uneven split
    ob, lb = attention_forward(q, k[:, :, 11:], v[:, :, 11:], False, tau)
    l_m = torch.logaddexp(la, lb)
    o_m = torch.exp(la - l_m)[..., None] * oa + torch.exp(lb - l_m)[..., None] * ob
    assert torch.allclose(lse, l_m, atol=1e-13) and torch.allclose(o, o_m, atol=1e-13)


def test_large_logits_stay_finite():
    q, k, v = rnd(32, 1, 1, 16, 8, scale=8.0), rnd(33, 1, 1, 16, 8, scale=8.0), rnd(34, 1, 1, 16, 8)
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, causal)
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
        assert float(lse.abs().max()) > 50       # the scores really are large
        bo, bl = bf_forward(q, k, v, causal, default_scale(8))
        assert max_rel(o, bo) < 1e-12 and max_rel(lse, bl) < 1e-12


# --------------------------------------------------------------------------
# gradients
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G", [1, 2])
def test_gradients_finite_differences(causal, G):
    B, Hkv, N, d = 1, 1, 6, 3
    Hq = Hkv * G
    q, k, v, do = rnd(35, B, Hq, N, d), rnd(36, B, Hkv, N, d), rnd(37, B, Hkv, N, d), rnd(38, B, Hq, N, d)
    tau = 0.53
    dq, dk, dv = attention_backward(q, k, v, do, causal, tau)

    def loss(q_, k_, v_):
        o, _ = attention_forward(q_, k_, v_, causal, tau)
        return float((o * do).sum())

    h = 1e-6
    for tensor, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        fd = torch.zeros_like(tensor)
        flat = tensor.view(-1)
        for idx in range(flat.numel()):
            old = float(flat[idx])
            flat[idx] = old + h
            lp = loss(q, k, v)
            flat[idx] = old - h
            lm = loss(q, k, v)
            flat[idx] = old
            fd.view(-1)[idx] = (lp - lm) / (2 * h)
        err = float((fd - grad).abs().max()) / max(1e-3, float(grad.abs().max()))
        assert err < 1e-6, (which, err)


@pytest.mark.parametrize("causal", [True, False])
def test_gradient_identities(causal):
    B, Hq, Hkv, N, d = 2, 4, 2, 19, 8
    q, k, v, do = rnd(39, B, Hq, N, d), rnd(40, B, Hkv, N, d), rnd(41, B, Hkv, N, d), rnd(42, B, Hq, N, d)
    o, _ = attention_forward(q, k, v, causal)
    dq, dk, dv = attention_backward(q, k, v, do, causal)
    # rows of dS sum to zero -> sum_j dK_j = 0
    assert float(dk.sum(2).abs().max()) < 1e-12
    # rows of P sum to one -> sum_j dV_j = sum over the group's heads and rows of dO
    G = Hq // Hkv
    want = do.view(B, Hkv, G, N, d).sum((2, 3))
    assert torch.allclose(dv.sum(2), want, atol=1e-12)
    if causal:
        assert float(dq[:, :, 0].abs().max()) == 0.0
    # c_i = sum_k P_ik dP_ik equals dO_i . O_i (the shortcut a kernel may use)
    p = attention_probs(q, k, causal)
    vv = v.repeat_interleave(G, dim=1)
    dp = do @ vv.transpose(-1, -2)
    c = (p * dp).sum(-1)
    assert torch.allclose(c, (do * o).sum(-1), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_repeated_heads(causal):
    B, Hq, Hkv, N, d = 1, 6, 2, 14, 8
    G = Hq // Hkv
    q, k, v, do = rnd(43, B, Hq, N, d), rnd(44, B, Hkv, N, d), rnd(45, B, Hkv, N, d), rnd(46, B, Hq, N, d)
    o, lse = attention_forward(q, k, v, causal)
    kr, vr = k.repeat_interleave(G, 1), v.repeat_interleave(G, 1)
    o2, lse2 = attention_forward(q, kr, vr, causal)
    assert torch.allclose(o, o2, atol=1e-14) and torch.allclose(lse, lse2, atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, causal)
    dq2, dk2, dv2 = attention_backward(q, kr, vr, do, causal)
    assert torch.allclose(dq, dq2, atol=1e-13)
    assert torch.allclose(dk, dk2.view(B, Hkv, G, N, d).sum(2), atol=1e-13)
    assert torch.allclose(dv, dv2.view(B, Hkv, G, N, d).sum(2), atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_fp64(causal):
    """Library identity: torch's CPU scaled_dot_product_attention in float64."""
    q, k, v = rnd(47, 2, 3, 37, 16), rnd(48, 2, 3, 37, 16), rnd(49, 2, 3, 37, 16)
    o, _ = attention_forward(q, k, v, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    assert torch.allclose(o, ref, atol=1e-12)
    # gradients through autograd of the library routine
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    do = rnd(50, 2, 3, 37, 16)
    torch.nn.functional.scaled_dot_product_attention(qa, ka, va, is_causal=causal).backward(do)
    dq, dk, dv = attention_backward(q, k, v, do, causal)
    assert torch.allclose(dq, qa.grad, atol=1e-12)
    assert torch.allclose(dk, ka.grad, atol=1e-12)
    assert torch.allclose(dv, va.grad, atol=1e-12)


def test_row_samplers_match_full():
    B, Hq, Hkv, N, d = 1, 4, 2, 50, 8
    q, k, v, do = rnd(51, B, Hq, N, d), rnd(52, B, Hkv, N, d), rnd(53, B, Hkv, N, d), rnd(54, B, Hq, N, d)
    rows = [0, 3, 17, 49]
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, causal)
        dq, _, _ = attention_backward(q, k, v, do, causal)
        for h in range(Hq):
            orow, lrow = forward_rows(q, k, v, causal, None, 0, h, rows)
            assert torch.allclose(orow, o[0, h, rows], atol=1e-14)
            assert torch.allclose(lrow, lse[0, h, rows], atol=1e-14)
            assert torch.allclose(backward_dq_rows(q, k, v, do, causal, None, 0, h, rows),
                                  dq[0, h, rows], atol=1e-14)


@pytest.mark.parametrize("nq", [10, 4], ids=["square", "decode"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_probability_rows_match_bruteforce(causal, nq):
    """P itself, pinned to the scalar brute force: with V the identity (d = N_k)
    the brute force's output row i is sum_j P_ij e_j, i.e. row i of P.  Covers
    grouped heads (4 query heads on 2 K/V heads) and, with N_q = 4 < N_k = 10,
    queries at the last positions (decode alignment).  Both the full matrix
    (``attention_probs``) and selected rows (``probs_rows``) are checked."""
    Hq, Hkv, Nk = 4, 2, 10
    q, k = rnd(61, 1, Hq, nq, Nk), rnd(62, 1, Hkv, Nk, Nk)
    eye = torch.eye(Nk, dtype=torch.float64).expand(1, Hkv, Nk, Nk).contiguous()
    bo, _ = bf_forward(q, k, eye, causal, 0.37)
    bp = torch.tensor(bo, dtype=torch.float64)
    assert torch.allclose(attention_probs(q, k, causal, 0.37), bp, atol=1e-13)
    for h in range(Hq):
        rows = [nq - 1, 0, nq // 2]
        assert torch.allclose(probs_rows(q, k, causal, 0.37, 0, h, rows), bp[0, h, rows], atol=1e-13)
    if causal and nq < Nk:
        # the first decode query sits at position Nk - nq: it sees keys 0 .. Nk - nq only
        assert bool((bp[0, :, 0, Nk - nq + 1:] == 0).all()) and bool((bp[0, :, 0, :Nk - nq + 1] > 0).all())


def test_row_blocking_does_not_change_results():
    q, k, v, do = rnd(55, 1, 2, 70, 8), rnd(56, 1, 2, 70, 8), rnd(57, 1, 2, 70, 8), rnd(58, 1, 2, 70, 8)
    for causal in (True, False):
        a = attention_forward(q, k, v, causal, row_block=7)
        b = attention_forward(q, k, v, causal, row_block=512)
        assert torch.allclose(a[0], b[0], atol=1e-15) and torch.allclose(a[1], b[1], atol=1e-15)
        ga = attention_backward(q, k, v, do, causal, row_block=9)
        gb = attention_backward(q, k, v, do, causal, row_block=512)
        for x, y in zip(ga, gb):
            assert torch.allclose(x, y, atol=1e-13)


# --------------------------------------------------------------------------
# sliding window ([LONGCTX] §4): keys with |i - j| <= w, intersected with the
# causal mask
# --------------------------------------------------------------------------
WINDOWS = [0, 1, 2, 5, 8, 40]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_forward_matches_bruteforce(window, causal):
    B, Hq, Hkv, N, d = 2, 4, 2, 17, 8
    q, k, v = rnd(40, B, Hq, N, d), rnd(41, B, Hkv, N, d), rnd(42, B, Hkv, N, d)
    o, lse = attention_forward(q, k, v, causal, 0.41, row_block=5, window=window)
    bo, bl = bf_forward(q, k, v, causal, 0.41, window=window)
    assert max_rel(o, bo) < 1e-12 and max_rel(lse, bl) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [0, 1, 3, 11])
def test_window_backward_matches_bruteforce(window, causal):
    B, Hq, Hkv, N, d = 1, 4, 2, 12, 4
    q, k, v = rnd(43, B, Hq, N, d), rnd(44, B, Hkv, N, d), rnd(45, B, Hkv, N, d)
    do = rnd(46, B, Hq, N, d)
    dq, dk, dv = attention_backward(q, k, v, do, causal, 0.29, row_block=5, window=window)
    bq, bk, bv = bf_backward(q, k, v, do, causal, 0.29, window=window)
    assert max_rel(dq, bq) < 1e-11 and max_rel(dk, bk) < 1e-11 and max_rel(dv, bv) < 1e-11


@pytest.mark.parametrize("causal", [True, False])
def test_window_zero_is_identity(causal):
    """w = 0: every query sees only its own key, so O_i = v_i and LSE_i = tau q_i.k_i;
    P_ii = 1 makes dS = 0 (dQ = dK = 0) and dV_i the sum of dO_i over the group."""
    B, Hq, Hkv, N, d = 1, 4, 2, 10, 6
    q, k, v = rnd(47, B, Hq, N, d), rnd(48, B, Hkv, N, d), rnd(49, B, Hkv, N, d)
    do = rnd(50, B, Hq, N, d)
    tau = 0.7
    o, lse = attention_forward(q, k, v, causal, tau, window=0)
    G = Hq // Hkv
    for h in range(Hq):
        assert torch.allclose(o[0, h], v[0, h // G], rtol=0, atol=1e-15)
        assert torch.allclose(lse[0, h], tau * (q[0, h] * k[0, h // G]).sum(-1), rtol=0, atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, causal, tau, window=0)
    assert float(dq.abs().max()) < 1e-14 and float(dk.abs().max()) < 1e-14
    want_dv = do.reshape(B, Hkv, G, N, d).sum(2)
    assert torch.allclose(dv, want_dv, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_window_covering_everything_changes_nothing(causal):
    B, Hq, Hkv, N, d = 1, 2, 1, 23, 8
    q, k, v = rnd(51, B, Hq, N, d), rnd(52, B, Hkv, N, d), rnd(53, B, Hkv, N, d)
    o0, l0 = attention_forward(q, k, v, causal)
    for w in (N - 1, N, 10 * N):
        o, l = attention_forward(q, k, v, causal, window=w)
        assert torch.equal(o, o0) and torch.equal(l, l0)


def test_noncausal_window_is_symmetric_under_reversal():
    """The band |i - j| <= w is symmetric: reversing the sequence order of Q, K
    and V reverses the output rows (a causal mask would not survive this)."""
    B, Hq, Hkv, N, d = 1, 2, 2, 19, 8
    q, k, v = rnd(54, B, Hq, N, d), rnd(55, B, Hkv, N, d), rnd(56, B, Hkv, N, d)
    o, lse = attention_forward(q, k, v, False, window=4)
    o_r, lse_r = attention_forward(q.flip(2), k.flip(2), v.flip(2), False, window=4)
    assert torch.allclose(o_r.flip(2), o, atol=1e-13) and torch.allclose(lse_r.flip(2), lse, atol=1e-13)


def test_window_row_samplers_match_full():
    B, Hq, Hkv, N, d = 1, 2, 1, 50, 8
    q, k, v = rnd(57, B, Hq, N, d), rnd(58, B, Hkv, N, d), rnd(59, B, Hkv, N, d)
    do = rnd(60, B, Hq, N, d)
    o, lse = attention_forward(q, k, v, True, window=7)
    dq, _, _ = attention_backward(q, k, v, do, True, window=7)
    rows = [0, 3, 7, 8, 30, 49]
    ro, rl = forward_rows(q, k, v, True, None, 0, 1, rows, window=7)
    rq = backward_dq_rows(q, k, v, do, True, None, 0, 1, rows, window=7)
    assert torch.allclose(ro, o[0, 1, rows], atol=1e-14) and torch.allclose(rl, lse[0, 1, rows], atol=1e-14)
    assert torch.allclose(rq, dq[0, 1, rows], atol=1e-14)


def test_negative_window_is_rejected():
    q = rnd(61, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        attention_forward(q, q, q, True, window=-1)


# --------------------------------------------------------------------------
# decoding against a KV cache: N_q < N_k, queries are the last N_q positions
# ([EVOL] §1 and §3, [LONGCTX] §1.5)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("nq", [1, 2, 5, 13])
def test_decode_matches_bruteforce(nq, causal):
    B, Hq, Hkv, Nk, d = 2, 4, 2, 13, 8
    q, k, v = rnd(70, B, Hq, nq, d), rnd(71, B, Hkv, Nk, d), rnd(72, B, Hkv, Nk, d)
    o, lse = attention_forward(q, k, v, causal, 0.43, row_block=2)
    bo, bl = bf_forward(q, k, v, causal, 0.43)
    assert max_rel(o, bo) < 1e-12 and max_rel(lse, bl) < 1e-12


@pytest.mark.parametrize("window", [None, 3])
def test_decode_is_the_tail_of_the_full_problem(window):
    """Bottom-right alignment: the last N_q rows of the full causal problem are
    exactly the decode of those N_q queries against all N_k keys."""
    B, Hq, Hkv, Nk, d = 1, 4, 1, 40, 8
    q, k, v = rnd(73, B, Hq, Nk, d), rnd(74, B, Hkv, Nk, d), rnd(75, B, Hkv, Nk, d)
    o, lse = attention_forward(q, k, v, True, window=window)
    for nq in (1, 3, 17):
        od, ld = attention_forward(q[:, :, -nq:], k, v, True, window=window)
        assert torch.allclose(od, o[:, :, -nq:], atol=1e-14) and torch.allclose(ld, lse[:, :, -nq:], atol=1e-14)
        ro, rl = forward_rows(q[:, :, -nq:], k, v, True, None, 0, 2, [0, nq - 1], window=window)
        assert torch.allclose(ro, o[0, 2, [Nk - nq, Nk - 1]], atol=1e-14)


def test_decode_single_query_sees_every_key():
    """N_q = 1, causal: the one query sits at the last position, so the mask
    hides nothing and the result equals the unmasked one."""
    q, k, v = rnd(76, 1, 2, 1, 8), rnd(77, 1, 2, 30, 8), rnd(78, 1, 2, 30, 8)
    o1, l1 = attention_forward(q, k, v, True)
    o0, l0 = attention_forward(q, k, v, False)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_positional_mask_needs_enough_keys():
    q, k = rnd(79, 1, 1, 5, 4), rnd(80, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        attention_forward(q, k, k, True)
    attention_forward(q, k, k, False)           # no mask: any number of keys
