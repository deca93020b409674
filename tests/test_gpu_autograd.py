"""The autograd entry points (``attention``, ``attention_varlen``) on the GPU.

They only route tensors: O and every gradient must be bitwise what the direct
calls (``fwd``/``bwd``, ``fwd_varlen``/``bwd_varlen``) return for the same
inputs, including when the upstream gradient reaches the backward as a
non-contiguous tensor.  One case is also checked against the fp64 oracle at the
parity tolerances.
"""
import pytest
import torch

from gpu_helpers import TOL_GRAD_REL, TOL_O, dev_f64, max_abs, rel_maxnorm, say, to_dev, to_f64
from oracle import attention_backward, attention_forward
from synth_inputs import cu_from_lengths, make_custom_inputs

pytestmark = pytest.mark.gpu


def leaf(bits):
    return to_dev(bits).requires_grad_(True)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("window", [None, 64], ids=["nowin", "w64"])
def test_attention_autograd_is_fwd_bwd(gpu_lib, causal, window):
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 128
    say(f"autograd attention causal={causal} window={window}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=900 + causal + (window or 0), with_grad=True)
    q, k, v = leaf(x["q"]), leaf(x["k"]), leaf(x["v"])
    do = to_dev(x["do"])
    o, lse = gpu_lib.attention(q, k, v, causal=causal, window=window, return_lse=True)
    o.backward(do)
    torch.cuda.synchronize()
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o_ref, lse_ref = gpu_lib.fwd(qd, kd, vd, causal=causal, window=window)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o_ref, lse_ref, do, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
    assert not lse.requires_grad


def test_attention_autograd_against_oracle(gpu_lib):
    B, Hq, Hkv, N, d = 1, 4, 1, 257, 64
    say("autograd attention vs oracle")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=911, with_grad=True)
    q, k, v = leaf(x["q"]), leaf(x["k"]), leaf(x["v"])
    o = gpu_lib.attention(q, k, v, causal=True)
    o.backward(to_dev(x["do"]))
    torch.cuda.synchronize()
    args = [to_f64(x[n]) for n in ("q", "k", "v")]
    ro, _ = attention_forward(*args, True)
    rq, rk, rv = attention_backward(*args, to_f64(x["do"]), True)
    assert max_abs(dev_f64(o), ro) <= TOL_O
    floor = 1e-3 * max(float(t.abs().max()) for t in (rq, rk, rv))
    for g, r in ((q.grad, rq), (k.grad, rk), (v.grad, rv)):
        assert rel_maxnorm(dev_f64(g), r, floor) <= TOL_GRAD_REL


def test_attention_autograd_noncontiguous_upstream(gpu_lib):
    # loss = sum(O * w) with w broadcast from one row: the gradient reaching the
    # backward is an expanded (stride-0) tensor
    B, Hq, Hkv, N, d = 1, 2, 2, 200, 128
    say("autograd attention, expanded upstream gradient")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=921)
    q, k, v = leaf(x["q"]), leaf(x["k"]), leaf(x["v"])
    w = torch.linspace(-1, 1, d, device="cuda", dtype=torch.bfloat16).expand(B, Hq, N, d)
    (gpu_lib.attention(q, k, v, causal=True) * w).sum().backward()
    torch.cuda.synchronize()
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o_ref, lse_ref = gpu_lib.fwd(qd, kd, vd, causal=True)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o_ref, lse_ref, w.contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


def test_attention_varlen_autograd_is_fwd_bwd(gpu_lib):
    lengths, Hq, Hkv, d = [5, 0, 17, 300, 1], 4, 2, 128
    T = sum(lengths)
    say(f"autograd attention_varlen lengths={lengths}")
    x = make_custom_inputs(1, Hq, Hkv, T, d, seed=931, with_grad=True)
    q, k, v = (leaf(x[n][0]) for n in ("q", "k", "v"))
    do = to_dev(x["do"][0])
    cu = torch.from_numpy(cu_from_lengths(lengths)).cuda()
    o = gpu_lib.attention_varlen(q, k, v, cu, max(lengths), causal=True)
    o.backward(do)
    torch.cuda.synchronize()
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o_ref, lse_ref = gpu_lib.fwd_varlen(qd, kd, vd, cu, max(lengths), causal=True)
    dq, dk, dv = gpu_lib.bwd_varlen(qd, kd, vd, o_ref, lse_ref, do, cu, max(lengths), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
