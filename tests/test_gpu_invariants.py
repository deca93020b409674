"""GPU-side invariants at sizes where the oracle would be slow.

Each test runs the HIP path twice on inputs that the mathematics relates and
checks the relation, at the parity tolerances (max |O| error <= 1e-2, max
|LSE| error <= 1e-3, gradients <= 2e-2 of the max-norm):

  * permuting K and V together leaves non-causal attention unchanged, and the
    key gradients permute with them (the softmax sums over keys without regard
    to order: page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §4);
  * attention over two disjoint key sets, merged through their log-sum-exps,
    is attention over their union (the rescaling identity behind the blockwise
    softmax: page "6.1 … 長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.2);
  * adding one vector u to every key adds tau q_i . u to every score of row i,
    which the softmax cancels: O, dQ, dK, dV are unchanged and LSE_i moves by
    tau q_i . u.  K is drawn on a 1/64 grid in [-1.5, 1.5] so that K and K + 1
    are both exact in bf16.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_GRAD_REL, TOL_LSE, TOL_O, max_abs, rel_maxnorm, say, to_dev
from synth_inputs import f32_to_bf16_bits, make_custom_inputs

pytestmark = pytest.mark.gpu


def f64(t: torch.Tensor) -> torch.Tensor:
    return t.detach().double().cpu()


def test_key_permutation_noncausal(gpu_lib):
    B, Hq, Hkv, N, d = 1, 4, 2, 8192, 128
    say(f"invariant: key permutation B{B} Hq{Hq} Hkv{Hkv} N{N} d{d}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=811, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    perm = torch.from_numpy(np.random.default_rng(812).permutation(N)).cuda()
    kp, vp = k[:, :, perm].contiguous(), v[:, :, perm].contiguous()
    o, lse = gpu_lib.fwd(q, k, v, causal=False)
    op, lsep = gpu_lib.fwd(q, kp, vp, causal=False)
    dq, dk, dv = gpu_lib.bwd(q, k, v, o, lse, do, causal=False)
    dqp, dkp, dvp = gpu_lib.bwd(q, kp, vp, op, lsep, do, causal=False)
    torch.cuda.synchronize()
    assert max_abs(f64(op), f64(o)) <= TOL_O
    assert max_abs(f64(lsep), f64(lse)) <= TOL_LSE
    assert rel_maxnorm(f64(dqp), f64(dq)) <= TOL_GRAD_REL
    assert rel_maxnorm(f64(dkp), f64(dk[:, :, perm])) <= TOL_GRAD_REL
    assert rel_maxnorm(f64(dvp), f64(dv[:, :, perm])) <= TOL_GRAD_REL


@pytest.mark.parametrize("split", [3000, 4096, 127])
def test_lse_split_merge(gpu_lib, split):
    # queries against the whole cache, and against keys [0, split) and
    # [split, Nk) separately (non-causal decode calls), merged by LSE
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 96, 8192, 128
    say(f"invariant: LSE split-merge Nq{Nq} Nk{Nk} split{split}")
    xq = make_custom_inputs(B, Hq, Hkv, Nq, d, seed=820 + split)
    xk = make_custom_inputs(B, Hq, Hkv, Nk, d, seed=830 + split)
    q, k, v = to_dev(xq["q"]), to_dev(xk["k"]), to_dev(xk["v"])
    assert min(split, Nk - split) >= Nq   # the decode call needs Nq <= Nk
    parts = [gpu_lib.fwd_decode(q, k[:, :, lo:hi].contiguous(), v[:, :, lo:hi].contiguous(), causal=False)
             for lo, hi in ((0, split), (split, Nk))]
    o, lse = gpu_lib.fwd_decode(q, k, v, causal=False)
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = ((f64(a), f64(b)) for a, b in parts)
    lm = torch.logaddexp(l1, l2)
    om = torch.exp(l1 - lm)[..., None] * o1 + torch.exp(l2 - lm)[..., None] * o2
    assert max_abs(om, f64(o)) <= TOL_O
    assert max_abs(lm, f64(lse)) <= TOL_LSE


def grid_keys(shape, seed):
    rng = np.random.default_rng(seed)
    k = np.clip(np.round(rng.standard_normal(shape) * 16) / 16, -6, 6).astype(np.float32)
    return k


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_key_shift(gpu_lib, causal):
    B, Hq, Hkv, N, d = 1, 4, 2, 4099, 128
    say(f"invariant: key shift causal={causal} N{N}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=840 + causal, with_grad=True)
    kf = grid_keys((B, Hkv, N, d), 841 + causal) * 0.25      # grid 1/64, |k| <= 1.5
    kbits = f32_to_bf16_bits(kf)
    kbits_shift = f32_to_bf16_bits(kf + 1.0)
    # the grid makes both exact in bf16 (8 significant bits cover 2.5 in steps of 1/64)
    assert np.array_equal(kbits.astype(np.uint32) << 16, kf.view(np.uint32))
    assert np.array_equal(kbits_shift.astype(np.uint32) << 16, (kf + 1.0).astype(np.float32).view(np.uint32))
    q, v, do = to_dev(x["q"]), to_dev(x["v"]), to_dev(x["do"])
    k, ks = to_dev(kbits), to_dev(kbits_shift)
    tau = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.fwd(q, k, v, causal=causal)
    os_, lses = gpu_lib.fwd(q, ks, v, causal=causal)
    dq, dk, dv = gpu_lib.bwd(q, k, v, o, lse, do, causal=causal)
    dqs, dks, dvs = gpu_lib.bwd(q, ks, v, os_, lses, do, causal=causal)
    torch.cuda.synchronize()
    shift = tau * f64(q).sum(-1)                                # tau q_i . u with u = 1
    assert max_abs(f64(os_), f64(o)) <= TOL_O
    assert max_abs(f64(lses), f64(lse) + shift) <= TOL_LSE
    assert rel_maxnorm(f64(dqs), f64(dq)) <= TOL_GRAD_REL
    assert rel_maxnorm(f64(dks), f64(dk)) <= TOL_GRAD_REL
    assert rel_maxnorm(f64(dvs), f64(dv)) <= TOL_GRAD_REL
