"""GPU backward parity: dQ, dK, dV from the HIP kernels against the fp64 oracle.

Bar: for each G in (dQ, dK, dV), max |G_gpu - G_ref| / max |G_ref| <= 2e-2.
The backward consumes the GPU forward's own O and LSE (as a caller would);
the oracle recomputes everything from the same bf16 inputs.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (TOL_GRAD_REL, TOL_LSE, TOL_O, assert_same_sum_to_bf16_ulp, bwd_head_split, dev_f64,
                         max_abs, rel_maxnorm, say, to_dev, to_f64)
from oracle import attention_backward, attention_forward
from synth_inputs import make_custom_inputs, make_inputs

pytestmark = pytest.mark.gpu


def run_fwd_bwd(attn, x, causal, scale=None):
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = attn.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_grads(attn, x, causal, scale=None, label=""):
    o, lse, dq, dk, dv = run_fwd_bwd(attn, x, causal, scale)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = attention_forward(f["q"], f["k"], f["v"], causal, scale)
    rdq, rdk, rdv = attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale)
    floor = 1e-3 * max(float(t.abs().max()) for t in (rdq, rdk, rdv))
    errs = {"O": max_abs(dev_f64(o), ro), "LSE": max_abs(dev_f64(lse), rl),
            "dQ": rel_maxnorm(dev_f64(dq), rdq, floor), "dK": rel_maxnorm(dev_f64(dk), rdk, floor),
            "dV": rel_maxnorm(dev_f64(dv), rdv, floor)}
    print(f"{label} causal={causal}: " + " ".join(f"{k}={v:.3g}" for k, v in errs.items()))
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE
    assert max(errs["dQ"], errs["dK"], errs["dV"]) <= TOL_GRAD_REL, errs
    return errs


SMALL = [
    # B, Hq, Hkv, N, d
    (1, 1, 1, 1, 128),
    (1, 1, 1, 2, 64),
    (2, 4, 2, 17, 128),
    (1, 2, 1, 255, 64),
    (1, 4, 4, 257, 128),
    (1, 8, 1, 300, 128),    # multi-query: dK/dV summed over 8 heads
    (3, 2, 2, 100, 64),
    (1, 2, 2, 64, 128),
    (1, 6, 3, 513, 128),
    (1, 4, 2, 1000, 64),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}".format(*s))
def test_bwd_small_shapes(gpu_lib, shape, causal):
    B, Hq, Hkv, N, d = shape
    say(f"bwd small {shape} causal={causal}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=300 + N + d, with_grad=True)
    check_grads(gpu_lib, x, causal, label=str(shape))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_bwd_tiny_workload(gpu_lib, causal):
    say(f"bwd tiny causal={causal}")
    x = make_inputs("tiny")
    x.update({"do": make_custom_inputs(1, 2, 2, 256, 64, seed=1000, with_grad=True)["do"]})
    check_grads(gpu_lib, x, causal, label="tiny")


def test_bwd_custom_scale(gpu_lib):
    say("bwd custom scale")
    x = make_custom_inputs(1, 4, 2, 333, 128, seed=12, with_grad=True)
    check_grads(gpu_lib, x, True, scale=0.3, label="scale0.3")
    check_grads(gpu_lib, x, False, scale=0.05, label="scale0.05")


def test_bwd_gqa_2k(gpu_lib):
    say("bwd gqa 2K")
    x = make_custom_inputs(1, 16, 2, 2048, 128, seed=13, with_grad=True)
    check_grads(gpu_lib, x, True, label="gqa Hq16 Hkv2 N2048")


@pytest.mark.timeout(900)
def test_bwd_fb_32k_full(gpu_lib):
    """B=1, H=8, N=32768, d=128 causal: every element of O, LSE, dQ, dK, dV
    against the oracle, one head at a time (each head is independent here)."""
    say("bwd fb-32K full")
    x = make_inputs("fb-32K")
    o, lse, dq, dk, dv = run_fwd_bwd(gpu_lib, x, True)
    tensors = {n: dev_f64(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    worst = {"O": 0.0, "LSE": 0.0}
    num = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    den = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for h in range(8):
        f = {n: to_f64(x[n][:, h:h + 1]) for n in ("q", "k", "v", "do")}
        ro, rl = attention_forward(f["q"], f["k"], f["v"], True)
        rdq, rdk, rdv = attention_backward(f["q"], f["k"], f["v"], f["do"], True)
        worst["O"] = max(worst["O"], max_abs(tensors["o"][:, h:h + 1], ro))
        worst["LSE"] = max(worst["LSE"], max_abs(tensors["lse"][:, h:h + 1], rl))
        for key, got, ref in (("dQ", tensors["dq"][:, h:h + 1], rdq), ("dK", tensors["dk"][:, h:h + 1], rdk),
                              ("dV", tensors["dv"][:, h:h + 1], rdv)):
            num[key] = max(num[key], max_abs(got, ref))
            den[key] = max(den[key], float(ref.abs().max()))
        print(f"  head {h}: O={worst['O']:.3g} LSE={worst['LSE']:.3g} "
              + " ".join(f"{k}={num[k] / den[k]:.3g}" for k in num), flush=True)
    rel = {k: num[k] / den[k] for k in num}
    print(f"fb-32K full check: {worst} {rel}")
    assert worst["O"] <= TOL_O and worst["LSE"] <= TOL_LSE
    assert max(rel.values()) <= TOL_GRAD_REL, rel


@pytest.mark.parametrize("shape", [(1, 8, 2, 1200, 128), (4, 8, 8, 1200, 128)], ids=["split", "plain"])
def test_bwd_deterministic(gpu_lib, shape):
    """Bitwise run-to-run determinism, with and without the head split."""
    say(f"bwd determinism {shape}")
    assert bwd_head_split(gpu_lib, *shape) == (shape[1] != shape[2])
    x = make_custom_inputs(*shape, seed=14, with_grad=True)
    a = run_fwd_bwd(gpu_lib, x, True)
    b = run_fwd_bwd(gpu_lib, x, True)
    for t1, t2 in zip(a, b):
        assert torch.equal(t1, t2)


# Shapes whose backward shares each K/V head's query heads out over several
# workgroups (fp32 partial dK/dV in the workspace, added by a reduction):
# multi-query with many heads, grouped heads with a ragged last key block,
# d = 64, a batch, a prime group size.
HEAD_SPLIT = [
    # B, Hq, Hkv, N, d
    (1, 16, 1, 1000, 128),
    (1, 12, 2, 777, 64),
    (2, 8, 2, 300, 128),
    (1, 6, 3, 129, 128),
    (1, 31, 1, 500, 64),     # prime group: its only split is all 31 heads apart
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", HEAD_SPLIT, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}".format(*s))
def test_bwd_head_split(gpu_lib, shape, causal):
    say(f"bwd head split {shape} causal={causal}")
    assert bwd_head_split(gpu_lib, *shape)
    x = make_custom_inputs(*shape, seed=1700 + shape[3] + shape[1], with_grad=True)
    check_grads(gpu_lib, x, causal, label=f"split {shape}")


@pytest.mark.parametrize("window", [None, 500], ids=["causal", "causal_w500"])
def test_bwd_workgroup_sizes_agree_bitwise(gpu_lib, window):
    """At d = 128 the gradient launch takes 4-wave blocks (64 keys, 128
    queries) when its 8-wave grid has fewer than 256 blocks, 8-wave blocks
    above; a wave's work is the same in both.  With one query head per K/V
    head the heads are independent, so the first half of the heads (192
    eight-wave blocks: a 4-wave launch) must give bitwise the gradients the
    whole problem (384: an 8-wave launch) gives for them."""
    say(f"bwd 4-wave vs 8-wave workgroups window={window}")
    x = make_custom_inputs(1, 8, 8, 4096, 128, seed=18, with_grad=True)
    half = {n: np.ascontiguousarray(x[n][:, :4]) for n in ("q", "k", "v", "do")}

    def grads(inp):
        q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
        o, lse = gpu_lib.fwd(q, k, v, causal=True, window=window)
        return gpu_lib.bwd(q, k, v, o, lse, do, causal=True, window=window)

    full_g, half_g = grads(x), grads(half)
    torch.cuda.synchronize()
    for a, b in zip(full_g, half_g):
        assert torch.equal(a[:, :4], b)


@pytest.mark.timeout(600)
def test_bwd_head_split_mqa_4k(gpu_lib):
    """Multi-query at its working size: 32 query heads over one K/V head,
    N = 4096, causal -- the backward splits the heads 16 ways (512 dK/dV
    workgroups); every element of dQ, dK, dV against the oracle."""
    shape = (1, 32, 1, 4096, 128)
    say(f"bwd head split mqa {shape}")
    assert bwd_head_split(gpu_lib, *shape)
    x = make_custom_inputs(*shape, seed=1750, with_grad=True)
    check_grads(gpu_lib, x, True, label="mqa 32/1 4K")


def test_bwd_workspace_errors(gpu_lib):
    say("bwd workspace too small")
    x = make_custom_inputs(1, 2, 2, 64, 128, seed=15, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.fwd(q, k, v)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.AttnError) as e:
        gpu_lib.bwd(q, k, v, o, lse, do, workspace=small)
    assert e.value.code == 4


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape,split", [((4, 8, 4, 2048, 128), False), ((2, 6, 2, 700, 128), True),
                                         ((4, 8, 4, 2048, 64), False)],
                         ids=["plain", "split", "plain_d64"])
def test_bwd_stages_equal_bwd(gpu_lib, shape, split, causal):
    """preprocess -> dkdv -> dq and preprocess -> grads give what attn_bwd
    gives: bitwise without the head split; with it, dQ bitwise and dK, dV (one
    fp32 sum over the query heads in the stages, per-split sums added in split
    order in attn_bwd) to one bf16 unit in the last place."""
    say(f"bwd stages {shape} causal={causal}")
    assert bwd_head_split(gpu_lib, *shape) == split
    x = make_custom_inputs(*shape, seed=16, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.fwd(q, k, v, causal=causal)
    dq, dk, dv = gpu_lib.bwd(q, k, v, o, lse, do, causal=causal)
    delta = gpu_lib.bwd_preprocess(o, do)
    dk2, dv2 = gpu_lib.bwd_dkdv(q, k, v, do, lse, delta, causal=causal)
    dq2 = gpu_lib.bwd_dq(q, k, v, do, lse, delta, causal=causal)
    dq3, dk3, dv3 = gpu_lib.bwd_grads(q, k, v, do, lse, delta, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dq, dq3)
    assert torch.equal(dk2, dk3) and torch.equal(dv2, dv3)
    if split:
        assert_same_sum_to_bf16_ulp(dk, dk2)
        assert_same_sum_to_bf16_ulp(dv, dv2)
    else:
        assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # delta is the softmax-Jacobian row term: rowsum(dO * O) of the bf16 tensors
    ref = (do.float() * o.float()).sum(-1)
    assert float((delta - ref).abs().max()) <= 1e-4 * float(ref.abs().max())
