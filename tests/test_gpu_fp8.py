"""GPU parity of the 8-bit (E4M3) forward against the fp64 oracle.

The oracle gives the exact attention of the dequantized inputs.  The kernel
rounds one more thing -- the probabilities, scaled by 2^8 and rounded to
E4M3 before the P V product (relative error <= 2^-4; in the subnormal range
absolute error <= 2^-18 of the row's largest probability) -- so the bar for
every element of O is the bound that rounding implies,

    |O_it - O_ref_it| <= sum_j max(2^-4 P_ij, 2^-18 max_k P_ik) |v_jt|
                         + 2^-8 |O_ref_it| (O's bf16 rounding)
                         + 1e-4 sum_j P_ij |v_jt| (fp32 scores, exp2, sums),

and LSE (fp32 statistics of unrounded probabilities) keeps the bf16 forward's
bar, |LSE - LSE_ref| <= 1e-3.
"""
import pytest
import torch

from gpu_helpers import TOL_LSE, dev_f64, say
from oracle import attention_probs, dequantize, forward_rows, fp8_attention_forward, probs_rows
from synth_inputs import WORKLOADS, make_fp8_inputs, make_inputs

pytestmark = pytest.mark.gpu


def dev_u8(a):
    return torch.from_numpy(a).cuda()


def run(attn, x, causal, scale=None):
    o, lse = attn.fwd_fp8(dev_u8(x["q8"]), dev_u8(x["k8"]), dev_u8(x["v8"]),
                          torch.from_numpy(x["q_descale"]).cuda(), torch.from_numpy(x["k_descale"]).cuda(),
                          torch.from_numpy(x["v_descale"]).cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dev_f64(o), dev_f64(lse)


def bound(p, v_abs, o_ref):
    """Per-element tolerance from the rows of P ([rows, N_k]), |V| ([N_k, d]) and O_ref."""
    pmax = p.max(dim=1, keepdim=True).values
    e = torch.maximum(2.0 ** -4 * p, (2.0 ** -18) * pmax * (p > 0))
    return e @ v_abs + 2.0 ** -8 * o_ref.abs() + 1e-4 * (p @ v_abs)


def check(attn, x, causal, scale=None, label=""):
    o, lse = run(attn, x, causal, scale)
    ro, rl = fp8_attention_forward(x["q8"], x["k8"], x["v8"], x["q_descale"], x["k_descale"],
                                   x["v_descale"], causal, scale)
    q, k, v = (dequantize(x[n + "8"], x[n + "_descale"]) for n in ("q", "k", "v"))
    P = attention_probs(q, k, causal, scale)
    G = q.shape[1] // k.shape[1]
    worst, mean_err = 0.0, 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            tol = bound(P[b, h], v[b, h // G].abs(), ro[b, h])
            err = (o[b, h] - ro[b, h]).abs()
            # a zero bound (a head whose values are all zero) admits no error
            worst = max(worst, float((err / tol.clamp_min(1e-300)).max()))
            mean_err = max(mean_err, float(err.mean()))
    el = float((lse - rl).abs().max())
    print(f"{label}: max err/bound={worst:.3g} mean |err|={mean_err:.3g} LSE={el:.3g}")
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert worst <= 1.0 and el <= TOL_LSE, (worst, el)


SMALL = [
    # B, Hq, Hkv, N
    (1, 1, 1, 1),
    (1, 2, 1, 17),
    (2, 4, 2, 255),
    (1, 4, 4, 257),
    (1, 8, 1, 300),     # multi-query
    (1, 2, 2, 1000),
    (1, 3, 3, 1500),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}".format(*s))
def test_fp8_small(gpu_lib, shape, causal):
    B, Hq, Hkv, N = shape
    say(f"fp8 {shape} causal={causal}")
    check(gpu_lib, make_fp8_inputs(B, Hq, Hkv, N, 128, seed=N + Hq), causal, label=str(shape))


def test_fp8_custom_scale(gpu_lib):
    say("fp8 custom scale")
    check(gpu_lib, make_fp8_inputs(1, 2, 1, 400, 128, seed=77), True, scale=0.3, label="scale 0.3")


def test_fp8_benchmark_shape_sampled_rows(gpu_lib):
    """The benchmarked 8-bit forward (B=1, H=32, N=8192, d=128, causal) in the
    launch configuration the bench times; sampled rows of every head against
    the oracle, each under its own bound."""
    say("fp8 fwd-8K sampled rows")
    w = WORKLOADS["fp8-8K"]
    x = make_inputs(w)
    o, lse = run(gpu_lib, x, True)
    q, k, v = (dequantize(x[n + "8"], x[n + "_descale"]) for n in ("q", "k", "v"))
    rows = [0, 1, 31, 32, 255, 256, 1000, 4095, 4096, 6000, 8190, 8191]
    worst, el = 0.0, 0.0
    for h in range(0, w.Hq, 3):
        ro, rl = forward_rows(q, k, v, True, None, 0, h, rows)
        p = probs_rows(q, k, True, None, 0, h, rows)
        tol = bound(p, v[0, h].abs(), ro)
        worst = max(worst, float(((o[0, h, rows] - ro).abs() / tol).max()))
        el = max(el, float((lse[0, h, rows] - rl).abs().max()))
    print(f"fp8-8K sampled: max err/bound={worst:.3g} LSE={el:.3g}")
    assert worst <= 1.0 and el <= TOL_LSE


def test_fp8_deterministic(gpu_lib):
    say("fp8 determinism")
    x = make_fp8_inputs(1, 8, 2, 1200, 128, seed=13)
    a = run(gpu_lib, x, True)
    b = run(gpu_lib, x, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("causal,heads", [(True, 16), (False, 8)], ids=["causal", "full"])
def test_fp8_workgroup_sizes_agree_bitwise(gpu_lib, causal, heads):
    """The launch takes 4-wave workgroups when 8-wave ones would not fill the
    chip (causal: at most one 8-wave block per CU; otherwise: fewer than one)
    and 8-wave ones above that; a wave's work is the same in both.  Heads are
    independent, so the first half of the heads of an N = 8192 problem (a
    4-wave launch) must give bitwise the outputs the whole problem (an 8-wave
    launch) gives for them."""
    say(f"fp8 4-wave vs 8-wave workgroups causal={causal}")
    x = make_fp8_inputs(1, heads, heads, 8192, 128, seed=47)
    half = {n: x[n][:, : heads // 2].copy() for n in ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")}
    o_all, lse_all = run(gpu_lib, x, causal)
    o_half, lse_half = run(gpu_lib, half, causal)
    assert torch.equal(o_all[:, : heads // 2], o_half) and torch.equal(lse_all[:, : heads // 2], lse_half)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_fp8_zero_descales(gpu_lib, causal):
    """A zero descale is an all-zero head: zero queries (uniform attention over
    the visible keys), zero keys (the same), zero values (O = 0).  Checked
    against the oracle on the dequantized values under the usual bound."""
    say(f"fp8 zero descales causal={causal}")
    x = make_fp8_inputs(1, 6, 3, 300, 128, seed=41)
    x["q_descale"][0, 1] = 0.0          # query head 1
    x["k_descale"][0, 1] = 0.0          # K/V head 1: query heads 2 and 3
    x["v_descale"][0, 2] = 0.0          # K/V head 2: query heads 4 and 5
    check(gpu_lib, x, causal, label="zero descales")


def test_fp8_negative_descale_product_is_nan(gpu_lib):
    """q_descale * k_descale < 0 has no meaningful max-shift in the kernel: that
    head's outputs are NaN, every other head is unaffected."""
    say("fp8 negative descale product")
    x = make_fp8_inputs(1, 4, 2, 260, 128, seed=43)
    clean = run(gpu_lib, x, True)
    x["q_descale"][0, 3] = -x["q_descale"][0, 3]
    o, lse = run(gpu_lib, x, True)
    assert bool(torch.isnan(o[0, 3]).all()) and bool(torch.isnan(lse[0, 3]).all())
    assert torch.equal(o[0, :3], clean[0][0, :3]) and torch.equal(lse[0, :3], clean[1][0, :3])
