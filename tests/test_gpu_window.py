"""GPU parity of sliding-window attention against the fp64 oracle.

The window follows the long-context page's sliding-window passage (section on
sparse attention): query i sees key j only when |i - j| <= w, intersected with
j <= i under the causal mask.  Same bars as the plain path: max |O| error <=
1e-2, max |LSE| error <= 1e-3, and max |G_gpu - G_ref| / max |G_ref| <= 2e-2
for dQ, dK, dV.  Windows cover the edge cases of the tiling: 0 (only the
diagonal), below, at and just past the 32-key MFMA block and the 128-key tile,
windows that leave rows whose first visited tile is entirely outside their
band, and windows that cover every key (the plain kernels, bitwise).
"""
import pytest
import torch

from gpu_helpers import (TOL_GRAD_REL, TOL_LSE, TOL_O, assert_same_sum_to_bf16_ulp, bwd_head_split, dev_f64,
                         max_abs, rel_maxnorm, say, to_dev, to_f64)
from oracle import attention_backward, attention_forward, backward_dq_rows, forward_rows
from synth_inputs import make_custom_inputs

pytestmark = pytest.mark.gpu


def run(attn, x, causal, window, scale=None, with_grad=True):
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = attn.fwd(q, k, v, causal=causal, scale=scale, window=window)
    grads = None
    if with_grad:
        do = to_dev(x["do"])
        grads = attn.bwd(q, k, v, o, lse, do, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    return o, lse, grads


def check(attn, x, causal, window, scale=None, label=""):
    o, lse, (dq, dk, dv) = run(attn, x, causal, window, scale)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = attention_forward(f["q"], f["k"], f["v"], causal, scale, window=window)
    rdq, rdk, rdv = attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale, window=window)
    floor = 1e-3 * max(float(t.abs().max()) for t in (rdq, rdk, rdv))
    errs = {"O": max_abs(dev_f64(o), ro), "LSE": max_abs(dev_f64(lse), rl),
            "dQ": rel_maxnorm(dev_f64(dq), rdq, floor), "dK": rel_maxnorm(dev_f64(dk), rdk, floor),
            "dV": rel_maxnorm(dev_f64(dv), rdv, floor)}
    print(f"{label} causal={causal} w={window}: " + " ".join(f"{k}={v:.3g}" for k, v in errs.items()))
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE, errs
    assert max(errs["dQ"], errs["dK"], errs["dV"]) <= TOL_GRAD_REL, errs


CASES = [
    # B, Hq, Hkv, N, d, window
    (1, 2, 2, 300, 128, 0),
    (1, 2, 1, 300, 128, 1),
    (1, 4, 2, 700, 128, 31),
    (1, 2, 2, 700, 64, 32),
    (2, 2, 2, 513, 128, 100),
    (1, 4, 4, 1000, 128, 127),
    (1, 2, 2, 1000, 128, 128),
    (1, 8, 1, 777, 128, 129),     # multi-query
    (1, 2, 2, 1100, 64, 255),
    (1, 3, 3, 1300, 128, 600),
    (1, 2, 2, 200, 128, 198),     # w = N - 2: the windowed kernels, nearly no effect
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_N{}_d{}_w{}".format(*c))
def test_window_small(gpu_lib, case, causal):
    B, Hq, Hkv, N, d, w = case
    say(f"window {case} causal={causal}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=300 + N + w, with_grad=True)
    check(gpu_lib, x, causal, w, label=str(case))


def test_window_custom_scale(gpu_lib):
    say("window custom scale")
    x = make_custom_inputs(1, 4, 2, 600, 128, seed=31, with_grad=True)
    check(gpu_lib, x, True, 77, scale=0.3)
    check(gpu_lib, x, False, 200, scale=0.05)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_window_covering_every_key_is_the_plain_call(gpu_lib, causal):
    """w >= N - 1 is exactly the unwindowed problem and takes the plain kernels."""
    say(f"window >= N-1 causal={causal}")
    x = make_custom_inputs(1, 4, 2, 700, 128, seed=32, with_grad=True)
    base = run(gpu_lib, x, causal, None)
    for w in (699, 700, 10 ** 6):
        got = run(gpu_lib, x, causal, w)
        assert torch.equal(got[0], base[0]) and torch.equal(got[1], base[1])
        for a, b in zip(got[2], base[2]):
            assert torch.equal(a, b)


@pytest.mark.parametrize("shape,split", [((2, 4, 2, 900, 128), True), ((4, 8, 4, 2048, 128), False)],
                         ids=["split", "plain"])
def test_window_deterministic_and_stages(gpu_lib, shape, split):
    """Bitwise run-to-run determinism; preprocess + grads_window equals
    bwd_window (bitwise; dK and dV to one bf16 unit in the last place when
    bwd_window splits the query heads of each K/V head)."""
    say(f"window determinism and stages {shape}")
    assert bwd_head_split(gpu_lib, *shape) == split
    x = make_custom_inputs(*shape, seed=33, with_grad=True)
    a = run(gpu_lib, x, True, 130)
    b = run(gpu_lib, x, True, 130)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for u, v in zip(a[2], b[2]):
        assert torch.equal(u, v)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = a[0], a[1]
    delta = gpu_lib.bwd_preprocess(o, do)
    g = gpu_lib.bwd_grads(q, k, v, do, lse, delta, causal=True, window=130)
    torch.cuda.synchronize()
    assert torch.equal(g[0], a[2][0])
    for u, v in zip(g[1:], a[2][1:]):
        if split:
            assert_same_sum_to_bf16_ulp(v, u)
        else:
            assert torch.equal(u, v)


def test_window_medium_full_check(gpu_lib):
    """N = 4096 over several 256-row query blocks and 128-key tiles, checked in full."""
    say("window medium N=4096 w=700")
    x = make_custom_inputs(1, 2, 1, 4096, 128, seed=34, with_grad=True)
    check(gpu_lib, x, True, 700, label="N4096")


def test_window_long_sampled_rows(gpu_lib):
    """The benchmarked sliding-window shape (B=1, H=8, N=32768, d=128, causal,
    w=4096), in the launch configuration the benchmark times: O, LSE and dQ on
    sampled rows of two heads, each row computed by the oracle on its own."""
    say("window long N=32768 w=4096 sampled rows")
    N, w = 32768, 4096
    x = make_custom_inputs(1, 8, 8, N, 128, seed=35, with_grad=True)
    o, lse, (dq, dk, dv) = run(gpu_lib, x, True, w)
    rows = [0, 1, 127, 128, 4095, 4096, 4097, 9000, 20000, N - 129, N - 1]
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    for h in (0, 5):
        ro, rl = forward_rows(f["q"], f["k"], f["v"], True, None, 0, h, rows, window=w)
        assert max_abs(dev_f64(o[0, h, rows]), ro) <= TOL_O
        assert max_abs(dev_f64(lse[0, h, rows]), rl) <= TOL_LSE
        rq = backward_dq_rows(f["q"], f["k"], f["v"], f["do"], True, None, 0, h, rows, window=w)
        assert rel_maxnorm(dev_f64(dq[0, h, rows]), rq) <= TOL_GRAD_REL
    for t in (dk, dv):
        assert bool(torch.isfinite(t.float()).all())
