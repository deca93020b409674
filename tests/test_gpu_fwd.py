"""GPU forward parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Every input is the seeded bf16 draw of ``synth_inputs``; the oracle consumes
the exact same bf16 values decoded to fp64.  Bar: max |O| error <= 1e-2 and
max |LSE| error <= 1e-3.  Small problems are compared element by element;
the full-size workloads are compared on sampled rows that the oracle computes
one by one, in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_LSE, TOL_O, dev_f64, max_abs, say, to_dev, to_f64
from oracle import attention_forward, forward_rows
from synth_inputs import WORKLOADS, make_custom_inputs, make_inputs

pytestmark = pytest.mark.gpu


def run_fwd(attn, x, causal, scale=None):
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o, lse = attn.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def check_full(attn, x, causal, scale=None, tol_o=TOL_O, tol_l=TOL_LSE):
    o, lse = run_fwd(attn, x, causal, scale)
    ro, rl = attention_forward(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), causal, scale)
    eo, el = max_abs(dev_f64(o), ro), max_abs(dev_f64(lse), rl)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    assert eo <= tol_o and el <= tol_l, (eo, el)
    return eo, el


SMALL = [
    # B, Hq, Hkv, N, d
    (1, 1, 1, 1, 64),
    (1, 1, 1, 1, 128),
    (1, 2, 1, 2, 128),
    (2, 4, 2, 17, 128),
    (1, 2, 1, 255, 64),
    (1, 4, 4, 257, 128),
    (1, 8, 1, 1000, 128),   # multi-query, ragged tail
    (3, 2, 2, 100, 64),
    (1, 2, 2, 64, 128),     # exactly one tile
    (1, 2, 2, 128, 64),
    (1, 6, 3, 513, 128),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}".format(*s))
def test_fwd_small_shapes(gpu_lib, shape, causal):
    B, Hq, Hkv, N, d = shape
    say(f"fwd small {shape} causal={causal}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=100 + N + d)
    check_full(gpu_lib, x, causal)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_fwd_tiny_workload(gpu_lib, causal):
    say(f"fwd tiny causal={causal}")
    x = make_inputs("tiny", keep_f32=True)
    eo, el = check_full(gpu_lib, x, causal)
    # logged, not gated: distance to the oracle on the unrounded fp32 draws
    o, lse = run_fwd(gpu_lib, x, causal)
    ro32, _ = attention_forward(torch.from_numpy(x["q_f32"]).double(), torch.from_numpy(x["k_f32"]).double(),
                                torch.from_numpy(x["v_f32"]).double(), causal)
    print(f"tiny causal={causal}: err vs bf16 oracle O={eo:.3g} LSE={el:.3g}; "
          f"vs fp32-draw oracle O={max_abs(dev_f64(o), ro32):.3g}")


def test_fwd_custom_scale(gpu_lib):
    say("fwd custom scale")
    x = make_custom_inputs(1, 4, 2, 300, 128, seed=7)
    check_full(gpu_lib, x, True, scale=0.3)
    check_full(gpu_lib, x, False, scale=0.05)


def test_fwd_large_logits(gpu_lib):
    """Q and K scaled by 8 (exact in binary): scaled scores reach about +-100,
    so exp would overflow without the running max.  V keeps unit scale, so O
    stays in the range the absolute tolerance is meant for."""
    say("fwd large logits")
    x = make_custom_inputs(1, 2, 2, 384, 128, seed=8, in_scale=8.0)
    x["v"] = make_custom_inputs(1, 2, 2, 384, 128, seed=18)["v"]
    # Near one-hot rows put P close to 1, where its bf16 rounding (the MFMA
    # operand) is worth up to 2^-9 * max|V|, and O's own bf16 rounding adds
    # 2^-9 * max|O|: together about 2^-8 * max|V|.  This stress case is not one
    # of the graded workloads, so it is held to that derived bound (plus 50%).
    vmax = float(to_f64(x["v"]).abs().max())
    tol = 1.5 * 2.0 ** -8 * vmax
    for causal in (True, False):
        eo, el = check_full(gpu_lib, x, causal, tol_o=tol)
        print(f"large logits causal={causal}: O err {eo:.3g} (bound {tol:.3g}), LSE err {el:.3g}")


def test_fwd_2k_workload_full(gpu_lib):
    """B=4, H=16, N=2048, d=128 causal: every element against the oracle."""
    say("fwd fwd-2K full")
    x = make_inputs("fwd-2K")
    eo, el = check_full(gpu_lib, x, True)
    print(f"fwd-2K: max err O={eo:.3g} LSE={el:.3g}")


def sampled_rows(N, rng, n=48):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    rand = rng.integers(0, N, size=n).tolist()
    return sorted(set(r for r in fixed + rand if 0 <= r < N))


@pytest.mark.parametrize("name", ["fwd-8K", "gqa-16K", "fb-32K"])
def test_fwd_full_size_sampled(gpu_lib, name):
    w = WORKLOADS[name]
    say(f"fwd {name} sampled rows")
    x = make_inputs(name)
    o, lse = run_fwd(gpu_lib, x, True)
    rng = np.random.default_rng(11)
    heads = sorted(set([0, w.Hq - 1] + rng.integers(0, w.Hq, size=6).tolist()))
    o_h = o.float().cpu()
    l_h = lse.cpu()
    worst_o = worst_l = 0.0
    for h in heads:
        rows = sampled_rows(w.N, rng)
        g = h // w.group
        ro, rl = forward_rows(to_f64(x["q"][:, h:h + 1]), to_f64(x["k"][:, g:g + 1]),
                              to_f64(x["v"][:, g:g + 1]), True, None, 0, 0, rows)
        worst_o = max(worst_o, max_abs(o_h[0, h, rows].double(), ro))
        worst_l = max(worst_l, max_abs(l_h[0, h, rows].double(), rl))
    print(f"{name}: sampled max err O={worst_o:.3g} LSE={worst_l:.3g}")
    assert worst_o <= TOL_O and worst_l <= TOL_LSE
    assert bool(torch.isfinite(o_h).all()) and bool(torch.isfinite(l_h).all())


def test_fwd_deterministic(gpu_lib):
    say("fwd determinism")
    x = make_custom_inputs(2, 8, 4, 1500, 128, seed=9)
    o1, l1 = run_fwd(gpu_lib, x, True)
    o2, l2 = run_fwd(gpu_lib, x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_causal_prefix_on_gpu(gpu_lib):
    """Causal rows < m of a length-N problem equal the length-m problem (bitwise)."""
    say("fwd causal prefix")
    x = make_custom_inputs(1, 4, 4, 3000, 128, seed=10)
    o, lse = run_fwd(gpu_lib, x, True)
    m = 1777
    xm = {n: np.ascontiguousarray(x[n][:, :, :m]) for n in ("q", "k", "v")}
    om, lm = run_fwd(gpu_lib, xm, True)
    assert torch.equal(o[:, :, :m], om) and torch.equal(lse[:, :, :m], lm)


def test_fwd_rejects_bad_input_without_launch(gpu_lib):
    say("fwd argument errors")
    q = torch.zeros(1, 2, 16, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.fwd(q, q, q)
    assert gpu_lib.device_check(torch.cuda.current_device()) == 0
