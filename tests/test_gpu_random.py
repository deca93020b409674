"""Seeded random shapes through every entry point, against the fp64 oracle.

Each case draws B, H_q, H_kv (a divisor), N (ragged, 1..700), d, the causal
flag, an optional window and an optional scale from a fixed seed, then checks
the forward and backward (fixed-length and windowed), the decode forward
(N_q < N_k) and the packed variable-length calls at the usual bars, and the
8-bit forward (d = 128, no window) at its per-element rounding bound.  The
cases are small, so every element is compared.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_GRAD_REL, TOL_LSE, TOL_O, dev_f64, max_abs, rel_maxnorm, say, to_dev, to_f64
from oracle import attention_backward, attention_forward, varlen_backward, varlen_forward
from synth_inputs import cu_from_lengths, make_custom_inputs, make_fp8_inputs
from test_gpu_fp8 import check as check_fp8

pytestmark = pytest.mark.gpu


def draw_case(i):
    r = np.random.default_rng(1000 + i)
    Hkv = int(r.choice([1, 2, 3, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    return dict(B=int(r.integers(1, 3)), Hq=Hq, Hkv=Hkv, N=int(r.integers(1, 701)),
                d=int(r.choice([64, 128])), causal=bool(r.integers(0, 2)),
                window=int(r.integers(0, 300)) if r.random() < 0.35 else None,
                scale=float(r.uniform(0.05, 0.2)) if r.random() < 0.3 else None, seed=2000 + i)


def grads_err(got, ref):
    floor = 1e-3 * max(float(t.abs().max()) for t in ref)
    return max(rel_maxnorm(dev_f64(g), r, floor) for g, r in zip(got, ref))


@pytest.mark.parametrize("i", range(16))
def test_random_fixed_length(gpu_lib, i):
    c = draw_case(i)
    say(f"random fixed-length case {i}: {c}")
    x = make_custom_inputs(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], seed=c["seed"], with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.fwd(q, k, v, causal=c["causal"], scale=c["scale"], window=c["window"])
    g = gpu_lib.bwd(q, k, v, o, lse, do, causal=c["causal"], scale=c["scale"], window=c["window"])
    torch.cuda.synchronize()
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = attention_forward(f["q"], f["k"], f["v"], c["causal"], c["scale"], window=c["window"])
    rg = attention_backward(f["q"], f["k"], f["v"], f["do"], c["causal"], c["scale"], window=c["window"])
    eo, el, eg = max_abs(dev_f64(o), ro), max_abs(dev_f64(lse), rl), grads_err(g, rg)
    print(f"O={eo:.3g} LSE={el:.3g} grads={eg:.3g}")
    assert eo <= TOL_O and el <= TOL_LSE and eg <= TOL_GRAD_REL


@pytest.mark.parametrize("i", range(8))
def test_random_decode(gpu_lib, i):
    c = draw_case(100 + i)
    r = np.random.default_rng(3000 + i)
    nq = int(r.integers(1, min(c["N"], 40) + 1))
    say(f"random decode case {i}: {c} nq={nq}")
    x = make_custom_inputs(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], seed=c["seed"])
    xq = make_custom_inputs(c["B"], c["Hq"], c["Hkv"], nq, c["d"], seed=c["seed"] + 1)
    splits = int(r.integers(0, 6))
    o, lse = gpu_lib.fwd_decode(to_dev(xq["q"]), to_dev(x["k"]), to_dev(x["v"]), causal=c["causal"],
                                scale=c["scale"], window=c["window"], num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = attention_forward(to_f64(xq["q"]), to_f64(x["k"]), to_f64(x["v"]), c["causal"], c["scale"],
                               window=c["window"])
    eo, el = max_abs(dev_f64(o), ro), max_abs(dev_f64(lse), rl)
    print(f"O={eo:.3g} LSE={el:.3g}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("i", range(8))
def test_random_packed(gpu_lib, i):
    c = draw_case(200 + i)
    r = np.random.default_rng(4000 + i)
    lengths = [int(n) for n in r.integers(0, 500, size=int(r.integers(1, 6)))]
    if sum(lengths) == 0:
        lengths[0] = 1
    say(f"random packed case {i}: {c} lengths={lengths}")
    T = sum(lengths)
    x = make_custom_inputs(1, c["Hq"], c["Hkv"], T, c["d"], seed=c["seed"], with_grad=True)
    x = {n: a[0] for n, a in x.items()}
    cu = cu_from_lengths(lengths)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.fwd_varlen(q, k, v, torch.from_numpy(cu), causal=c["causal"], scale=c["scale"],
                                window=c["window"])
    g = gpu_lib.bwd_varlen(q, k, v, o, lse, do, torch.from_numpy(cu), causal=c["causal"],
                           scale=c["scale"], window=c["window"])
    torch.cuda.synchronize()
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = varlen_forward(f["q"], f["k"], f["v"], cu.tolist(), c["causal"], c["scale"], window=c["window"])
    rg = varlen_backward(f["q"], f["k"], f["v"], f["do"], cu.tolist(), c["causal"], c["scale"],
                         window=c["window"])
    eo, el, eg = max_abs(dev_f64(o), ro), max_abs(dev_f64(lse), rl), grads_err(g, rg)
    print(f"O={eo:.3g} LSE={el:.3g} grads={eg:.3g}")
    assert eo <= TOL_O and el <= TOL_LSE and eg <= TOL_GRAD_REL


@pytest.mark.parametrize("i", range(6))
def test_random_fp8(gpu_lib, i):
    c = draw_case(300 + i)
    say(f"random 8-bit case {i}: B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} N={c['N']} causal={c['causal']} "
        f"scale={c['scale']}")
    x = make_fp8_inputs(c["B"], c["Hq"], c["Hkv"], c["N"], 128, seed=c["seed"])
    check_fp8(gpu_lib, x, c["causal"], c["scale"], label=f"random fp8 {i}")
