"""GPU parity of the KV-cache decode forward (split keys, LSE merge) against
the fp64 oracle.

N_q queries at the last N_q positions attend to N_k >= N_q cached keys (the
reading in the oracle).  Bars as for the forward: max |O| error <= 1e-2, max
|LSE| error <= 1e-3.  Cases cover one and several query rows per K/V head
group (G * N_q of 1, 8, 32, 40 rows: one and two 32-row blocks), ragged cache
lengths, one chunk, many chunks, chunks ending mid-way through the causal
diagonal, windows, d = 64 and 128 (each with chunks long enough to cycle the
LDS ring), and N_q = N_k.
"""
import pytest
import torch

from gpu_helpers import TOL_LSE, TOL_O, dev_f64, max_abs, say, to_dev, to_f64
from oracle import attention_forward
from synth_inputs import make_custom_inputs

pytestmark = pytest.mark.gpu


def draw(B, Hq, Hkv, Nq, Nk, d, seed):
    x = make_custom_inputs(B, Hq, Hkv, Nk, d, seed=seed)      # K, V: the cache
    xq = make_custom_inputs(B, Hq, Hkv, Nq, d, seed=seed + 1)  # Q: the new rows
    return xq["q"], x["k"], x["v"]


def check(attn, q, k, v, causal, window=None, splits=0, scale=None, label=""):
    o, lse = attn.fwd_decode(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale,
                             window=window, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = attention_forward(to_f64(q), to_f64(k), to_f64(v), causal, scale, window=window)
    eo, el = max_abs(dev_f64(o), ro), max_abs(dev_f64(lse), rl)
    print(f"{label}: O={eo:.3g} LSE={el:.3g}")
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)
    return o, lse


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, window, splits
    (1, 1, 1, 1, 1, 128, None, 0),
    (1, 8, 8, 1, 300, 128, None, 0),
    (2, 8, 1, 1, 1000, 128, None, 0),       # MQA: 8 rows per block
    (1, 32, 4, 4, 777, 128, None, 3),       # G * Nq = 32 rows
    (1, 16, 2, 5, 2049, 64, None, 0),       # 40 rows: two row blocks
    (1, 8, 2, 3, 4096, 128, None, 1),       # one chunk
    (2, 4, 4, 2, 4096, 128, None, 32),      # one tile per chunk
    (1, 8, 2, 7, 130, 128, None, 2),        # the causal diagonal crosses a chunk edge
    (1, 8, 2, 2, 3000, 128, 500, 0),
    (1, 4, 1, 16, 1200, 64, 100, 4),
    (1, 4, 2, 300, 300, 128, None, 0),      # N_q = N_k
    (1, 8, 2, 1, 5000, 64, None, 1),        # d = 64: one 40-tile chunk through the 4-stage ring
    (1, 8, 8, 3, 6000, 64, 2500, 2),        # d = 64 ring with a long window
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_w{}_s{}".format(*c))
def test_decode_small(gpu_lib, case, causal):
    B, Hq, Hkv, Nq, Nk, d, w, s = case
    say(f"decode {case} causal={causal}")
    q, k, v = draw(B, Hq, Hkv, Nq, Nk, d, seed=500 + Nk + Nq)
    check(gpu_lib, q, k, v, causal, window=w, splits=s, label=str(case))


def test_decode_custom_scale(gpu_lib):
    say("decode custom scale")
    q, k, v = draw(1, 8, 2, 2, 1500, 128, seed=41)
    check(gpu_lib, q, k, v, True, scale=0.3, label="scale 0.3")
    check(gpu_lib, q, k, v, False, scale=0.05, label="scale 0.05")


def test_decode_split_counts_agree_and_are_deterministic(gpu_lib):
    """Every split count meets the oracle; a fixed split count is bitwise
    reproducible."""
    say("decode split counts")
    q, k, v = draw(2, 16, 4, 2, 5000, 128, seed=42)
    outs = {s: check(gpu_lib, q, k, v, True, splits=s, label=f"splits={s}") for s in (1, 2, 7, 0, 64)}
    again = gpu_lib.fwd_decode(to_dev(q), to_dev(k), to_dev(v), causal=True, num_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(again[0], outs[7][0]) and torch.equal(again[1], outs[7][1])


def test_decode_matches_plain_forward_tail(gpu_lib):
    """The decode of the last N_q rows against the whole sequence is the tail of
    the plain causal forward over the whole sequence (within rounding)."""
    say("decode vs plain forward tail")
    x = make_custom_inputs(1, 8, 2, 2000, 128, seed=43)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = gpu_lib.fwd(q, k, v, causal=True)
    od, ld = gpu_lib.fwd_decode(q[:, :, -5:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    assert max_abs(dev_f64(od), dev_f64(o[:, :, -5:])) <= 2 * TOL_O
    assert max_abs(dev_f64(ld), dev_f64(lse[:, :, -5:])) <= 2 * TOL_LSE


def test_decode_benchmark_shape(gpu_lib):
    """The benchmarked decode step (B=16, Hq=32, Hkv=8, one query, 32768 cached
    keys, d=128, causal) in the launch configuration the benchmark times, every
    row checked against the oracle."""
    say("decode benchmark shape")
    q, k, v = draw(16, 32, 8, 1, 32768, 128, seed=44)
    check(gpu_lib, q, k, v, True, label="decode-32K")
