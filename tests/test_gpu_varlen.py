"""GPU parity of packed variable-length batches against the fp64 oracle.

B sequences of different lengths are packed back to back ([H, T, d]), each
its own attention problem.  Bars as for the fixed-length calls: max |O|
error <= 1e-2, max |LSE| error <= 1e-3, max |G - G_ref| / max |G_ref| <= 2e-2
for each gradient.  Cases: empty and one-token sequences, lengths on and off
tile edges, several tiles per sequence, grouped and multi-query heads,
d = 64 and 128, windows, batches of up to 700 sequences on both sides of
the 512-sequence limit of the per-block launch, and the packed benchmark
workload element by element.  The packed calls must also be bitwise equal to calling the
fixed-length entry points on every sequence alone.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (TOL_GRAD_REL, TOL_LSE, TOL_O, assert_same_sum_to_bf16_ulp, bwd_head_split, dev_f64,
                         max_abs, rel_maxnorm, say, to_dev, to_f64, varlen_head_split)
from oracle import attention_backward, attention_forward, varlen_backward, varlen_forward
from synth_inputs import cu_from_lengths, make_custom_inputs, make_inputs

pytestmark = pytest.mark.gpu


def pack_draw(lengths, Hq, Hkv, d, seed, in_scale=1.0):
    x = make_custom_inputs(1, Hq, Hkv, sum(lengths), d, seed=seed, with_grad=True, in_scale=in_scale)
    x = {n: a[0] for n, a in x.items()}
    x["cu_seqlens"] = cu_from_lengths(lengths)
    return x


def run(attn, x, causal, window=None, scale=None):
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(x["cu_seqlens"])
    o, lse = attn.fwd_varlen(q, k, v, cu, causal=causal, window=window, scale=scale)
    dq, dk, dv = attn.bwd_varlen(q, k, v, o, lse, do, cu, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


CASES = [
    # lengths, Hq, Hkv, d, window
    ([1], 1, 1, 128, None),
    ([5, 0, 17, 1, 300], 4, 2, 128, None),      # empty and one-token sequences, ragged tails
    ([256, 257, 255, 1000], 8, 1, 128, None),   # multi-query; lengths at tile edges
    ([700, 33, 1200], 4, 4, 64, None),
    ([130, 513, 64, 2049], 6, 3, 128, None),
    ([900, 400, 1300], 4, 2, 128, 100),         # sliding window within each sequence
    ([3000, 10], 2, 2, 64, 700),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_Hq{}_Hkv{}_d{}_w{}".format(
    "-".join(map(str, c[0])), *c[1:]))
def test_varlen_small(gpu_lib, case, causal):
    lengths, Hq, Hkv, d, window = case
    say(f"varlen {lengths} Hq={Hq} Hkv={Hkv} d={d} w={window} causal={causal}")
    x = pack_draw(lengths, Hq, Hkv, d, seed=sum(lengths) + Hq)
    o, lse, dq, dk, dv = run(gpu_lib, x, causal, window)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    cu = x["cu_seqlens"].tolist()
    ro, rl = varlen_forward(f["q"], f["k"], f["v"], cu, causal, window=window)
    rdq, rdk, rdv = varlen_backward(f["q"], f["k"], f["v"], f["do"], cu, causal, window=window)
    floor = 1e-3 * max(float(t.abs().max()) for t in (rdq, rdk, rdv))
    errs = {"O": max_abs(dev_f64(o), ro), "LSE": max_abs(dev_f64(lse), rl),
            "dQ": rel_maxnorm(dev_f64(dq), rdq, floor), "dK": rel_maxnorm(dev_f64(dk), rdk, floor),
            "dV": rel_maxnorm(dev_f64(dv), rdv, floor)}
    print(" ".join(f"{k}={v:.3g}" for k, v in errs.items()))
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE, errs
    assert max(errs["dQ"], errs["dK"], errs["dV"]) <= TOL_GRAD_REL, errs


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_varlen_equals_per_sequence_calls(gpu_lib, causal):
    """Packing changes nothing: every sequence's rows of O, LSE, dQ, dK, dV are
    bitwise those of the fixed-length calls on that sequence alone -- except
    that where either backward shares each K/V head's query heads out over
    several workgroups (each picks its own split count), dK and dV agree to
    one bf16 unit in the last place (fp32 sums in another order)."""
    lengths = [300, 1, 777, 1024, 0, 129]
    say(f"varlen vs per-sequence calls causal={causal}")
    x = pack_draw(lengths, 8, 2, 128, seed=31)
    o, lse, dq, dk, dv = run(gpu_lib, x, causal)
    cu = x["cu_seqlens"].tolist()
    packed_split = varlen_head_split(gpu_lib, len(lengths), sum(lengths), max(lengths), 8, 2, 128)
    for s0, s1 in zip(cu, cu[1:]):
        if s1 == s0:
            continue
        q, k, v, do = (to_dev(np.ascontiguousarray(x[n][None, :, s0:s1])) for n in ("q", "k", "v", "do"))
        so, sl = gpu_lib.fwd(q, k, v, causal=causal)
        sdq, sdk, sdv = gpu_lib.bwd(q, k, v, so, sl, do, causal=causal)
        torch.cuda.synchronize()
        for packed, alone in ((o, so), (lse, sl), (dq, sdq)):
            assert torch.equal(packed[:, s0:s1], alone[0]), (s0, s1)
        split = packed_split or bwd_head_split(gpu_lib, 1, 8, 2, s1 - s0, 128)
        for packed, alone in ((dk, sdk), (dv, sdv)):
            if split:
                assert_same_sum_to_bf16_ulp(alone[0], packed[:, s0:s1])
            else:
                assert torch.equal(packed[:, s0:s1], alone[0]), (s0, s1)


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


# (number of sequences, longest, Hq, Hkv, d): batches of at most 512 sequences
# are launched over their real blocks only (each workgroup finds its sequence,
# head and block from the table, heaviest first); larger ones over the plain
# (sequence, head, block) grid.  Outputs start as NaN, so a block that no
# workgroup computes shows as non-finite rows.  The draws are at half scale:
# rows of sequences this short average only a few values of V, so |O| comes
# close to max |V| (about 5 at unit scale), where half a bf16 ulp of the
# output alone reaches 0.0156; at half scale it stays under the 1e-2 bar.
MANY = [
    (40, 1500, 4, 1, 128),     # few long, heterogeneous sequences: heaviest-first order across them
    (300, 60, 4, 2, 64),       # many short ones, some empty
    (512, 40, 2, 2, 64),       # the largest batch taken by block
    (700, 40, 2, 1, 64),       # past it: the plain grid
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", MANY, ids=lambda c: "B{}_max{}_Hq{}_Hkv{}_d{}".format(*c))
def test_varlen_many_sequences(gpu_lib, case, causal):
    nseq, longest, Hq, Hkv, d = case
    rng = np.random.default_rng(nseq + longest)
    lengths = [int(round(np.exp(rng.uniform(0.0, np.log(longest))))) for _ in range(nseq)]
    for i in range(3, nseq, 11):
        lengths[i] = 0
    T = sum(lengths)
    say(f"varlen many: B={nseq} T={T} longest={max(lengths)} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    x = pack_draw(lengths, Hq, Hkv, d, seed=nseq + 7, in_scale=0.5)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    o, lse = _nan_like((Hq, T, d), torch.bfloat16), _nan_like((Hq, T), torch.float32)
    gpu_lib.fwd_varlen(q, k, v, cu, max(lengths), causal=causal, out=o, lse=lse)
    dq = _nan_like((Hq, T, d), torch.bfloat16)
    dk, dv = _nan_like((Hkv, T, d), torch.bfloat16), _nan_like((Hkv, T, d), torch.bfloat16)
    gpu_lib.bwd_varlen(q, k, v, o, lse, do, cu, max(lengths), causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    cul = x["cu_seqlens"].tolist()
    ro, rl = varlen_forward(f["q"], f["k"], f["v"], cul, causal)
    rdq, rdk, rdv = varlen_backward(f["q"], f["k"], f["v"], f["do"], cul, causal)
    floor = 1e-3 * max(float(t.abs().max()) for t in (rdq, rdk, rdv))
    errs = {"O": max_abs(dev_f64(o), ro), "LSE": max_abs(dev_f64(lse), rl),
            "dQ": rel_maxnorm(dev_f64(dq), rdq, floor), "dK": rel_maxnorm(dev_f64(dk), rdk, floor),
            "dV": rel_maxnorm(dev_f64(dv), rdv, floor)}
    print(" ".join(f"{kk}={vv:.3g}" for kk, vv in errs.items()))
    assert errs["O"] <= TOL_O and errs["LSE"] <= TOL_LSE, errs
    assert max(errs["dQ"], errs["dK"], errs["dV"]) <= TOL_GRAD_REL, errs


def test_varlen_device_table_and_stages(gpu_lib):
    """A device-resident table with max_seqlen given is used unread by the
    host; the split pre-pass + gradient stage equals bwd_varlen (bitwise with
    the smallest workspace; with the default one bwd_varlen splits this
    batch's query heads, and dK, dV then agree to one bf16 ulp)."""
    lengths = [400, 1500, 3]
    say("varlen device table, stages")
    x = pack_draw(lengths, 4, 2, 128, seed=41)
    assert varlen_head_split(gpu_lib, 3, sum(lengths), 1500, 4, 2, 128)
    o, lse, dq, dk, dv = run(gpu_lib, x, True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    cu_dev = torch.from_numpy(x["cu_seqlens"]).cuda()
    o2, lse2 = gpu_lib.fwd_varlen(q, k, v, cu_dev, max_seqlen=1500, causal=True)
    delta = gpu_lib.bwd_preprocess(o2[None], do[None])[0]
    g = gpu_lib.bwd_grads_varlen(q, k, v, do, lse2, delta, cu_dev, max_seqlen=1500, causal=True)
    small = torch.empty(gpu_lib.bwd_varlen_workspace_bytes(4, sum(lengths), 128), dtype=torch.uint8,
                        device="cuda")
    g1 = gpu_lib.bwd_varlen(q, k, v, o2, lse2, do, cu_dev, max_seqlen=1500, causal=True, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(g1, g):
        assert torch.equal(a, b)
    assert torch.equal(dq, g[0])
    assert_same_sum_to_bf16_ulp(dk, g[1])
    assert_same_sum_to_bf16_ulp(dv, g[2])


# Packed batches whose dK/dV grid is short: few K/V heads over a few thousand
# packed rows.  With the default workspace bwd_varlen splits each K/V head's
# query heads over several workgroups (real-block order; the last case has
# more than 512 sequences and takes the plain grid).
PACKED_SPLIT = [
    # lengths, Hq, Hkv, d
    ([700, 1, 1500, 0, 333], 16, 1, 128),
    ([129, 64, 1000, 7], 12, 2, 64),
    ([3] * 520 + [250], 4, 1, 64),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", PACKED_SPLIT, ids=["mqa16", "gqa12_2_d64", "b521_plain_grid"])
def test_varlen_head_split(gpu_lib, case, causal):
    """Oracle parity with the split; against the smallest workspace (no
    split): dQ bitwise, dK and dV to one bf16 ulp; run to run bitwise."""
    lengths, Hq, Hkv, d = case
    T = sum(lengths)
    say(f"varlen head split B={len(lengths)} T={T} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    assert varlen_head_split(gpu_lib, len(lengths), T, max(lengths), Hq, Hkv, d)
    x = pack_draw(lengths, Hq, Hkv, d, seed=61 + Hq, in_scale=0.5)
    o, lse, dq, dk, dv = run(gpu_lib, x, causal)
    _, _, dq2, dk2, dv2 = run(gpu_lib, x, causal)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(x["cu_seqlens"])
    small = torch.empty(gpu_lib.bwd_varlen_workspace_bytes(Hq, T, d), dtype=torch.uint8, device="cuda")
    g1 = gpu_lib.bwd_varlen(q, k, v, o, lse, do, cu, causal=causal, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.equal(dq, g1[0])
    assert_same_sum_to_bf16_ulp(dk, g1[1])
    assert_same_sum_to_bf16_ulp(dv, g1[2])
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    cul = x["cu_seqlens"].tolist()
    rdq, rdk, rdv = varlen_backward(f["q"], f["k"], f["v"], f["do"], cul, causal)
    floor = 1e-3 * max(float(t.abs().max()) for t in (rdq, rdk, rdv))
    errs = [rel_maxnorm(dev_f64(a), r, floor) for a, r in ((dq, rdq), (dk, rdk), (dv, rdv))]
    print(f"packed split {case[1:]} causal={causal}: dQ/dK/dV = {errs}")
    assert max(errs) <= TOL_GRAD_REL, errs


def test_varlen_empty_batch_and_host_checks(gpu_lib):
    say("varlen empty batch, host checks")
    q = torch.empty((4, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = gpu_lib.fwd_varlen(q, k, k, [0, 0, 0], causal=True)
    assert o.shape == (4, 0, 128) and lse.shape == (4, 0)
    x = pack_draw([10, 20], 2, 2, 64, seed=3)
    qq, kk = to_dev(x["q"]), to_dev(x["k"])
    with pytest.raises(ValueError):
        gpu_lib.fwd_varlen(qq, kk, kk, [0, 10, 31])          # does not end at T
    with pytest.raises(ValueError):
        gpu_lib.fwd_varlen(qq, kk, kk, [0, 10, 30], max_seqlen=15)   # shorter than a sequence


def test_varlen_deterministic(gpu_lib):
    say("varlen determinism")
    x = pack_draw([1000, 37, 2000], 8, 2, 128, seed=51)
    a = run(gpu_lib, x, True)
    b = run(gpu_lib, x, True)
    for t1, t2 in zip(a, b):
        assert torch.equal(t1, t2)


@pytest.mark.timeout(900)
def test_varlen_32k_full(gpu_lib):
    """The packed benchmark workload (32768 tokens in sequences of 512..16384,
    H = 8, d = 128, causal) in the launch configuration the bench times: every
    element of O, LSE, dQ, dK, dV against the oracle, one (sequence, head) at a
    time."""
    say("varlen-32K full")
    x = make_inputs("varlen-32K")
    o, lse, dq, dk, dv = run(gpu_lib, x, True)
    got = {n: dev_f64(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    cu = x["cu_seqlens"].tolist()
    worst = {"O": 0.0, "LSE": 0.0}
    num = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    den = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for s0, s1 in zip(cu, cu[1:]):
        for h in range(8):
            f = {n: to_f64(x[n][None, h:h + 1, s0:s1]) for n in ("q", "k", "v", "do")}
            ro, rl = attention_forward(f["q"], f["k"], f["v"], True)
            rdq, rdk, rdv = attention_backward(f["q"], f["k"], f["v"], f["do"], True)
            worst["O"] = max(worst["O"], max_abs(got["o"][h, s0:s1], ro[0, 0]))
            worst["LSE"] = max(worst["LSE"], max_abs(got["lse"][h, s0:s1], rl[0, 0]))
            for key, g, r in (("dQ", got["dq"][h, s0:s1], rdq), ("dK", got["dk"][h, s0:s1], rdk),
                              ("dV", got["dv"][h, s0:s1], rdv)):
                num[key] = max(num[key], max_abs(g, r[0, 0]))
                den[key] = max(den[key], float(r.abs().max()))
        print(f"  sequence [{s0}, {s1}): O={worst['O']:.3g} LSE={worst['LSE']:.3g} "
              + " ".join(f"{k}={num[k] / den[k]:.3g}" for k in num), flush=True)
    rel = {k: num[k] / den[k] for k in num}
    assert worst["O"] <= TOL_O and worst["LSE"] <= TOL_LSE
    assert max(rel.values()) <= TOL_GRAD_REL, rel
