"""Every entry point writes its outputs and nothing else.

The method keeps only O and the log-sum-exp in device memory (page "6.1 2023
年代：長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.2), and the backward
writes only dQ, dK and dV (plus its caller-owned workspace).  Here every output
buffer, and every workspace, sits inside a larger allocation with guard bytes
on both sides; after each call the guard bytes must be bitwise intact, so a
stray row at a ragged tail, a packed-sequence boundary or a decode chunk edge
shows up even where aggregate write counters cannot see it.  The outputs
themselves are pre-filled with NaN bit patterns and must come back finite:
every element was written.  Results are also checked against the oracle, so a
kernel cannot pass by writing the wrong rows.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_GRAD_REL, TOL_LSE, TOL_O, dev_f64, max_abs, rel_maxnorm, say, to_dev, to_f64
from oracle import (attention_backward, attention_forward, fp8_attention_forward, varlen_backward,
                    varlen_forward)
from synth_inputs import cu_from_lengths, make_custom_inputs, make_fp8_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side (keeps the 16-byte alignment of the allocation)
PATTERN = 0xA5


class Guarded:
    """Tensors carved out of guarded allocations; check() verifies the guards."""

    def __init__(self):
        self.bufs = []

    def tensor(self, shape, dtype, fill_nan=True):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        body = buf[GUARD:GUARD + n]
        if fill_nan:
            body.fill_(0xFF)            # all-ones: NaN in bf16 and fp32
        self.bufs.append(buf)
        return body.view(dtype).view(shape)

    def workspace(self, nbytes):
        return self.tensor((max(int(nbytes), 16),), torch.uint8, fill_nan=False)

    def check(self, label):
        torch.cuda.synchronize()
        for i, buf in enumerate(self.bufs):
            head = buf[:GUARD].cpu().numpy()
            tail = buf[-GUARD:].cpu().numpy()
            bad_h = int((head != PATTERN).sum())
            bad_t = int((tail != PATTERN).sum())
            assert bad_h == 0 and bad_t == 0, f"{label}: buffer {i} guard overwritten ({bad_h} before, {bad_t} after)"


def finite(*ts):
    return all(bool(torch.isfinite(t.float()).all()) for t in ts)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", [(2, 4, 2, 257, 128), (1, 3, 1, 130, 64), (1, 2, 2, 1, 128)],
                         ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}".format(*s))
def test_forward_and_backward_write_only_their_outputs(gpu_lib, shape, causal):
    B, Hq, Hkv, N, d = shape
    say(f"canary fwd+bwd {shape} causal={causal}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=900 + N, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    g = Guarded()
    o = g.tensor((B, Hq, N, d), torch.bfloat16)
    lse = g.tensor((B, Hq, N), torch.float32)
    gpu_lib.fwd(q, k, v, causal=causal, out=o, lse=lse)
    g.check("attn_fwd")
    dq = g.tensor((B, Hq, N, d), torch.bfloat16)
    dk = g.tensor((B, Hkv, N, d), torch.bfloat16)
    dv = g.tensor((B, Hkv, N, d), torch.bfloat16)
    ws = g.workspace(gpu_lib.bwd_workspace_bytes(B, Hq, Hkv, N, d))
    gpu_lib.bwd(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)
    g.check("attn_bwd")
    assert finite(o, lse, dq, dk, dv)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = attention_forward(f["q"], f["k"], f["v"], causal)
    rg = attention_backward(f["q"], f["k"], f["v"], f["do"], causal)
    assert max_abs(dev_f64(o), ro) <= TOL_O and max_abs(dev_f64(lse), rl) <= TOL_LSE
    floor = 1e-3 * max(float(r.abs().max()) for r in rg)
    for got, ref in zip((dq, dk, dv), rg):
        assert rel_maxnorm(dev_f64(got), ref, floor) <= TOL_GRAD_REL


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_stages_and_window_write_only_their_outputs(gpu_lib, causal):
    """The backward's stages (D pre-pass, dK/dV, dQ, the merged gradients) and
    the windowed calls, each with its outputs guarded."""
    B, Hq, Hkv, N, d, w = 1, 4, 2, 333, 128, 45
    say(f"canary stages + window causal={causal}")
    x = make_custom_inputs(B, Hq, Hkv, N, d, seed=931, with_grad=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    g = Guarded()
    o = g.tensor((B, Hq, N, d), torch.bfloat16)
    lse = g.tensor((B, Hq, N), torch.float32)
    gpu_lib.fwd(q, k, v, causal=causal, out=o, lse=lse, window=w)
    delta = g.tensor((B, Hq, N), torch.float32)
    gpu_lib.bwd_preprocess(o, do, delta)
    dk = g.tensor((B, Hkv, N, d), torch.bfloat16)
    dv = g.tensor((B, Hkv, N, d), torch.bfloat16)
    dq = g.tensor((B, Hq, N, d), torch.bfloat16)
    gpu_lib.bwd_grads(q, k, v, do, lse, delta, causal=causal, dq=dq, dk=dk, dv=dv, window=w)
    g.check("windowed fwd, pre-pass, windowed gradients")
    assert finite(o, lse, delta, dq, dk, dv)
    g2 = Guarded()
    o2 = g2.tensor((B, Hq, N, d), torch.bfloat16)
    lse2 = g2.tensor((B, Hq, N), torch.float32)
    gpu_lib.fwd(q, k, v, causal=causal, out=o2, lse=lse2)
    delta2 = g2.tensor((B, Hq, N), torch.float32)
    gpu_lib.bwd_preprocess(o2, do, delta2)
    dk2 = g2.tensor((B, Hkv, N, d), torch.bfloat16)
    dv2 = g2.tensor((B, Hkv, N, d), torch.bfloat16)
    gpu_lib.bwd_dkdv(q, k, v, do, lse2, delta2, causal=causal, dk=dk2, dv=dv2)
    dq2 = g2.tensor((B, Hq, N, d), torch.bfloat16)
    gpu_lib.bwd_dq(q, k, v, do, lse2, delta2, causal=causal, dq=dq2)
    g2.check("pre-pass, dK/dV, dQ")
    assert finite(dq2, dk2, dv2)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    rg = attention_backward(f["q"], f["k"], f["v"], f["do"], causal, window=w)
    floor = 1e-3 * max(float(r.abs().max()) for r in rg)
    for got, ref in zip((dq, dk, dv), rg):
        assert rel_maxnorm(dev_f64(got), ref, floor) <= TOL_GRAD_REL


@pytest.mark.parametrize("splits", [0, 1, 3, 8])
def test_decode_writes_only_its_outputs(gpu_lib, splits):
    """Decode with the cache length off the 128-key tile grid and chunk edges
    inside the causal diagonal; O, LSE and the workspace of partials guarded."""
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 3, 1000, 128
    say(f"canary decode splits={splits}")
    xk = make_custom_inputs(B, Hq, Hkv, Nk, d, seed=941)
    xq = make_custom_inputs(B, Hq, Hkv, Nq, d, seed=942)
    q, k, v = to_dev(xq["q"]), to_dev(xk["k"]), to_dev(xk["v"])
    g = Guarded()
    o = g.tensor((B, Hq, Nq, d), torch.bfloat16)
    lse = g.tensor((B, Hq, Nq), torch.float32)
    ws = g.workspace(gpu_lib.decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, splits))
    gpu_lib.fwd_decode(q, k, v, causal=True, num_splits=splits, out=o, lse=lse, workspace=ws)
    g.check(f"attn_fwd_decode splits={splits}")
    assert finite(o, lse)
    ro, rl = attention_forward(to_f64(xq["q"]), to_f64(xk["k"]), to_f64(xk["v"]), True)
    assert max_abs(dev_f64(o), ro) <= TOL_O and max_abs(dev_f64(lse), rl) <= TOL_LSE


@pytest.mark.parametrize("split", [False, True], ids=["min_workspace", "split_workspace"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_packed_batches_write_only_their_outputs(gpu_lib, causal, split):
    """A packed batch with a one-token sequence, an empty one and ragged tails:
    O, LSE, D, dQ, dK, dV and the workspace guarded; every packed row written.
    With the split-size workspace the backward also writes its partial sums
    there (two K/V heads of two query heads each, split two ways)."""
    lengths, Hq, Hkv, d = [1, 0, 129, 1, 270, 0, 64], 4, 2, 128
    T = sum(lengths)
    say(f"canary packed {lengths} causal={causal}")
    x = make_custom_inputs(1, Hq, Hkv, T, d, seed=951, with_grad=True)
    x = {n: a[0] for n, a in x.items()}
    cu_np = cu_from_lengths(lengths)
    cu = torch.from_numpy(cu_np).cuda()
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    g = Guarded()
    o = g.tensor((Hq, T, d), torch.bfloat16)
    lse = g.tensor((Hq, T), torch.float32)
    gpu_lib.fwd_varlen(q, k, v, cu, max(lengths), causal=causal, out=o, lse=lse)
    dq = g.tensor((Hq, T, d), torch.bfloat16)
    dk = g.tensor((Hkv, T, d), torch.bfloat16)
    dv = g.tensor((Hkv, T, d), torch.bfloat16)
    ws = g.workspace(gpu_lib.bwd_varlen_split_workspace_bytes(len(lengths), T, max(lengths), Hq, Hkv, d)
                     if split else gpu_lib.bwd_varlen_workspace_bytes(Hq, T, d))
    gpu_lib.bwd_varlen(q, k, v, o, lse, do, cu, max(lengths), causal=causal, dq=dq, dk=dk, dv=dv,
                       workspace=ws)
    g.check("packed fwd + bwd")
    assert finite(o, lse, dq, dk, dv)
    f = {n: to_f64(x[n]) for n in ("q", "k", "v", "do")}
    ro, rl = varlen_forward(f["q"], f["k"], f["v"], cu_np.tolist(), causal)
    rg = varlen_backward(f["q"], f["k"], f["v"], f["do"], cu_np.tolist(), causal)
    assert max_abs(dev_f64(o), ro) <= TOL_O and max_abs(dev_f64(lse), rl) <= TOL_LSE
    floor = 1e-3 * max(float(r.abs().max()) for r in rg)
    for got, ref in zip((dq, dk, dv), rg):
        assert rel_maxnorm(dev_f64(got), ref, floor) <= TOL_GRAD_REL


def test_fp8_forward_writes_only_its_outputs(gpu_lib):
    B, Hq, Hkv, N = 1, 4, 2, 257
    say("canary fp8 forward")
    x = make_fp8_inputs(B, Hq, Hkv, N, 128, seed=961)
    g = Guarded()
    o = g.tensor((B, Hq, N, 128), torch.bfloat16)
    lse = g.tensor((B, Hq, N), torch.float32)
    dev = lambda n: torch.from_numpy(x[n]).cuda()
    gpu_lib.fwd_fp8(dev("q8"), dev("k8"), dev("v8"), dev("q_descale"), dev("k_descale"),
                    dev("v_descale"), causal=True, out=o, lse=lse)
    g.check("attn_fwd_fp8")
    assert finite(o, lse)
    _, rl = fp8_attention_forward(x["q8"], x["k8"], x["v8"], x["q_descale"], x["k_descale"],
                                  x["v_descale"], True)
    assert max_abs(dev_f64(lse), rl) <= TOL_LSE
