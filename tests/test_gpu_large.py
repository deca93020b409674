"""GPU parity at the large end: tensors past 4 GiB, a million-token sequence,
and a decode against a 4M-key cache whose last batch starts 4 GiB in.

The inputs come from the integer-only SplitMix64 stream of synth_inputs
(``hashed_bf16_bits``): the GPU tensors are generated on the device, and the
oracle regenerates on the CPU exactly the slices it checks (the same bits).
Bars as everywhere: |O| error <= 1e-2, |LSE| error <= 1e-3, gradients <= 2e-2
relative to the max-norm.  Sizes stay inside the checked limits of the C ABI
(N * d and B * Hq * N below 2^31).
"""
import math

import pytest
import torch

from gpu_helpers import TOL_GRAD_REL, TOL_LSE, TOL_O, dev_f64, max_abs, rel_maxnorm, say
from oracle import attention_backward, attention_forward, forward_rows
from synth_inputs import bf16_bits_to_f64, hashed_bf16_bits

pytestmark = pytest.mark.gpu


def dev_tensor(shape, seed):
    n = math.prod(shape)
    return hashed_bf16_bits(0, n, seed, device="cuda").view(torch.bfloat16).view(shape)


def cpu_rows(shape, seed, b, h, r0, r1):
    """Rows r0 .. r1-1 of head (b, h) of a [B, H, N, d] stream tensor, float64 [r1-r0, d]."""
    _, H, N, d = shape
    start = ((b * H + h) * N + r0) * d
    bits = hashed_bf16_bits(start, (r1 - r0) * d, seed).view(torch.uint16).numpy()
    return torch.from_numpy(bf16_bits_to_f64(bits)).view(r1 - r0, d)


@pytest.mark.timeout(900)
def test_tensors_past_4gib_fwd_bwd(gpu_lib):
    """B=8192, H=1, N=2048, d=128, causal: Q, K, V, O, dO, dQ, dK, dV are 4 GiB
    each, so the last batches sit past 2^32 bytes.  Three whole batches
    (first, middle, last) against the oracle."""
    B, N, d = 8192, 2048, 128
    shape = (B, 1, N, d)
    say("large: tensors past 4 GiB, fwd + bwd")
    q, k, v, do = (dev_tensor(shape, s) for s in (101, 102, 103, 104))
    o, lse = gpu_lib.fwd(q, k, v, causal=True)
    dq, dk, dv = gpu_lib.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for b in (0, 4321, B - 1):
        say(f"  oracle for batch {b}")
        f = [cpu_rows(shape, s, b, 0, 0, N)[None, None] for s in (101, 102, 103, 104)]
        ro, rl = attention_forward(f[0], f[1], f[2], True)
        g = attention_backward(f[0], f[1], f[2], f[3], True)
        eo, el = max_abs(dev_f64(o[b:b + 1]), ro), max_abs(dev_f64(lse[b:b + 1]), rl)
        eg = [rel_maxnorm(dev_f64(t[b:b + 1]), r) for t, r in zip((dq, dk, dv), g)]
        print(f"batch {b}: O={eo:.3g} LSE={el:.3g} dQ/dK/dV={eg}")
        assert eo <= TOL_O and el <= TOL_LSE and max(eg) <= TOL_GRAD_REL


@pytest.mark.timeout(900)
def test_million_token_sequence(gpu_lib):
    """B=1, Hq=2, Hkv=1, N=2^20, d=128, causal forward; sampled rows of both
    query heads (the first, the middle and the last) against the oracle."""
    N, d = 1 << 20, 128
    say("large: one sequence of 2^20 tokens")
    q = dev_tensor((1, 2, N, d), 111)
    k = dev_tensor((1, 1, N, d), 112)
    v = dev_tensor((1, 1, N, d), 113)
    o, lse = gpu_lib.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    say("  GPU done; regenerating K and V on the CPU")
    kc = cpu_rows((1, 1, N, d), 112, 0, 0, 0, N)[None, None]
    vc = cpu_rows((1, 1, N, d), 113, 0, 0, 0, N)[None, None]
    say("  oracle")
    rows = [0, 1, 255, 256, (N >> 1) + 3, N - 257, N - 2, N - 1]
    for h in range(2):
        qc = torch.zeros(1, 2, N, d, dtype=torch.float64)
        for r in rows:
            qc[0, h, r] = cpu_rows((1, 2, N, d), 111, 0, h, r, r + 1)[0]
        ro, rl = forward_rows(qc, kc, vc, True, None, 0, h, rows)
        eo = max_abs(dev_f64(o[0, h, rows]), ro)
        el = max_abs(dev_f64(lse[0, h, rows]), rl)
        print(f"head {h}: O={eo:.3g} LSE={el:.3g}")
        assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.timeout(900)
def test_decode_against_4m_key_cache(gpu_lib):
    """B=5, Hq=8, Hkv=1, one query, N_k=2^22, d=128: the cache is 5 GiB per
    tensor and the last batch starts 4 GiB in.  Every query head of the last
    batch against the oracle."""
    B, Hq, Nk, d = 5, 8, 1 << 22, 128
    say("large: decode against 2^22 cached keys")
    q = dev_tensor((B, Hq, 1, d), 121)
    k = dev_tensor((B, 1, Nk, d), 122)
    v = dev_tensor((B, 1, Nk, d), 123)
    o, lse = gpu_lib.fwd_decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    b = B - 1
    say("  GPU done; regenerating the last batch's K on the CPU")
    kc = cpu_rows((B, 1, Nk, d), 122, b, 0, 0, Nk)[None, None]
    say("  ... and V")
    vc = cpu_rows((B, 1, Nk, d), 123, b, 0, 0, Nk)[None, None]
    say("  oracle")
    qc = torch.stack([cpu_rows((B, Hq, 1, d), 121, b, h, 0, 1) for h in range(Hq)])[None]
    ro, rl = attention_forward(qc, kc, vc, True)
    eo, el = max_abs(dev_f64(o[b:b + 1]), ro), max_abs(dev_f64(lse[b:b + 1]), rl)
    print(f"decode 2^22 keys, batch {b}: O={eo:.3g} LSE={el:.3g}")
    assert eo <= TOL_O and el <= TOL_LSE
