"""attn_fwd_decode_static (the decode call that allocates nothing) against
attn_fwd_decode with a caller workspace, through the C ABI.

The two share their kernels and chunking, so for the same arguments the
outputs must be bitwise equal; both are also held to the oracle's bar.  Two
calls in a row, the second on a smaller problem, check that the static
scratch's earlier contents never leak into a result.
"""
import ctypes

import pytest
import torch

from gpu_helpers import TOL_LSE, TOL_O, dev_f64, max_abs, say, to_dev, to_f64
from oracle import attention_forward
from synth_inputs import make_custom_inputs

pytestmark = pytest.mark.gpu


def draw(B, Hq, Hkv, Nq, Nk, d, seed):
    xk = make_custom_inputs(B, Hq, Hkv, Nk, d, seed=seed)
    xq = make_custom_inputs(B, Hq, Hkv, Nq, d, seed=seed + 1)
    return xq["q"], xk["k"], xk["v"]


def static_call(L, q, k, v, o, lse, causal, window, scale, splits):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    return L.attn_fwd_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, int(causal),
                                    -1 if window is None else window, ctypes.c_float(scale),
                                    splits, stream)


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, window, splits -- the second is smaller
    (2, 16, 4, 3, 5000, 128, True, None, 0),
    (1, 4, 2, 2, 700, 64, True, 200, 3),
]


def test_static_decode_equals_workspace_decode(gpu_lib):
    L = gpu_lib.lib()
    for i, (B, Hq, Hkv, Nq, Nk, d, causal, window, splits) in enumerate(CASES):
        say(f"decode static call {i}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
            f"window={window} splits={splits}")
        qb, kb, vb = draw(B, Hq, Hkv, Nq, Nk, d, seed=1200 + i)
        q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
        scale = 1.0 / d ** 0.5
        o_ref, lse_ref = gpu_lib.fwd_decode(q, k, v, causal=causal, window=window,
                                            num_splits=splits, scale=scale)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device="cuda")
        rc = static_call(L, q, k, v, o, lse, causal, window, scale, splits)
        assert rc == 0, gpu_lib.strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        ro, rl = attention_forward(to_f64(qb), to_f64(kb), to_f64(vb), causal, scale, window=window)
        assert max_abs(dev_f64(o), ro) <= TOL_O and max_abs(dev_f64(lse), rl) <= TOL_LSE


def test_static_decode_binding_and_limit(gpu_lib):
    """The Python wrapper reaches the same entry point; a problem beyond the
    static scratch is refused with ATTN_ERR_SCRATCH and nothing is launched."""
    say("decode static binding and limit")
    qb, kb, vb = draw(1, 8, 2, 1, 1000, 128, seed=1300)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o, lse = gpu_lib.fwd_decode_static(q, k, v)
    o_ref, lse_ref = gpu_lib.fwd_decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    # a shape whose partials need more than the scratch: checked before any launch
    need = gpu_lib.decode_workspace_bytes(64, 64, 64, 16, 4096, 128, 32)
    assert need > gpu_lib.DECODE_STATIC_SCRATCH_BYTES
    L = gpu_lib.lib()
    rc = L.attn_fwd_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), 64, 64, 64, 16, 4096, 128, 1, -1,
                                  ctypes.c_float(0.1), 32, None)
    assert rc == 7
