"""The Python binding refuses outputs and workspaces the kernels could not
safely write -- host tensors, wrong shapes or dtypes, non-contiguous views --
before anything reaches the library.

Runs without a GPU: the tensors pose as device tensors (a subclass whose
``is_cuda`` is True) and the library handle is replaced by one that fails the
test if any compute entry point is called, so a missing check shows up as a
call instead of a ValueError.
"""
import pytest
import torch

import io_aware_exact_fwd_amd as attn


class _PoseAsDevice(torch.Tensor):
    """A host tensor that reports itself as a device tensor."""

    @property
    def is_cuda(self):
        return True


class _NoCompute:
    """Stands in for the loaded library: size queries answer, compute calls fail."""

    def __getattr__(self, name):
        if name.endswith("_workspace_bytes"):
            return lambda *a: 1 << 20
        def call(*a):
            raise AssertionError(f"{name} was called with arguments the binding should have refused")
        return call


@pytest.fixture
def no_compute(monkeypatch):
    monkeypatch.setattr(attn, "lib", lambda: _NoCompute())
    monkeypatch.setattr(attn, "_stream", lambda s: 0)


def dev(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype).as_subclass(_PoseAsDevice)


def host(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


B, HQ, HKV, N, D = 1, 4, 2, 32, 64


def dense_inputs():
    q, o, do = dev(B, HQ, N, D), dev(B, HQ, N, D), dev(B, HQ, N, D)
    k, v = dev(B, HKV, N, D), dev(B, HKV, N, D)
    lse = dev(B, HQ, N, dtype=torch.float32)
    return q, k, v, o, lse, do


BAD_GRADS = [
    ("dq", lambda: host(B, HQ, N, D)),                            # host memory
    ("dq", lambda: dev(B, HQ, N - 1, D)),                         # too short
    ("dk", lambda: dev(B, HQ, N, D)),                             # query heads instead of K/V heads
    ("dv", lambda: dev(B, HKV, N, D, dtype=torch.float32)),       # wrong dtype
    ("dk", lambda: dev(B, HKV, D, N).transpose(2, 3)),            # not contiguous
]


@pytest.mark.parametrize("name,make", BAD_GRADS)
def test_bwd_refuses_bad_gradient_buffers(no_compute, name, make):
    q, k, v, o, lse, do = dense_inputs()
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, do, **{name: make()})


@pytest.mark.parametrize("name,make", BAD_GRADS)
def test_bwd_grads_refuses_bad_gradient_buffers(no_compute, name, make):
    q, k, v, o, lse, do = dense_inputs()
    delta = dev(B, HQ, N, dtype=torch.float32)
    with pytest.raises(ValueError):
        attn.bwd_grads(q, k, v, do, lse, delta, **{name: make()})


@pytest.mark.parametrize("ws", [lambda: host(1 << 20, dtype=torch.uint8),
                                lambda: dev(64, 1 << 15, dtype=torch.uint8)[:, ::2]])
def test_bwd_refuses_bad_workspace(no_compute, ws):
    q, k, v, o, lse, do = dense_inputs()
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, do, workspace=ws())


def test_decode_refuses_host_workspace(no_compute):
    q = dev(B, HQ, 1, D)
    k, v = dev(B, HKV, N, D), dev(B, HKV, N, D)
    with pytest.raises(ValueError):
        attn.fwd_decode(q, k, v, workspace=host(1 << 20, dtype=torch.uint8))


@pytest.mark.parametrize("which", ["out", "lse"])
def test_fwd_refuses_host_outputs(no_compute, which):
    q, k, v, o, lse, do = dense_inputs()
    bad = {"out": host(B, HQ, N, D), "lse": host(B, HQ, N, dtype=torch.float32)}[which]
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, **{which: bad})


def test_bwd_refuses_host_lse(no_compute):
    q, k, v, o, lse, do = dense_inputs()
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, host(B, HQ, N, dtype=torch.float32), do)


T = 40
PACKED_BAD = [
    ("dq", lambda: host(HQ, T, D)),
    ("dk", lambda: dev(HKV, T + 1, D)),
    ("dv", lambda: dev(HQ, T, D)),
]


@pytest.mark.parametrize("name,make", PACKED_BAD)
def test_packed_backward_refuses_bad_gradient_buffers(no_compute, name, make):
    q, o, do = dev(HQ, T, D), dev(HQ, T, D), dev(HQ, T, D)
    k, v = dev(HKV, T, D), dev(HKV, T, D)
    lse, delta = dev(HQ, T, dtype=torch.float32), dev(HQ, T, dtype=torch.float32)
    cu = [0, 15, 40]
    with pytest.raises(ValueError):
        attn.bwd_varlen(q, k, v, o, lse, do, cu, 25, **{name: make()})
    with pytest.raises(ValueError):
        attn.bwd_grads_varlen(q, k, v, do, lse, delta, cu, 25, **{name: make()})


def test_packed_backward_refuses_host_workspace(no_compute):
    q, o, do = dev(HQ, T, D), dev(HQ, T, D), dev(HQ, T, D)
    k, v = dev(HKV, T, D), dev(HKV, T, D)
    lse = dev(HQ, T, dtype=torch.float32)
    with pytest.raises(ValueError):
        attn.bwd_varlen(q, k, v, o, lse, do, [0, 15, 40], 25,
                        workspace=host(1 << 20, dtype=torch.uint8))
