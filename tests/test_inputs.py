"""The seeded input generator: bf16 rounding and reproducibility."""
import numpy as np
import pytest

from synth_inputs import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                          make_custom_inputs, make_inputs)


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("bits_in, bits_out", [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # halfway, even kept (lower kept bit 0) -> down
    (0x3F818000, 0x3F82),   # halfway, odd -> up to even
    (0x3F808001, 0x3F81),   # just above halfway -> up
    (0x3F807FFF, 0x3F80),   # just below halfway -> down
    (0xBF818000, 0xBF82),   # sign symmetric
    (0x80000000, 0x8000),   # -0 stays -0
    (0x00000001, 0x0000),   # smallest subnormal rounds to +0
    (0x00018000, 0x0002),   # subnormal halfway, odd -> up
    (0x7F7FFFFF, 0x7F80),   # max float rounds up to +inf (RNE carries)
    (0x7F7F7FFF, 0x7F7F),   # largest value that stays finite
])
def test_bf16_rne_bit_patterns(bits_in, bits_out):
    assert int(f32_to_bf16_bits(f32(bits_in))[0]) == bits_out


def test_bf16_round_trip_is_nearest():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    b = f32_to_bf16_bits(x)
    y = bf16_bits_to_f32(b)
    # |x - y| <= half an ulp of bf16 (2^-8 relative to the binade)
    ulp = np.ldexp(np.float32(1), np.frexp(np.abs(x))[1] - 8).astype(np.float32)
    assert np.all(np.abs(x - y) <= ulp / 2)
    # neighbours are never closer
    up = bf16_bits_to_f32((b.astype(np.uint32) + 1).astype(np.uint16))
    assert np.all(np.abs(x - y) <= np.abs(x - up))


def test_reproducible_and_ordered():
    a = make_custom_inputs(1, 2, 1, 64, 8, seed=7, with_grad=True)
    b = make_custom_inputs(1, 2, 1, 64, 8, seed=7, with_grad=True)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n])
    c = make_custom_inputs(1, 2, 1, 64, 8, seed=8)
    assert not np.array_equal(a["q"], c["q"])
    # draw order: Q first, so Q does not depend on whether dO is drawn
    assert np.array_equal(a["q"], c["q"]) is False
    d = make_custom_inputs(1, 2, 1, 64, 8, seed=7, with_grad=False)
    assert np.array_equal(a["q"], d["q"]) and np.array_equal(a["v"], d["v"])


def test_workload_shapes_and_scale():
    w = WORKLOADS["tiny"]
    x = make_inputs(w, keep_f32=True)
    assert x["q"].shape == (1, 2, 256, 64) and x["q"].dtype == np.uint16
    assert np.array_equal(f32_to_bf16_bits(x["q_f32"]), x["q"])
    assert WORKLOADS["gqa-16K"].group == 8
    assert WORKLOADS["fwd-8K"].in_scale == 0.5
    # 0.5 is applied before rounding: the bf16 values are exactly half of unit draws
    half = make_custom_inputs(1, 1, 1, 32, 8, seed=2, in_scale=0.5)
    unit = make_custom_inputs(1, 1, 1, 32, 8, seed=2, in_scale=1.0)
    assert np.array_equal(bf16_bits_to_f32(half["k"]) * 2, bf16_bits_to_f32(unit["k"]))


def test_flop_counts():
    w = WORKLOADS["fwd-8K"]
    assert w.pairs(True) == 32 * 8192 * 8193 // 2
    assert w.fwd_flops(True) == 4 * 128 * w.pairs(True)
    assert abs(w.fwd_flops(True) - 5.498e11) / 5.498e11 < 1e-3
    assert WORKLOADS["fb-32K"].bwd_flops(True) == 10 * 128 * 8 * 32768 * 32769 // 2


def test_pack_lengths_fill_the_pack():
    from synth_inputs import cu_from_lengths, pack_lengths
    for seed in range(5):
        L = pack_lengths(32768, seed, 512, 16384)
        assert sum(L) == 32768 and all(n >= 1 for n in L)
        assert all(512 <= n <= 16384 for n in L[:-1])    # only the last one is cut
        assert L == pack_lengths(32768, seed, 512, 16384)
    assert pack_lengths(0, 1, 1, 4) == []
    cu = cu_from_lengths([3, 0, 5])
    assert cu.dtype == np.int32 and cu.tolist() == [0, 3, 3, 8]


def test_packed_workload_inputs():
    from synth_inputs import make_custom_inputs, make_inputs
    w = WORKLOADS["varlen-32K"]
    L = w.lengths()
    assert sum(L) == w.N and w.B == 1
    assert w.pairs(True) == w.Hq * sum(n * (n + 1) // 2 for n in L)
    x = make_inputs(w)
    assert x["q"].shape == (w.Hq, w.N, w.d) and x["k"].shape == (w.Hkv, w.N, w.d)
    assert x["do"].shape == (w.Hq, w.N, w.d)
    assert x["cu_seqlens"].tolist()[-1] == w.N
    # the packed draw is the [1, H, T, d] draw of the same seed
    from synth_inputs import Workload
    small = Workload("pack-small", 1, 2, 1, 64, 8, (True,), seed=3, with_grad=True, pack=(4, 16))
    p, y = make_inputs(small), make_custom_inputs(1, 2, 1, 64, 8, seed=3, with_grad=True)
    for name in ("q", "k", "v", "do"):
        assert (p[name] == y[name][0]).all()
    assert p["cu_seqlens"].tolist()[-1] == 64 and len(p["cu_seqlens"]) == len(small.lengths()) + 1


def test_hashed_stream_follows_splitmix64():
    """The integer-only large-input stream equals the published SplitMix64 on
    plain Python integers, and its bits decode to the stated values."""
    import torch
    from synth_inputs import hashed_bf16_bits, splitmix64_reference
    assert splitmix64_reference(0, 0) == 0xE220A8397B1DCDAF      # first output, seed 0
    for seed in (0, 12345, 2 ** 63 + 7):
        got = hashed_bf16_bits(1000, 300, seed, chunk=128).view(torch.uint16).to(torch.int64).tolist()
        for k, g in enumerate(got):
            h = splitmix64_reference(seed, 1000 + k) & 0xFFFF
            assert g == ((h >> 15) << 15) | ((124 + ((h >> 7) & 3)) << 7) | (h & 0x7F)
    v = bf16_bits_to_f32(hashed_bf16_bits(0, 4096, 3).view(torch.uint16).numpy())
    a = np.abs(v)
    assert (a >= 0.125).all() and (a < 2.0).all() and (v < 0).any() and (v > 0).any()
    # a slice of the stream is the same stream
    full = hashed_bf16_bits(0, 5000, 9, chunk=777)
    assert torch.equal(full[1234:2345], hashed_bf16_bits(1234, 1111, 9))
