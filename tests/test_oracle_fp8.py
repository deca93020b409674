"""Pins of the oracle's 8-bit (OCP E4M3) path and of the generator's encoder (CPU only).

The decoder is held to torch's float8_e4m3fn type (an implementation of the
same published format) on all 256 codes and to landmark values of the format;
the encoder to torch's rounding and to a round trip over every finite code;
fp8 attention to the scalar brute force run on values decoded by torch and
scaled per head by hand; the descale factors to closed-form relations.
Planted mistakes in a copy of the module must fail these pins.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

from oracle import bf_forward, dequantize, e4m3_to_f64, fp8_attention_forward
from synth_inputs import f32_to_e4m3_bits, make_fp8_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CODES = torch.arange(256, dtype=torch.int64)


def torch_decode(codes) -> torch.Tensor:
    c = torch.as_tensor(codes).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64)


def decode_pin(dec) -> bool:
    a, b = dec(CODES), torch_decode(CODES)
    return bool(torch.equal(torch.isnan(a), torch.isnan(b))) and bool(
        torch.equal(torch.nan_to_num(a), torch.nan_to_num(b)))


def test_decode_all_codes_matches_torch():
    assert decode_pin(e4m3_to_f64)


def test_decode_landmarks():
    v = e4m3_to_f64(CODES)
    assert float(v[0x38]) == 1.0 and float(v[0x7E]) == 448.0 and float(v[0xFE]) == -448.0
    assert float(v[0x01]) == 2.0 ** -9 and float(v[0x07]) == 7 * 2.0 ** -9 and float(v[0x08]) == 2.0 ** -6
    assert float(v[0x80]) == 0.0 and math.copysign(1.0, float(v[0x80])) == -1.0
    assert math.isnan(float(v[0x7F])) and math.isnan(float(v[0xFF]))
    pos = v[:0x7F]
    assert bool((pos[1:] > pos[:-1]).all())                       # codes 0..0x7E rise strictly
    assert torch.equal(v[0x80:0xFF], -v[:0x7F])                   # sign bit only flips the sign


def test_encoder_matches_torch_and_round_trips():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(2000) * 1e-3,
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    grid = e4m3_to_f64(CODES[:0x7F]).numpy()
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)        # exact ties (fp32 holds them)
    x = np.concatenate([x, mids, -mids])
    ours = f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()
    finite = [c for c in range(256) if c & 0x7F != 0x7F]
    vals = e4m3_to_f64(torch.tensor(finite)).numpy()
    assert (f32_to_e4m3_bits(vals) == np.array(finite, dtype=np.uint8)).all()
    with pytest.raises(ValueError):
        f32_to_e4m3_bits(np.array([465.0]))


def bf_fp8(x, causal, scale):
    """Brute force over values decoded by torch and scaled per head by hand."""
    vals = {}
    for n in ("q", "k", "v"):
        dec = torch_decode(torch.from_numpy(x[n + "8"]))
        s = x[n + "_descale"]
        for b in range(dec.shape[0]):
            for h in range(dec.shape[1]):
                dec[b, h] *= float(s[b, h])
        vals[n] = dec
    return bf_forward(vals["q"], vals["k"], vals["v"], causal, scale)


def fp8_pin(fwd) -> bool:
    x = make_fp8_inputs(2, 4, 2, 9, 8, seed=5)
    for causal in (True, False):
        o, lse = fwd(x["q8"], x["k8"], x["v8"], x["q_descale"], x["k_descale"], x["v_descale"], causal, 0.3)
        bo, bl = bf_fp8(x, causal, 0.3)
        if not (torch.allclose(o, torch.tensor(bo, dtype=torch.float64), atol=1e-10, rtol=1e-12)
                and torch.allclose(lse, torch.tensor(bl, dtype=torch.float64), atol=1e-10)):
            return False
    return True


def test_fp8_attention_matches_bruteforce_on_torch_decoded_values():
    assert fp8_pin(fp8_attention_forward)


def test_descale_relations():
    """Q or K descale x c = softmax scale x c; V descale x c = O x c, LSE unchanged."""
    x = make_fp8_inputs(1, 2, 1, 12, 8, seed=6)
    args = lambda **kw: [kw.get(n, x[n]) for n in ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")]
    o, lse = fp8_attention_forward(*args(), True, 0.25)
    o2, lse2 = fp8_attention_forward(*args(q_descale=x["q_descale"] * 2), True, 0.25)
    o3, lse3 = fp8_attention_forward(*args(), True, 0.5)
    assert torch.allclose(o2, o3, atol=1e-12) and torch.allclose(lse2, lse3, atol=1e-12)
    o4, lse4 = fp8_attention_forward(*args(k_descale=x["k_descale"] * 2), True, 0.25)
    assert torch.allclose(o4, o3, atol=1e-12) and torch.allclose(lse4, lse3, atol=1e-12)
    o5, lse5 = fp8_attention_forward(*args(v_descale=x["v_descale"] * 3), True, 0.25)
    assert torch.allclose(o5, 3 * o, atol=1e-12) and torch.allclose(lse5, lse, atol=1e-14)


def test_generated_inputs_use_the_range():
    x = make_fp8_inputs(2, 3, 1, 64, 16, seed=9)
    for n in ("q", "k", "v"):
        c = x[n + "8"]
        assert c.dtype == np.uint8 and not ((c & 0x7F) == 0x7F).any()
        v = e4m3_to_f64(torch.from_numpy(c))
        assert torch.allclose(v.abs().amax(dim=(2, 3)), torch.full(v.shape[:2], 448.0, dtype=torch.float64))
        assert x[n + "_descale"].dtype == np.float32 and x[n + "_descale"].shape == c.shape[:2]
    with pytest.raises(ValueError):
        dequantize(x["q8"], x["q_descale"].T)


MUTANTS = {
    "bias_8": ("torch.pow(2.0, e - 7.0)", "torch.pow(2.0, e - 8.0)"),
    "subnormal_exponent": ("(2.0 ** -6) * (m / 8.0)", "(2.0 ** -7) * (m / 8.0)"),
    "mantissa_over_16": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    "sign_ignored": ("sign * torch.pow", "torch.pow"),
    "nan_on_all_ones_exponent": ("(c & 0x7F) == 0x7F", "(c & 0x78) == 0x78"),
    "descale_per_head_swapped": ("x * s[:, :, None, None]", "x * s.flip(1)[:, :, None, None]"),
    "v_dequantized_with_k_descale": ("dequantize(v8, v_descale)", "dequantize(v8, k_descale)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_fp8_mutant(name):
    src = open(os.path.join(ROOT, "oracle", "fp8.py")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"fp8_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    try:
        ok = decode_pin(mod.e4m3_to_f64) and fp8_pin(mod.fp8_attention_forward)
    except Exception:
        ok = False
    assert not ok, f"pins did not catch {name}"
