"""Planted mistakes in a copy of the oracle must be caught by its pins.

Each mutant is the oracle's source with one plausible slip (a dropped term, a
wrong sign, an off-by-one mask, a wrong head map, a missing scale, a swapped
operand).  It is loaded as a separate module on the CPU; the real oracle is
untouched.  The test passes when the pins used in ``test_oracle.py`` (brute
force, the hand-worked examples) reject every mutant.
"""
import json
import os
import types

import numpy as np
import pytest
import torch

from oracle import bf_backward, bf_forward

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "attention.py")).read()
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "hand_worked.json")))["cases"]

MUTANTS = {
    "dropped_scale": ("s = scale * (q_rows @ k_head.transpose(0, 1))", "s = (q_rows @ k_head.transpose(0, 1))"),
    "mask_hides_diagonal": ("keys[None, :] > rows[:, None]", "keys[None, :] >= rows[:, None]"),
    "mask_shows_next_key": ("keys[None, :] > rows[:, None]", "keys[None, :] > rows[:, None] + 1"),
    "lse_drops_max": ("lse = m + torch.log(ell)", "lse = torch.log(ell)"),
    "gqa_modulo_heads": ("            g = h // G\n            for r0 in range(0, N, row_block):\n                r1 = min(N, r0 + row_block)\n                rows = torch.arange(r0, r1, dtype=torch.int64) + (k.shape[2] - N)   # positions\n                p, l_blk",
                         "            g = h % Hkv\n            for r0 in range(0, N, row_block):\n                r1 = min(N, r0 + row_block)\n                rows = torch.arange(r0, r1, dtype=torch.int64) + (k.shape[2] - N)   # positions\n                p, l_blk"),
    "decode_top_left_alignment": ("rows = torch.arange(r0, r1, dtype=torch.int64) + (k.shape[2] - N)   # positions\n                p, l_blk",
                                  "rows = torch.arange(r0, r1, dtype=torch.int64)\n                p, l_blk"),
    "jacobian_sign": ("ds = p * (dp - c[:, None])                     # dS_ij", "ds = p * (dp + c[:, None])                     # dS_ij"),
    "jacobian_drops_c": ("ds = p * (dp - c[:, None])                     # dS_ij", "ds = p * dp                     # dS_ij"),
    "dk_no_scale": ("dk[b, g] += tau * (ds.transpose(0, 1) @ q_blk)", "dk[b, g] += (ds.transpose(0, 1) @ q_blk)"),
    "dq_no_scale": ("dq[b, h, r0:r1] = tau * (ds @ k[b, g])", "dq[b, h, r0:r1] = (ds @ k[b, g])"),
    "dv_uses_ds": ("dv[b, g] += p.transpose(0, 1) @ do_blk", "dv[b, g] += ds.transpose(0, 1) @ do_blk"),
    "dp_uses_k": ("dp = do_blk @ v[b, g].transpose(0, 1)          # dP_ij", "dp = do_blk @ k[b, g].transpose(0, 1)          # dP_ij"),
    "dk_overwrites_group": ("dk[b, g] += tau", "dk[b, g] = tau"),
    "o_uses_k": ("o[b, h, r0:r1] = p @ v[b, g]", "o[b, h, r0:r1] = p @ k[b, g]"),
    "window_off_by_one_left": ("(dist < -int(window))", "(dist <= -int(window))"),
    "window_off_by_one_right": ("(dist > int(window))", "(dist >= int(window))"),
    "window_left_side_only": ("(dist < -int(window)) | (dist > int(window))", "(dist < -int(window))"),
    "window_ignored": ("if window is not None:\n        dist", "if False:\n        dist"),
    "varlen_keys_leak_from_earlier_sequences": (
        "ob, lb = attention_forward(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1],",
        "ob, lb = attention_forward(q[None, :, s0:s1], k[None, :, :s1], v[None, :, :s1],"),
    "varlen_skips_first_sequence": ("for s0, s1 in zip(cu, cu[1:]):", "for s0, s1 in zip(cu[1:], cu[2:]):"),
    "varlen_dk_dv_swapped": ("g[0][0], g[1][0], g[2][0]", "g[0][0], g[2][0], g[1][0]"),
    "probs_rows_top_left_alignment": (
        "p, _ = _row_probs(to_f64(q[b, h])[rows_t], to_f64(k[b, g]), rows_t + (k.shape[2] - q.shape[2]),",
        "p, _ = _row_probs(to_f64(q[b, h])[rows_t], to_f64(k[b, g]), rows_t,"),
    "probs_rows_modulo_heads": (
        "    g = h // (Hq // Hkv)\n    d = q.shape[-1]\n    tau = default_scale(d) if scale is None else float(scale)\n"
        "    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)\n    p, _ = _row_probs(",
        "    g = h % Hkv\n    d = q.shape[-1]\n    tau = default_scale(d) if scale is None else float(scale)\n"
        "    rows_t = torch.as_tensor(list(rows), dtype=torch.int64)\n    p, _ = _row_probs("),
    "attention_probs_top_left_alignment": (
        "rows = torch.arange(N, dtype=torch.int64) + (k.shape[2] - N)               # positions",
        "rows = torch.arange(N, dtype=torch.int64)"),
    "attention_probs_drops_scale": (
        "out[b, h], _ = _row_probs(q[b, h], k[b, h // G], rows, causal, tau, window)",
        "out[b, h], _ = _row_probs(q[b, h], k[b, h // G], rows, causal, 1.0, window)"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = SRC.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def rnd(seed, *shape):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape))


def pins_pass(mod) -> bool:
    """The brute-force and hand-worked pins, run against a candidate oracle."""
    try:
        for case in GOLDEN:
            q, k, v, do = (torch.tensor(case[n], dtype=torch.float64) for n in ("q", "k", "v", "do"))
            o, lse = mod.attention_forward(q, k, v, case["causal"], case["scale"])
            grads = mod.attention_backward(q, k, v, do, case["causal"], case["scale"])
            for got, n in zip((o, lse) + tuple(grads), ("o", "lse", "dq", "dk", "dv")):
                if not torch.allclose(got, torch.tensor(case[n], dtype=torch.float64), atol=1e-12):
                    return False
        B, Hq, Hkv, N, d = 1, 4, 2, 9, 4
        q, k, v, do = rnd(1, B, Hq, N, d), rnd(2, B, Hkv, N, d), rnd(3, B, Hkv, N, d), rnd(4, B, Hq, N, d)
        for causal in (True, False):
            o, lse = mod.attention_forward(q, k, v, causal, 0.37, row_block=4)
            bo, bl = bf_forward(q, k, v, causal, 0.37)
            if not (torch.allclose(o, torch.tensor(bo, dtype=torch.float64), atol=1e-11) and torch.allclose(lse, torch.tensor(bl, dtype=torch.float64), atol=1e-11)):
                return False
            g = mod.attention_backward(q, k, v, do, causal, 0.37, row_block=4)
            bg = bf_backward(q, k, v, do, causal, 0.37)
            for x, y in zip(g, bg):
                if not torch.allclose(x, torch.tensor(y, dtype=torch.float64), atol=1e-10):
                    return False
            qd = q[:, :, -3:]                       # decode: the last 3 queries against 9 keys
            o, lse = mod.attention_forward(qd, k, v, causal, 0.37, row_block=2)
            bo, bl = bf_forward(qd, k, v, causal, 0.37)
            if not (torch.allclose(o, torch.tensor(bo, dtype=torch.float64), atol=1e-11)
                    and torch.allclose(lse, torch.tensor(bl, dtype=torch.float64), atol=1e-11)):
                return False
            for w in (0, 2):
                o, lse = mod.attention_forward(q, k, v, causal, 0.37, row_block=4, window=w)
                bo, bl = bf_forward(q, k, v, causal, 0.37, window=w)
                if not (torch.allclose(o, torch.tensor(bo, dtype=torch.float64), atol=1e-11)
                        and torch.allclose(lse, torch.tensor(bl, dtype=torch.float64), atol=1e-11)):
                    return False
            # packed batch of sequences 3, 0, 4, 2 against the same-sequence-masked brute force
            pq, pk, pv, pdo = q[0, :, :9], k[0, :, :9], v[0, :, :9], do[0, :, :9]
            cu, seg = [0, 3, 3, 7, 9], [0, 0, 0, 2, 2, 2, 2, 3, 3]
            o, lse = mod.varlen_forward(pq, pk, pv, cu, causal, 0.37)
            bo, bl = bf_forward(pq[None], pk[None], pv[None], causal, 0.37, segments=seg)
            if not (torch.allclose(o, torch.tensor(bo, dtype=torch.float64)[0], atol=1e-11)
                    and torch.allclose(lse, torch.tensor(bl, dtype=torch.float64)[0], atol=1e-11)):
                return False
            g = mod.varlen_backward(pq, pk, pv, pdo, cu, causal, 0.37)
            bg = bf_backward(pq[None], pk[None], pv[None], pdo[None], causal, 0.37, segments=seg)
            for x, y in zip(g, bg):
                if not torch.allclose(x, torch.tensor(y, dtype=torch.float64)[0], atol=1e-10):
                    return False
        # rows of P (attention_probs, probs_rows) against the brute force with V = I
        Nk = 10
        for nq in (10, 4):
            pq, pk = rnd(61, 1, 4, nq, Nk), rnd(62, 1, 2, Nk, Nk)
            eye = torch.eye(Nk, dtype=torch.float64).expand(1, 2, Nk, Nk).contiguous()
            for causal in (True, False):
                bp = torch.tensor(bf_forward(pq, pk, eye, causal, 0.37)[0], dtype=torch.float64)
                if not torch.allclose(mod.attention_probs(pq, pk, causal, 0.37), bp, atol=1e-13):
                    return False
                for h in range(4):
                    rows = [nq - 1, 0, nq // 2]
                    if not torch.allclose(mod.probs_rows(pq, pk, causal, 0.37, 0, h, rows),
                                          bp[0, h, rows], atol=1e-13):
                        return False
    except Exception:
        return False
    return True


def test_unmutated_copy_passes():
    mod = types.ModuleType("oracle_copy")
    exec(compile(SRC, "<oracle copy>", "exec"), mod.__dict__)
    assert pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name):
    assert not pins_pass(load_mutant(name)), f"pins did not catch mutant {name}"
